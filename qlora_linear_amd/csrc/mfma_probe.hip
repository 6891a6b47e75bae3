// MFMA-only probe (gfx950): the bf16 matrix-core throughput this GPU sustains with
// no memory traffic, the practical ceiling next to the published 2.5 PFLOP/s.
// One 512-thread workgroup per CU (its LDS reservation keeps a second one off the
// CU), eight waves = two per SIMD, each issuing v_mfma_f32_32x32x16_bf16 back to
// back into eight independent accumulators on register operands.
#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeBlocks = 256;  // MI355X compute units

__global__ __launch_bounds__(kProbeThreads, 1) void mfma_probe_kernel(int iters, float* __restrict__ sink) {
  __shared__ float reserve[24 * 1024];  // 96 KB: one workgroup per CU
  const int lane = threadIdx.x & 63;
  // small bf16 operands (|value| < 1), distinct per lane
  const uint32_t a0 = 0x3C003C00u + static_cast<uint32_t>(lane), b0 = 0x3B803B80u + static_cast<uint32_t>(lane);
  const uint4 a = {a0, a0 ^ 1u, a0 ^ 2u, a0 ^ 3u}, b = {b0, b0 ^ 1u, b0 ^ 2u, b0 ^ 3u};
  f32x16_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = mfma32(a, b, acc[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[i][e];
  reserve[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = reserve[0] + reserve[kProbeThreads - 1];
}

}  // namespace

int64_t launch_mfma_probe(int iters, float* sink, hipStream_t stream) {
  mfma_probe_kernel<<<kProbeBlocks, kProbeThreads, 0, stream>>>(iters, sink);
  if (hipGetLastError() != hipSuccess) return -1;
  return static_cast<int64_t>(kProbeBlocks) * (kProbeThreads / 64) * iters * 8 * (2 * 32 * 32 * 16);
}

}  // namespace lnf4
