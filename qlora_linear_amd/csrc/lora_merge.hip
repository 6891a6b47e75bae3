// Merged base weight for export: W' = D + s (A B)^T, [d_out, d_in] (gfx950).
//
// After training the adapters are folded into the base weight and saved at 16
// bits ("Unsloth in three lines of code", section 4; "Reading the Unsloth
// changelog", the command-line part of section 2: saving turns the 4-bit model
// into a 16-bit one). Each element is
//     fl32( fl32(q[code] * absmax) + s * sum_j A[k][j] B[j][n] ),
// the low-rank sum accumulated in float32 by MFMA, then rounded once to the
// output type (bf16 nearest-even, or float32).
//
// One 256-thread workgroup per 64 x 256 tile (64 rows n of d_out, 256 columns k
// of d_in). The op is bound by HBM (0.5625 bytes of packed weight in, 2 or 4
// bytes out per element):
//   1. A rows k0 .. k0 + 255 and B columns n0 .. n0 + 63 go to LDS, rank padded
//      with zeros to a multiple of 32 (the only LDS use, so several workgroups
//      share a CU);
//   2. v_mfma_f32_16x16x32_bf16 forms (A B)^T with A as the row operand (its rows
//      are contiguous in the reduction j). The MFMA row m of block b reads A row
//      16 (m >> 2) + 4 b + (m & 3) of the wave's 64 columns, so that across the
//      four blocks a lane's accumulators hold 16 consecutive columns k of one row
//      n;
//   3. each lane dequantizes exactly those 16 elements (8 bytes of codes, one
//      absmax), adds s times its accumulators and stores 32 (bf16) or 64
//      (float32) contiguous bytes: no second pass through LDS.
#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kMN = 64;    // d_out rows per workgroup
constexpr int kMK = 256;   // d_in columns per workgroup (64 per wave)

template <int RP, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void lora_merge_kernel(int K, int N, int r, float s,
                                                              const uint8_t* __restrict__ codes,
                                                              const float* __restrict__ absmax,
                                                              const uint16_t* __restrict__ A,
                                                              const uint16_t* __restrict__ B,
                                                              void* __restrict__ out) {
  constexpr int RS = RP + 8;  // bf16 row stride of the staged factors
  __shared__ __align__(1024) float lut[16];
  __shared__ __align__(16) uint16_t at[kMK * RS];
  __shared__ __align__(16) uint16_t bt[kMN * RS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int k0 = blockIdx.x * kMK, n0 = blockIdx.y * kMN;
  const int kw = k0 + 64 * wave;  // this wave's 64 columns (one NF4 block per row)
  if (tid < 16) lut[tid] = nf4_level(tid);

  // step 3's codes and absmax, loaded first so their latency overlaps steps 1-2:
  // n-block nb, lane (l16, g): row n0 + 16 nb + l16, columns kw + 16 g .. +15
  const int K2 = K / 2, KB = K / 64;
  uint2 cw[4];
  float av[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int n = n0 + 16 * nb + l16;
    const bool ok = n < N && kw < K;
    cw[nb] = ok ? *reinterpret_cast<const uint2*>(codes + static_cast<size_t>(n) * K2 + kw / 2 + 8 * g)
                : uint2{0u, 0u};
    av[nb] = ok ? absmax[static_cast<size_t>(n) * KB + kw / 64] : 0.f;
  }

  // ---- 1. stage A and B (batches of 8 independent loads: a plain loop waits on
  // each). A rows k0 .. k0 + 255 are one contiguous run of 256 r elements.
  const int na = kMK * r;
  for (int e0 = tid; e0 < na; e0 += 8 * kThreads) {
    uint16_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * kThreads;
      v[u] = (e < na && k0 + e / r < K) ? A[static_cast<size_t>(k0) * r + e] : uint16_t(0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * kThreads;
      if (e < na) at[(e / r) * RS + e % r] = v[u];
    }
  }
  for (int e = tid; e < kMK * (RP - r); e += kThreads) {
    const int kk = e / (RP - r), j = r + e - kk * (RP - r);
    at[kk * RS + j] = 0;
  }
  for (int e0 = tid; e0 < kMN * RP; e0 += 8 * kThreads) {
    uint16_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * kThreads, j = e / kMN, nn = e % kMN;
      v[u] = (e < kMN * RP && j < r && n0 + nn < N) ? B[static_cast<size_t>(j) * N + n0 + nn] : uint16_t(0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * kThreads;
      if (e < kMN * RP) bt[(e % kMN) * RS + e / kMN] = v[u];
    }
  }
  __syncthreads();
  if (kw >= K) return;

  // ---- 2 + 3. per n-block: (A B)^T for 16 rows x 64 columns, then the elements
  const int arow = 64 * wave + 16 * (l16 >> 2) + (l16 & 3);  // + 4 b: A row of MFMA row l16, block b
  const unsigned char* lutb = reinterpret_cast<const unsigned char*>(lut);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int n = n0 + 16 * nb + l16;
    f32x4_t acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jq = 0; jq < RP / 32; ++jq) {
        const uint4 a = *reinterpret_cast<const uint4*>(at + (arow + 4 * b) * RS + 32 * jq + 8 * g);
        const uint4 bb = *reinterpret_cast<const uint4*>(bt + (16 * nb + l16) * RS + 32 * jq + 8 * g);
        acc[b] = mfma16(a, bb, acc[b]);
      }
    }
    if (n >= N) continue;
    // lane (l16, g) now holds column 16 g + 4 b + e of row n in acc[b][e]
    const float sc = av[nb];
    const uint32_t w2[2] = {cw[nb].x, cw[nb].y};
    float v[16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // 8 codes per dword, the even element in the low nibble
      uint32_t ev = (w2[h] << 2) & 0x3C3C3C3Cu, od = (w2[h] >> 2) & 0x3C3C3C3Cu;
      asm volatile("" : "+v"(ev), "+v"(od));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i0 = 8 * h + 2 * j, i1 = i0 + 1;
        v[i0] = *reinterpret_cast<const float*>(lutb + __builtin_amdgcn_ubfe(ev, 8 * j, 8)) * sc +
                s * acc[i0 >> 2][i0 & 3];
        v[i1] = *reinterpret_cast<const float*>(lutb + __builtin_amdgcn_ubfe(od, 8 * j, 8)) * sc +
                s * acc[i1 >> 2][i1 & 3];
      }
    }
    const size_t o = static_cast<size_t>(n) * K + kw + 16 * g;
    if constexpr (OUT_BF16) {
      uint4* op = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + o);
      op[0] = uint4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7])};
      op[1] = uint4{pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]), pack_bf16x2(v[12], v[13]),
                    pack_bf16x2(v[14], v[15])};
    } else {
      float4* op = reinterpret_cast<float4*>(static_cast<float*>(out) + o);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) op[q4] = float4{v[4 * q4], v[4 * q4 + 1], v[4 * q4 + 2], v[4 * q4 + 3]};
    }
  }
}

template <int RP>
hipError_t launch_merge_t(int K, int N, int r, float s, const uint8_t* codes, const float* absmax,
                          const uint16_t* A, const uint16_t* B, bool out_bf16, void* out,
                          hipStream_t stream) {
  const dim3 grid((K + kMK - 1) / kMK, (N + kMN - 1) / kMN);
  if (out_bf16)
    lora_merge_kernel<RP, true><<<grid, kThreads, 0, stream>>>(K, N, r, s, codes, absmax, A, B, out);
  else
    lora_merge_kernel<RP, false><<<grid, kThreads, 0, stream>>>(K, N, r, s, codes, absmax, A, B, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lora_merge(int K, int N, int r, float s, const uint8_t* codes, const float* absmax,
                             const uint16_t* A, const uint16_t* B, bool out_bf16, void* out,
                             hipStream_t stream) {
  switch ((r + 31) / 32) {
    case 1: return launch_merge_t<32>(K, N, r, s, codes, absmax, A, B, out_bf16, out, stream);
    case 2: return launch_merge_t<64>(K, N, r, s, codes, absmax, A, B, out_bf16, out, stream);
    case 3: return launch_merge_t<96>(K, N, r, s, codes, absmax, A, B, out_bf16, out, stream);
    default: return launch_merge_t<128>(K, N, r, s, codes, absmax, A, B, out_bf16, out, stream);
  }
}

}  // namespace lnf4
