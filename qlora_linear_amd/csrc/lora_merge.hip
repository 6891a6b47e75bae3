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
//      with zeros to a multiple of 32, at most 128 rank columns per pass (the only
//      LDS use, so several workgroups share a CU);
//   2. v_mfma_f32_16x16x32_bf16 forms (A B)^T with A as the row operand (its rows
//      are contiguous in the reduction j). The MFMA row m of block b reads A row
//      32 (b >> 1) + 8 (m >> 2) + 4 (b & 1) + (m & 3) of the wave's 64 columns, so
//      that a lane (m = l16, g) holds columns 8 g .. 8 g + 7 (blocks 0, 1) and
//      32 + 8 g .. 32 + 8 g + 7 (blocks 2, 3) of one row n;
//   3. each lane dequantizes exactly those 16 elements (2 x 4 bytes of codes, one
//      absmax), adds s times its accumulators and stores them: the four lanes of a
//      row write 64 contiguous bytes per bf16 store instruction (128 per float32
//      pair); no second pass through LDS.
#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kMN = 64;    // d_out rows per workgroup
constexpr int kMK = 256;   // d_in columns per workgroup (64 per wave)

// MP: more than one rank pass (r > RP); otherwise the pass loop is compiled out and
// only one n-block's accumulators are live at a time.
template <int RP, bool OUT_BF16, bool MP>
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
  // n-block nb, lane (l16, g): row n0 + 16 nb + l16, columns kw + 8 g .. +7 and
  // kw + 32 + 8 g .. +7
  const int K2 = K / 2, KB = K / 64;
  uint2 cw[4];
  float av[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int n = n0 + 16 * nb + l16;
    const bool ok = n < N && kw < K;
    const uint32_t* crow = reinterpret_cast<const uint32_t*>(codes + static_cast<size_t>(n) * K2 + kw / 2);
    cw[nb] = ok ? uint2{crow[g], crow[4 + g]} : uint2{0u, 0u};
    av[nb] = ok ? absmax[static_cast<size_t>(n) * KB + kw / 64] : 0.f;
  }

  // ---- 1. stage A and B, RP rank columns per pass (one pass up to r = 128). A rows
  // k0 .. k0 + 255 and B columns n0 .. n0 + 63 of the pass's rank columns go to LDS
  // as 16-byte pieces, element by element where a row of A (r % 8 != 0) or of B
  // (d_out % 8 != 0) is not 16-byte aligned; rank columns past r are zero.
  // ---- 2. per n-block: (A B)^T for 16 rows x 64 columns, accumulated over the passes.
  // A row of MFMA row l16 in block b: 64 wave + 32 (b >> 1) + 8 (l16 >> 2) + 4 (b & 1) + (l16 & 3)
  const int arow = 64 * wave + 8 * (l16 >> 2) + (l16 & 3);
  f32x4_t acc[4][4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[nb][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bool avec = r % 8 == 0, bvec = N % 8 == 0;
  auto stage = [&](int j0) {
    for (int c = tid; c < kMK * (RP / 8); c += kThreads) {
      const int kk = c / (RP / 8), j = j0 + 8 * (c - kk * (RP / 8));
      uint4 v = {0u, 0u, 0u, 0u};
      if (j < r && k0 + kk < K) {
        const uint16_t* src = A + static_cast<size_t>(k0 + kk) * r + j;
        v = avec ? *reinterpret_cast<const uint4*>(src) : load8_masked(src, r - j);
      }
      *reinterpret_cast<uint4*>(at + kk * RS + (j - j0)) = v;
    }
    for (int c = tid; c < RP * (kMN / 8); c += kThreads) {
      const int jj = c / (kMN / 8), nn = 8 * (c - jj * (kMN / 8)), j = j0 + jj;
      uint4 v = {0u, 0u, 0u, 0u};
      if (j < r && n0 + nn < N) {
        const uint16_t* src = B + static_cast<size_t>(j) * N + n0 + nn;
        v = bvec ? *reinterpret_cast<const uint4*>(src) : load8_masked(src, N - n0 - nn);
      }
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int t = 0; t < 8; ++t) bt[(nn + t) * RS + jj] = static_cast<uint16_t>(w[t >> 1] >> (16 * (t & 1)));
    }
  };
  auto product = [&](int nb, f32x4_t* a4) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int jq = 0; jq < RP / 32; ++jq) {
        const uint4 a = *reinterpret_cast<const uint4*>(at + (arow + 32 * (b >> 1) + 4 * (b & 1)) * RS + 32 * jq + 8 * g);
        const uint4 bb = *reinterpret_cast<const uint4*>(bt + (16 * nb + l16) * RS + 32 * jq + 8 * g);
        a4[b] = mfma16(a, bb, a4[b]);
      }
  };
  // every pass but the last accumulates all four n-blocks; the last pass forms each
  // n-block's product right before its elements (one pass for r <= 128)
  int j0 = 0;
  for (; MP && j0 + RP < r; j0 += RP) {
    stage(j0);
    __syncthreads();
    if (kw < K)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) product(nb, acc[nb]);
    __syncthreads();
  }
  stage(j0);
  __syncthreads();
  if (kw >= K) return;

  // ---- 3. the elements: lane (l16, g) holds column 32 (b >> 1) + 8 g + 4 (b & 1) + e
  // of row n in acc[nb][b][e]; v[i] is column 8 g + i (i < 8) or 32 + 8 g + i - 8,
  // i.e. acc[nb][i >> 2][i & 3]
  const unsigned char* lutb = reinterpret_cast<const unsigned char*>(lut);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int n = n0 + 16 * nb + l16;
    product(nb, acc[nb]);
    if (n >= N) continue;
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
        v[i0] = __fmul_rn(*reinterpret_cast<const float*>(lutb + __builtin_amdgcn_ubfe(ev, 8 * j, 8)), sc) +
                s * acc[nb][i0 >> 2][i0 & 3];
        v[i1] = __fmul_rn(*reinterpret_cast<const float*>(lutb + __builtin_amdgcn_ubfe(od, 8 * j, 8)), sc) +
                s * acc[nb][i1 >> 2][i1 & 3];
      }
    }
    const size_t o = static_cast<size_t>(n) * K + kw + 8 * g;
    if constexpr (OUT_BF16) {
      uint16_t* op = static_cast<uint16_t*>(out) + o;
      *reinterpret_cast<uint4*>(op) = uint4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                           pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
      *reinterpret_cast<uint4*>(op + 32) = uint4{pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]),
                                                pack_bf16x2(v[12], v[13]), pack_bf16x2(v[14], v[15])};
    } else {
      float* op = static_cast<float*>(out) + o;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4*>(op + (q4 >> 1) * 32 + (q4 & 1) * 4) =
            float4{v[4 * q4], v[4 * q4 + 1], v[4 * q4 + 2], v[4 * q4 + 3]};
    }
  }
}

template <int RP, bool MP = false>
hipError_t launch_merge_t(int K, int N, int r, float s, const uint8_t* codes, const float* absmax,
                          const uint16_t* A, const uint16_t* B, bool out_bf16, void* out,
                          hipStream_t stream) {
  const dim3 grid((K + kMK - 1) / kMK, (N + kMN - 1) / kMN);
  if (out_bf16)
    lora_merge_kernel<RP, true, MP><<<grid, kThreads, 0, stream>>>(K, N, r, s, codes, absmax, A, B, out);
  else
    lora_merge_kernel<RP, false, MP><<<grid, kThreads, 0, stream>>>(K, N, r, s, codes, absmax, A, B, out);
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
    case 4: return launch_merge_t<128>(K, N, r, s, codes, absmax, A, B, out_bf16, out, stream);
    default: return launch_merge_t<128, true>(K, N, r, s, codes, absmax, A, B, out_bf16, out, stream);
  }
}

}  // namespace lnf4
