// Fused NF4-LoRA linear, forward: y = x deq(Wt)^T + s (x A) B   (gfx950).
//
// One launch runs the whole chain the kernel-fusion section of "Unsloth
// acceleration principles: CUDA kernel fusion and memory optimization"
// describes (base linear, LoRA down-projection, LoRA up-projection, add); the
// only intermediate that reaches HBM is the optional bf16 copy of U = x A that
// the backward reuses.
//
// Work decomposition (MI355X, 256 CUs in 8 XCDs, 160 KB LDS per CU):
//   * 256 x 256 output tile per workgroup, 512 threads = 8 waves (2 per SIMD),
//     each wave owning a 128 x 64 sub-tile of 2 x 4 v_mfma_f32_32x32x16_bf16
//     accumulators. A large M-tile amortizes the in-loop dequantization: every
//     weight element is dequantized T/256 times over the whole GEMM.
//   * K-loop in steps of 64 = one NF4 block, so every weight row has exactly one
//     absmax per step. LDS holds two stages (x tile, dequantized weight tile,
//     A slice), XOR-swizzled for conflict-free 16-byte fragment reads; while the
//     MFMAs consume one stage, the next stage's x is stored and its packed codes
//     (already in registers) are dequantized into the other: level lookup in an
//     LDS table, multiply by the row's absmax, round to bf16.
//   * U = x A is accumulated in the same loop from the same x fragments: each
//     wave owns 32 token rows of U.
//   * Epilogue: bf16(s U) and B go through LDS, one more MFMA pass over the rank
//     dimension adds (s U) B into the accumulators, and bf16 y is stored.
#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int kThreads = 512;
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kTileElems = 256 * 64;  // one bf16 [256][64] tile

template <int RU>
struct FwdLds {
  static constexpr int kStageElems = 2 * kTileElems + RU * 64;  // x, W, A^T slice
  static constexpr int kLutByte = 2 * kStageElems * 2;
  static constexpr int kBytes = kLutByte + 64;
};

// RU: U columns accumulated in the K-loop (r rounded up to 32); RE: rank
// padded to the 16-wide reduction step of the epilogue MFMA.
template <int RU, int RE>
__global__ __launch_bounds__(kThreads) void lora_fwd_kernel(
    int T, int K, int N, int r, float s, const uint16_t* __restrict__ x,
    const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ y,
    uint16_t* __restrict__ u_save) {
  using L = FwdLds<RU>;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* const lds = reinterpret_cast<uint16_t*>(smem);
  float* const lut = reinterpret_cast<float*>(smem + L::kLutByte);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves, 128 x 64 each
  const int l32 = lane & 31, lh = lane >> 5;
  const int mt = (T + BM - 1) / BM, nt = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, mt * nt), mt, nt, 4, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int K2 = K / 2, KB = K / BK;

  if (tid < 16) lut[tid] = nf4_level(tid);
  // A^T slice rows r .. RU-1 stay zero in both stages
  for (int e = tid; e < 2 * (RU - r) * 64; e += kThreads) {
    const int st = e / ((RU - r) * 64), rem = e - st * (RU - r) * 64;
    lds[st * L::kStageElems + 2 * kTileElems + r * 64 + rem] = 0;
  }

  // ---- per-thread global->register staging of one K-step ------------------------
  // x: 4 chunks of 16 B (rows c>>3, chunk c&7 for c = tid + 512 i)
  // codes: row tid>>1, 16 bytes (32 codes) at half tid&1 of the 64-element block
  // A slice: the 64 x r block of A is contiguous; 8-element chunks tid + 512 i
  // (r % 8 == 0 on this path)
  constexpr int kAPer = (64 * RU / 8 + kThreads - 1) / kThreads;
  uint4 xr[4];
  uint4 cr;
  float ar;
  uint4 arr[kAPer];
  const int crow = tid >> 1, chalf = tid & 1;
  const bool crow_ok = n0 + crow < N;
  const uint8_t* cptr = codes + static_cast<size_t>(n0 + crow) * K2 + chalf * 16;
  const float* aptr = absmax + static_cast<size_t>(n0 + crow) * KB;

  auto load_stage = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i, row = c >> 3, ch = c & 7;
      xr[i] = (m0 + row < T)
                  ? *reinterpret_cast<const uint4*>(x + static_cast<size_t>(m0 + row) * K + k0 + ch * 8)
                  : uint4{0u, 0u, 0u, 0u};
    }
    if (crow_ok) {
      cr = *reinterpret_cast<const uint4*>(cptr + kt * 32);
      ar = aptr[kt];
    } else {
      cr = uint4{0u, 0u, 0u, 0u};
      ar = 0.f;
    }
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int c = tid + kThreads * i;
      arr[i] = (c < 8 * r) ? *reinterpret_cast<const uint4*>(A + static_cast<size_t>(k0) * r + c * 8)
                           : uint4{0u, 0u, 0u, 0u};
    }
  };

  auto store_stage = [&](int st) {
    uint16_t* xs = lds + st * L::kStageElems;
    uint16_t* ws = xs + kTileElems;
    uint16_t* as = ws + kTileElems;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i, row = c >> 3, ch = c & 7;
      *reinterpret_cast<uint4*>(xs + swz64(row, ch)) = xr[i];
    }
    const uint32_t cw[4] = {cr.x, cr.y, cr.z, cr.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w = cw[q];
      uint4 o;
      o.x = pack_bf16x2(lut[w & 15u] * ar, lut[(w >> 4) & 15u] * ar);
      o.y = pack_bf16x2(lut[(w >> 8) & 15u] * ar, lut[(w >> 12) & 15u] * ar);
      o.z = pack_bf16x2(lut[(w >> 16) & 15u] * ar, lut[(w >> 20) & 15u] * ar);
      o.w = pack_bf16x2(lut[(w >> 24) & 15u] * ar, lut[w >> 28] * ar);
      *reinterpret_cast<uint4*>(ws + swz64(crow, chalf * 4 + q)) = o;
    }
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int c = tid + kThreads * i;
      if (c < 8 * r) {
        const int e = c * 8, kk = e / r, j0 = e - kk * r;  // 8 consecutive j of one k (r % 8 == 0)
        const uint32_t v[4] = {arr[i].x, arr[i].y, arr[i].z, arr[i].w};
#pragma unroll
        for (int h = 0; h < 8; ++h)
          as[swz64(j0 + h, kk >> 3) + (kk & 7)] = static_cast<uint16_t>(v[h >> 1] >> (16 * (h & 1)));
      }
    }
  };

  f32x16_t acc[4][2];
  f32x16_t uacc[RU / 32 > 0 ? RU / 32 : 1];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
#pragma unroll
  for (int u = 0; u < (RU / 32 > 0 ? RU / 32 : 1); ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) uacc[u][e] = 0.f;

  load_stage(0);
  __syncthreads();  // lut and zeroed A^T rows visible
  store_stage(0);
  if (KB > 1) load_stage(1);
  __syncthreads();

  for (int kt = 0; kt < KB; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KB) store_stage(cur ^ 1);
    if (kt + 2 < KB) load_stage(kt + 2);
    const uint16_t* xs = lds + cur * L::kStageElems;
    const uint16_t* ws = xs + kTileElems;
    const uint16_t* as = ws + kTileElems;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = 2 * ks + lh;
      uint4 a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const uint4*>(xs + swz64(wm * 128 + i * 32 + l32, ch));
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const uint4*>(ws + swz64(wn * 64 + j * 32 + l32, ch));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
      if constexpr (RU > 0) {
        const uint4 au = *reinterpret_cast<const uint4*>(xs + swz64(wm * 128 + wn * 32 + l32, ch));
#pragma unroll
        for (int u = 0; u < RU / 32; ++u) {
          const uint4 bu = *reinterpret_cast<const uint4*>(as + swz64(u * 32 + l32, ch));
          uacc[u] = mfma32(au, bu, uacc[u]);
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: acc += bf16(s U) B ---------------------------------------------
  constexpr int ES = RE + 8;  // LDS row stride (bf16) of the rank-wide tiles
  uint16_t* us = lds;             // [256][ES]
  uint16_t* bt = lds + 256 * ES;  // [256][ES]: B^T tile
#pragma unroll
  for (int u = 0; u < RU / 32; ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = wm * 128 + wn * 32 + mfma32_row(e, lane), col = u * 32 + l32;
      const float uv = uacc[u][e];
      if (col < RE) us[row * ES + col] = to_bf16(s * uv);
      if (u_save != nullptr && tn == 0 && col < r && m0 + row < T)
        u_save[static_cast<size_t>(m0 + row) * r + col] = to_bf16(uv);
    }
  for (int e = tid; e < 256 * RE; e += kThreads) {
    const int j = e >> 8, c = e & 255;
    bt[c * ES + j] = (j < r && n0 + c < N) ? B[static_cast<size_t>(j) * N + n0 + c] : uint16_t(0);
  }
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < RE / 16; ++ks) {
    uint4 a[4], b[2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const uint4*>(us + (wm * 128 + i * 32 + l32) * ES + ks * 16 + lh * 8);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b[j] = *reinterpret_cast<const uint4*>(bt + (wn * 64 + j * 32 + l32) * ES + ks * 16 + lh * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * 128 + i * 32 + mfma32_row(e, lane);
        if (row < T && col < N) y[static_cast<size_t>(row) * N + col] = to_bf16(acc[i][j][e]);
      }
    }
}

template <int RU, int RE>
hipError_t launch_fwd_t(int T, int K, int N, int r, float s, const uint16_t* x, const uint8_t* codes,
                        const float* absmax, const uint16_t* A, const uint16_t* B, uint16_t* y,
                        uint16_t* u_save, hipStream_t stream) {
  constexpr int bytes = FwdLds<RU>::kBytes;
  static bool attr_set = false;  // benign race: every thread sets the same value
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lora_fwd_kernel<RU, RE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int tiles = ((T + BM - 1) / BM) * ((N + BN - 1) / BN);
  lora_fwd_kernel<RU, RE><<<tiles, kThreads, bytes, stream>>>(T, K, N, r, s, x, codes, absmax, A, B, y,
                                                              u_save);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lora_fwd(int T, int K, int N, int r, float s, const uint16_t* x,
                           const uint8_t* codes, const float* absmax, const uint16_t* A,
                           const uint16_t* B, uint16_t* y, uint16_t* u_save, hipStream_t stream) {
  if (r % 8 != 0)
    return launch_lora_fwd_generic(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
  switch ((r + 15) / 16) {
    case 1: return launch_fwd_t<32, 16>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    case 2: return launch_fwd_t<32, 32>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    case 3: return launch_fwd_t<64, 48>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    case 4: return launch_fwd_t<64, 64>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    default:
      return launch_lora_fwd_generic(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
  }
}

}  // namespace lnf4
