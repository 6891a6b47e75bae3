// Fused NF4-LoRA linear, forward, generic-rank variant (any r up to the
// library maximum): y = x deq(Wt)^T + s (x A) B   (gfx950). 128 x 128 tiles,
// 16x16x32 MFMA; used for ranks the 256 x 256 kernel does not fuse (r > 64).
//
// One launch does the whole chain the kernel-fusion section of "Unsloth
// acceleration principles: CUDA kernel fusion and memory optimization"
// describes (base linear, LoRA down-projection, LoRA up-projection, add), with
// no intermediate written to HBM except the optional bf16 copy of U = x A that
// the backward reuses:
//   * K-loop in steps of 64 = one NF4 block per weight row, so each row of the
//     weight tile has exactly one absmax per step;
//   * the packed codes of the step are dequantized in registers (level lookup
//     in an LDS table, multiply by the row's absmax, round to bf16) and written
//     to LDS, where every wave reads its bf16 MFMA fragments;
//   * x fragments serve both the base product and U = x A in the same step
//     (A's 64 x r slice is staged transposed in LDS);
//   * the epilogue forms bf16(s U) and adds (s U) B into the fp32 accumulators
//     with one more MFMA pass over the rank dimension, then stores bf16 y.
#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int kThreads = 256;  // 4 waves in a 2 x 2 grid over the output tile
constexpr int kBK = 64;        // reduction step = one NF4 block
constexpr int kLds = kBK + 8;  // LDS row stride in bf16: 144 B keeps b128 fragment reads conflict-free

template <int BM, int BN, int RT>
struct FwdCfg {
  static constexpr int WM = BM / 2, WN = BN / 2;        // wave tile
  static constexpr int TM = WM / 16, TN = WN / 16;      // 16 x 16 MFMA tiles per wave
  static constexpr int RP = ((RT * 16 + 31) / 32) * 32; // rank padded to the MFMA reduction step
  static constexpr int UT = (RT + 1) / 2;               // U column tiles per wave (split over wn)
  static constexpr int EC = RP < 64 ? RP : 64;          // rank columns per epilogue pass
  static constexpr int ES = EC + 8;                     // epilogue LDS row stride
  static constexpr int SX = (BM * (ES > kLds ? ES : kLds));
  static constexpr int SW = (BN * (ES > kLds ? ES : kLds));
};

template <int BM, int BN, int RT>
__global__ __launch_bounds__(kThreads) void lora_fwd_kernel(
    int T, int K, int N, int r, float s, const uint16_t* __restrict__ x,
    const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ y,
    uint16_t* __restrict__ u_save) {
  using C = FwdCfg<BM, BN, RT>;
  __shared__ __align__(16) uint16_t xs[C::SX];
  __shared__ __align__(16) uint16_t ws[C::SW];
  __shared__ __align__(16) uint16_t as_[RT * 16 * kLds];
  __shared__ float lut[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, lq = lane >> 4;
  const int mt = (T + BM - 1) / BM, nt = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, mt * nt), mt, nt, 8, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int K2 = K / 2, KB = K / kBK;

  if (tid < 16) lut[tid] = nf4_level_reg(tid);

  f32x4_t acc[C::TM][C::TN];
  f32x4_t uacc[C::TM][C::UT];
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < C::UT; ++u) uacc[i][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  for (int kt = 0; kt < KB; ++kt) {
    const int k0 = kt * kBK;
    __syncthreads();  // the previous step's fragment reads are complete (and lut is visible)

    // x tile [BM x 64] -> xs (row-major, 16-byte chunks)
    for (int c = tid; c < BM * 8; c += kThreads) {
      const int row = c >> 3, ch = c & 7;
      uint4 v = {0u, 0u, 0u, 0u};
      if (m0 + row < T)
        v = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(m0 + row) * K + k0 + ch * 8);
      *reinterpret_cast<uint4*>(xs + row * kLds + ch * 8) = v;
    }
    // A slice [64 x r] -> as_ transposed (row j, reduction index contiguous)
    for (int e = tid; e < kBK * RT * 16; e += kThreads) {
      const int kk = e / (RT * 16), j = e - kk * (RT * 16);
      as_[j * kLds + kk] = (j < r) ? A[static_cast<size_t>(k0 + kk) * r + j] : uint16_t(0);
    }
    // NF4 weight tile [BN x 64]: two threads per row, 32 codes (16 bytes) each
    for (int c = tid; c < BN * 2; c += kThreads) {
      const int row = c >> 1, half = c & 1, n = n0 + row;
      uint4 cw = {0u, 0u, 0u, 0u};
      float a = 0.f;
      if (n < N) {
        cw = *reinterpret_cast<const uint4*>(codes + static_cast<size_t>(n) * K2 + k0 / 2 + half * 16);
        a = absmax[static_cast<size_t>(n) * KB + kt];
      }
      const uint32_t cws[4] = {cw.x, cw.y, cw.z, cw.w};
      uint16_t* dst = ws + row * kLds + half * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w = cws[q];
        uint4 o;
        o.x = pack_bf16x2(lut[w & 15u] * a, lut[(w >> 4) & 15u] * a);
        o.y = pack_bf16x2(lut[(w >> 8) & 15u] * a, lut[(w >> 12) & 15u] * a);
        o.z = pack_bf16x2(lut[(w >> 16) & 15u] * a, lut[(w >> 20) & 15u] * a);
        o.w = pack_bf16x2(lut[(w >> 24) & 15u] * a, lut[w >> 28] * a);
        *reinterpret_cast<uint4*>(dst + q * 8) = o;
      }
    }
    __syncthreads();

#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kc = kk * 32 + lq * 8;
      uint4 af[C::TM], bfr[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        af[i] = *reinterpret_cast<const uint4*>(xs + (wm * C::WM + i * 16 + l16) * kLds + kc);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        bfr[j] = *reinterpret_cast<const uint4*>(ws + (wn * C::WN + j * 16 + l16) * kLds + kc);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
#pragma unroll
      for (int u = 0; u < C::UT; ++u) {
        const int jt = 2 * u + wn;
        if (jt < RT) {
          const uint4 bu = *reinterpret_cast<const uint4*>(as_ + (jt * 16 + l16) * kLds + kc);
#pragma unroll
          for (int i = 0; i < C::TM; ++i) uacc[i][u] = mfma16(af[i], bu, uacc[i][u]);
        }
      }
    }
  }

  // ---- epilogue: acc += bf16(s U) B, EC rank columns per pass ---------------------
  if (u_save != nullptr && tn == 0) {
#pragma unroll
    for (int u = 0; u < C::UT; ++u) {
      const int jt = 2 * u + wn;
      if (jt < RT) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = wm * C::WM + i * 16 + lq * 4 + e, col = jt * 16 + l16;
            if (col < r && m0 + row < T) u_save[static_cast<size_t>(m0 + row) * r + col] = to_bf16(uacc[i][u][e]);
          }
      }
    }
  }
  uint16_t* us = xs;   // [BM][ES]  bf16(s U) columns c0 .. c0 + EC - 1, zero past the rank
  uint16_t* bts = ws;  // [BN][ES]  the same columns of B^T
#pragma unroll
  for (int c0 = 0; c0 < C::RP; c0 += C::EC) {
    __syncthreads();  // the previous pass (or the K-loop) is done with xs and ws
#pragma unroll
    for (int u = 0; u < C::UT; ++u) {
      const int jt = 2 * u + wn;
      if (jt < RT && jt * 16 >= c0 && jt * 16 < c0 + C::EC) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = wm * C::WM + i * 16 + lq * 4 + e;
            us[row * C::ES + jt * 16 - c0 + l16] = to_bf16(s * uacc[i][u][e]);
          }
      }
    }
    const int kTail = (RT * 16 > c0 && RT * 16 < c0 + C::EC) ? c0 + C::EC - RT * 16 : 0;
    if (RT * 16 <= c0) {
      for (int e = tid; e < BM * C::EC; e += kThreads) us[(e / C::EC) * C::ES + e % C::EC] = 0;
    } else if (kTail > 0) {
      for (int e = tid; e < BM * kTail; e += kThreads) {
        const int row = e / kTail, col = RT * 16 - c0 + (e - row * kTail);
        us[row * C::ES + col] = 0;
      }
    }
    for (int e = tid; e < C::EC * BN; e += kThreads) {
      const int j = e / BN, c = e - j * BN;
      bts[c * C::ES + j] = (c0 + j < r && n0 + c < N) ? B[static_cast<size_t>(c0 + j) * N + n0 + c] : uint16_t(0);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < C::EC / 32; ++ks) {
      const int kc = ks * 32 + lq * 8;
      uint4 af[C::TM], bfr[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        af[i] = *reinterpret_cast<const uint4*>(us + (wm * C::WM + i * 16 + l16) * C::ES + kc);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        bfr[j] = *reinterpret_cast<const uint4*>(bts + (wn * C::WN + j * 16 + l16) * C::ES + kc);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm * C::WM + i * 16 + lq * 4 + e;
        const int col = n0 + wn * C::WN + j * 16 + l16;
        if (row < T && col < N) y[static_cast<size_t>(row) * N + col] = to_bf16(acc[i][j][e]);
      }
}

template <int RT>
hipError_t launch_fwd_rt(int T, int K, int N, int r, float s, const uint16_t* x,
                         const uint8_t* codes, const float* absmax, const uint16_t* A,
                         const uint16_t* B, uint16_t* y, uint16_t* u_save, hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
  const int tiles = ((T + BM - 1) / BM) * ((N + BN - 1) / BN);
  lora_fwd_kernel<BM, BN, RT><<<tiles, kThreads, 0, stream>>>(T, K, N, r, s, x, codes, absmax, A, B,
                                                              y, u_save);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lora_fwd_generic(int T, int K, int N, int r, float s, const uint16_t* x,
                           const uint8_t* codes, const float* absmax, const uint16_t* A,
                           const uint16_t* B, uint16_t* y, uint16_t* u_save, hipStream_t stream) {
  switch (generic_rank_tiles(r)) {
    case 1: return launch_fwd_rt<1>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    case 2: return launch_fwd_rt<2>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    case 3: return launch_fwd_rt<3>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    case 4: return launch_fwd_rt<4>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    case 5: return launch_fwd_rt<5>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    case 6: return launch_fwd_rt<6>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    case 7: return launch_fwd_rt<7>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    case 8: return launch_fwd_rt<8>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    case 12: return launch_fwd_rt<12>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    case 16: return launch_fwd_rt<16>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lnf4
