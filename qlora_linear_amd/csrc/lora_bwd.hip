// Fused NF4-LoRA linear, backward (gfx950).
//
// The pages replace autograd with hand-written backward kernels ("Unlocking AI
// potential: Unsloth's algorithms and implementation", core-algorithms section;
// "Unsloth performance measured: is it really 2x faster?", section 3). For the
// LoRA linear with frozen NF4 base, s = alpha / r and D = deq(Wt):
//     G  = s dY B^T        dX = dY D + G A^T        dA = x^T G        dB = s U^T dY
// Kernels, all on the caller's stream with no host synchronization:
//   1. lora_dx_kernel   — K-loop over d_out in NF4-block steps: dequantizes the
//      weight tile into LDS transposed (reduction index contiguous), bf16 MFMA
//      for dY D; G = s dY B^T accumulated from the same dY fragments; epilogue
//      adds G A^T and stores dX; the first column tile also writes bf16 G.
//   2. lora_u_kernel    — U = x A when the forward's copy is not supplied.
//   3. skinny_tn_kernel — split-T partial sums of M^T V for the two rank-r
//      gradients (dA: M = x, V = G; dB: M = dY, V = U), bf16 MFMA on tiles
//      staged transposed in LDS.
//   4. skinny_reduce_kernel — fixed-order sum of the partials (deterministic),
//      scale, bf16 store in the gradient's layout.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;
constexpr int kLds = kBK + 8;

template <int BM, int BN, int RT>
struct DxCfg {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int RP = ((RT * 16 + 31) / 32) * 32;
  static constexpr int UT = (RT + 1) / 2;
  static constexpr int EC = RP < 64 ? RP : 64;  // rank columns per epilogue pass
  static constexpr int ES = EC + 8;
  static constexpr int SX = (BM * (ES > kLds ? ES : kLds));
  static constexpr int SW = (BN * (ES > kLds ? ES : kLds));
  static constexpr int KPW = BN / 4;  // weight columns (k) dequantized per wave per step
};

template <int BM, int BN, int RT>
__global__ __launch_bounds__(kThreads) void lora_dx_kernel(
    int T, int K, int N, int r, float s, const uint16_t* __restrict__ dy,
    const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ dx,
    uint16_t* __restrict__ g_out) {
  using C = DxCfg<BM, BN, RT>;
  __shared__ __align__(16) uint16_t dys[C::SX];   // dY tile [BM][64 of n]
  __shared__ __align__(16) uint16_t ds[C::SW];    // deq weight, transposed: [BN of k][64 of n]
  __shared__ __align__(16) uint16_t bs[RT * 16 * kLds];  // B slice [r][64 of n]
  __shared__ float lut[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, lq = lane >> 4;
  const int mt = (T + BM - 1) / BM, kt_tiles = (K + BN - 1) / BN;
  int tm, tk;
  tile_coords(xcd_remap(blockIdx.x, mt * kt_tiles), mt, kt_tiles, 8, tm, tk);
  const int m0 = tm * BM, k0 = tk * BN;
  const int K2 = K / 2, KB = K / kBK;

  if (tid < 16) lut[tid] = nf4_level_reg(tid);

  f32x4_t acc[C::TM][C::TN];
  f32x4_t gacc[C::TM][C::UT];
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < C::UT; ++u) gacc[i][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int NS = (N + kBK - 1) / kBK;
  const bool vec = (N & 7) == 0;
  for (int ns = 0; ns < NS; ++ns) {
    const int n0 = ns * kBK;
    __syncthreads();
    // dY tile [BM x 64]
    // (16-byte loads when d_out % 8 == 0; otherwise rows are not 16-byte aligned and
    // the last chunk of a row would run into the next, so element by element)
    for (int c = tid; c < BM * 8; c += kThreads) {
      const int row = c >> 3, ch = c & 7;
      uint4 v = {0u, 0u, 0u, 0u};
      if (m0 + row < T && n0 + ch * 8 < N) {
        const uint16_t* src = dy + static_cast<size_t>(m0 + row) * N + n0 + ch * 8;
        v = vec ? *reinterpret_cast<const uint4*>(src) : load8_masked(src, N - n0 - ch * 8);
      }
      *reinterpret_cast<uint4*>(dys + row * kLds + ch * 8) = v;
    }
    // B slice [r x 64] (rows of B are contiguous in n)
    for (int c = tid; c < RT * 16 * 8; c += kThreads) {
      const int j = c >> 3, ch = c & 7;
      uint4 v = {0u, 0u, 0u, 0u};
      if (j < r && n0 + ch * 8 < N) {
        const uint16_t* src = B + static_cast<size_t>(j) * N + n0 + ch * 8;
        v = vec ? *reinterpret_cast<const uint4*>(src) : load8_masked(src, N - n0 - ch * 8);
      }
      *reinterpret_cast<uint4*>(bs + j * kLds + ch * 8) = v;
    }
    // weight tile: lane = row n (64 rows), wave = a run of KPW columns k;
    // dequantized values are written transposed, ds[k][n].
    {
      const int n = n0 + lane;
#pragma unroll
      for (int part = 0; part < C::KPW / 32; ++part) {
        const int kl = wave * C::KPW + part * 32;  // local k of this 32-run
        const int kg = k0 + kl;
        uint4 cw = {0u, 0u, 0u, 0u};
        float a = 0.f;
        if (n < N && kg < K) {
          cw = *reinterpret_cast<const uint4*>(codes + static_cast<size_t>(n) * K2 + kg / 2);
          a = absmax[static_cast<size_t>(n) * KB + kg / kBK];
        }
        const uint32_t cws[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int h = 0; h < 8; ++h) {
            const float v = lut[(cws[q] >> (4 * h)) & 15u] * a;
            ds[(kl + q * 8 + h) * kLds + lane] = to_bf16(v);
          }
        }
      }
    }
    __syncthreads();

#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kc = kk * 32 + lq * 8;
      uint4 af[C::TM], bfr[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        af[i] = *reinterpret_cast<const uint4*>(dys + (wm * C::WM + i * 16 + l16) * kLds + kc);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        bfr[j] = *reinterpret_cast<const uint4*>(ds + (wn * C::WN + j * 16 + l16) * kLds + kc);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
#pragma unroll
      for (int u = 0; u < C::UT; ++u) {
        const int jt = 2 * u + wn;
        if (jt < RT) {
          const uint4 bu = *reinterpret_cast<const uint4*>(bs + (jt * 16 + l16) * kLds + kc);
#pragma unroll
          for (int i = 0; i < C::TM; ++i) gacc[i][u] = mfma16(af[i], bu, gacc[i][u]);
        }
      }
    }
  }

  // ---- epilogue: acc += bf16(G) A^T, G = s dY B^T, EC rank columns per pass --------
  if (tk == 0) {
#pragma unroll
    for (int u = 0; u < C::UT; ++u) {
      const int jt = 2 * u + wn;
      if (jt < RT) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = wm * C::WM + i * 16 + lq * 4 + e, col = jt * 16 + l16;
            if (col < r && m0 + row < T) g_out[static_cast<size_t>(m0 + row) * r + col] = to_bf16(s * gacc[i][u][e]);
          }
      }
    }
  }
  if (dx == nullptr) return;
  uint16_t* gs = dys;  // [BM][ES]: bf16(G) columns c0 .. c0 + EC - 1, zero past the rank
  uint16_t* at = ds;   // [BN][ES]: rows k, the same rank columns (A is [K, r] row-major)
#pragma unroll
  for (int c0 = 0; c0 < C::RP; c0 += C::EC) {
    __syncthreads();  // the previous pass (or the K-loop) is done with dys and ds
#pragma unroll
    for (int u = 0; u < C::UT; ++u) {
      const int jt = 2 * u + wn;
      if (jt < RT && jt * 16 >= c0 && jt * 16 < c0 + C::EC) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = wm * C::WM + i * 16 + lq * 4 + e;
            gs[row * C::ES + jt * 16 - c0 + l16] = to_bf16(s * gacc[i][u][e]);
          }
      }
    }
    const int tail = (RT * 16 > c0 && RT * 16 < c0 + C::EC) ? c0 + C::EC - RT * 16 : 0;
    for (int e = tid; e < BM * tail; e += kThreads) {
      const int row = e / tail, col = RT * 16 - c0 + (e - row * tail);
      gs[row * C::ES + col] = 0;
    }
    for (int e = tid; e < BN * C::EC; e += kThreads) {
      const int c = e / C::EC, j = e - c * C::EC;
      at[c * C::ES + j] = (c0 + j < r && k0 + c < K) ? A[static_cast<size_t>(k0 + c) * r + c0 + j] : uint16_t(0);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < C::EC / 32; ++ks) {
      const int kc = ks * 32 + lq * 8;
      uint4 af[C::TM], bfr[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        af[i] = *reinterpret_cast<const uint4*>(gs + (wm * C::WM + i * 16 + l16) * C::ES + kc);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        bfr[j] = *reinterpret_cast<const uint4*>(at + (wn * C::WN + j * 16 + l16) * C::ES + kc);
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
        const int col = k0 + wn * C::WN + j * 16 + l16;
        if (row < T && col < K) dx[static_cast<size_t>(row) * K + col] = to_bf16(acc[i][j][e]);
      }
}

// U = x A, bf16 [T, r]: 64 token rows per workgroup, one 16-row strip per wave.
template <int RT>
__global__ __launch_bounds__(kThreads) void lora_u_kernel(int T, int K, int r,
                                                          const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ A,
                                                          uint16_t* __restrict__ u) {
  __shared__ __align__(16) uint16_t xs[64 * kLds];
  __shared__ __align__(16) uint16_t as_[RT * 16 * kLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int m0 = blockIdx.x * 64;
  f32x4_t uacc[RT];
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) uacc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();
    for (int c = tid; c < 64 * 8; c += kThreads) {
      const int row = c >> 3, ch = c & 7;
      uint4 v = {0u, 0u, 0u, 0u};
      if (m0 + row < T)
        v = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(m0 + row) * K + k0 + ch * 8);
      *reinterpret_cast<uint4*>(xs + row * kLds + ch * 8) = v;
    }
    for (int e = tid; e < kBK * RT * 16; e += kThreads) {
      const int kk = e / (RT * 16), j = e - kk * (RT * 16);
      as_[j * kLds + kk] = (j < r) ? A[static_cast<size_t>(k0 + kk) * r + j] : uint16_t(0);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kc = kk * 32 + lq * 8;
      const uint4 af = *reinterpret_cast<const uint4*>(xs + (wave * 16 + l16) * kLds + kc);
#pragma unroll
      for (int jt = 0; jt < RT; ++jt) {
        const uint4 bu = *reinterpret_cast<const uint4*>(as_ + (jt * 16 + l16) * kLds + kc);
        uacc[jt] = mfma16(af, bu, uacc[jt]);
      }
    }
  }
#pragma unroll
  for (int jt = 0; jt < RT; ++jt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = m0 + wave * 16 + lq * 4 + e, col = jt * 16 + l16;
      if (row < T && col < r) u[static_cast<size_t>(row) * r + col] = to_bf16(uacc[jt][e]);
    }
}

// partial[split][c][j] = sum over the split's token range of M[t][c] * V[t][j].
// M is [T, C] (any C), V is [T, r]. 128 columns per workgroup; each wave
// owns 32 columns x all rank tiles. Both operands are staged transposed in LDS
// so the token (reduction) index is contiguous for the MFMA fragments.
template <int RT>
__global__ __launch_bounds__(kThreads) void skinny_tn_kernel(int T, int Ccols, int r, int t_chunk,
                                                             const uint16_t* __restrict__ M,
                                                             const uint16_t* __restrict__ V,
                                                             float* __restrict__ partial) {
  constexpr int BC = 128;
  __shared__ __align__(16) uint16_t mts[BC * kLds];
  __shared__ __align__(16) uint16_t vts[RT * 16 * kLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int c0 = blockIdx.x * BC;
  const int split = blockIdx.y;
  const int t_begin = split * t_chunk;
  const int t_end = min(T, t_begin + t_chunk);
  f32x4_t acc[2][RT];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jt = 0; jt < RT; ++jt) acc[i][jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int t0 = t_begin; t0 < t_end; t0 += kBK) {
    __syncthreads();
    for (int c = tid; c < kBK * (BC / 8); c += kThreads) {
      const int tl = c / (BC / 8), ch = c - tl * (BC / 8);
      uint4 v = {0u, 0u, 0u, 0u};
      if (t0 + tl < t_end && c0 + ch * 8 < Ccols) {
        const uint16_t* src = M + static_cast<size_t>(t0 + tl) * Ccols + c0 + ch * 8;
        v = (Ccols & 7) == 0 ? *reinterpret_cast<const uint4*>(src) : load8_masked(src, Ccols - c0 - ch * 8);
      }
      const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        mts[(ch * 8 + 2 * h) * kLds + tl] = static_cast<uint16_t>(vv[h] & 0xFFFFu);
        mts[(ch * 8 + 2 * h + 1) * kLds + tl] = static_cast<uint16_t>(vv[h] >> 16);
      }
    }
    for (int e = tid; e < kBK * RT * 16; e += kThreads) {
      const int tl = e / (RT * 16), j = e - tl * (RT * 16);
      vts[j * kLds + tl] = (j < r && t0 + tl < t_end) ? V[static_cast<size_t>(t0 + tl) * r + j] : uint16_t(0);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kc = kk * 32 + lq * 8;
      uint4 af[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const uint4*>(mts + (wave * 32 + i * 16 + l16) * kLds + kc);
#pragma unroll
      for (int jt = 0; jt < RT; ++jt) {
        const uint4 bv = *reinterpret_cast<const uint4*>(vts + (jt * 16 + l16) * kLds + kc);
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i][jt] = mfma16(af[i], bv, acc[i][jt]);
      }
    }
  }
  constexpr int RS = RT * 16;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jt = 0; jt < RT; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = c0 + wave * 32 + i * 16 + lq * 4 + e, j = jt * 16 + l16;
        if (c < Ccols) partial[(static_cast<size_t>(split) * Ccols + c) * RS + j] = acc[i][jt][e];
      }
}

// out = scale * sum_split partial, in split order; bf16 [C, r] or, transposed, [r, C].
__global__ __launch_bounds__(kThreads) void skinny_reduce_kernel(const float* __restrict__ partial,
                                                                 int splits, int Ccols, int r, int rs,
                                                                 float scale, int transposed,
                                                                 uint16_t* __restrict__ out) {
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= Ccols * r) return;
  int c, j;
  if (transposed) {
    j = idx / Ccols;
    c = idx - j * Ccols;
  } else {
    c = idx / r;
    j = idx - c * r;
  }
  float sum = 0.f;
  for (int sp = 0; sp < splits; ++sp) sum += partial[(static_cast<size_t>(sp) * Ccols + c) * rs + j];
  out[idx] = to_bf16(scale * sum);
}

template <int RT>
hipError_t launch_bwd_rt(int T, int K, int N, int r, float s, const uint16_t* x,
                         const uint16_t* dy, const uint8_t* codes, const float* absmax,
                         const uint16_t* A, const uint16_t* B, const uint16_t* u_saved,
                         uint16_t* dx, uint16_t* dA, uint16_t* dB, void* workspace,
                         const BwdPlan& p, hipStream_t stream, const SkinnyAdamW* adam) {
  if (adam != nullptr && !p.fast) return hipErrorInvalidValue;
  char* ws = static_cast<char*>(workspace);
  uint16_t* g = reinterpret_cast<uint16_t*>(ws + p.off_g);
  uint16_t* u = reinterpret_cast<uint16_t*>(ws + p.off_u);
  float* pa = reinterpret_cast<float*>(ws + p.off_pa);
  float* pb = reinterpret_cast<float*>(ws + p.off_pb);
  hipError_t e;
  if (p.splitk) {
    e = launch_lora_dx_splitk(T, K, N, r, s, dy, codes, absmax, A, B, dx, g,
                              reinterpret_cast<float*>(ws + p.off_px),
                              reinterpret_cast<float*>(ws + p.off_pg), stream);
  } else if (p.rwx) {
    e = launch_dx_rw(T, K, N, s, dy, codes, absmax, A, B, dx, g, ws + p.off_w, stream);
  } else if (p.fast) {
    const bool split = p.splits_x > 1;
    uint16_t* w = p.dqx ? reinterpret_cast<uint16_t*>(ws + p.off_w) : nullptr;
    if (p.dqx && (e = launch_nf4_dequantize(codes, absmax, N, K, true, w, stream)) != hipSuccess) return e;
    if (p.gpass) {
      // G = s dY B^T in a pass of its own; the dX tiles (if any) read it back
      if ((e = launch_gpass(T, N, r, s, dy, B, g, r, stream)) != hipSuccess) return e;
      e = dx == nullptr ? hipSuccess
                        : launch_lora_dx(T, K, N, r, s, dy, codes, absmax, A, B, w, dx, g, nullptr, nullptr,
                                         stream, true);
    } else {
      e = launch_lora_dx(T, K, N, r, s, dy, codes, absmax, A, B, w, dx, g,
                         split ? reinterpret_cast<float*>(ws + p.off_px) : nullptr,
                         split ? reinterpret_cast<float*>(ws + p.off_pg) : nullptr, stream);
    }
  } else {
    constexpr int BM = 128, BN = 128;
    const int tiles = ((T + BM - 1) / BM) * ((K + BN - 1) / BN);
    lora_dx_kernel<BM, BN, RT><<<tiles, kThreads, 0, stream>>>(T, K, N, r, s, dy, codes, absmax, A,
                                                               B, dx, g);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  const uint16_t* uu = u_saved;
  if (uu == nullptr) {
    lora_u_kernel<RT><<<(T + 63) / 64, kThreads, 0, stream>>>(T, K, r, x, A, u);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    uu = u;
  }
  if (p.fast) {
    DaOut da{};
    da.p[0] = dA;
    da.gw = r;
    return launch_lora_skinny(T, K, N, r, r, r, s, x, g, dy, uu, pa, pb, p.splits_a, da, dB, stream, adam);
  }
  const int tca = (T + p.splits_a - 1) / p.splits_a;
  const int tcb = (T + p.splits_b - 1) / p.splits_b;
  skinny_tn_kernel<RT><<<dim3((K + 127) / 128, p.splits_a), kThreads, 0, stream>>>(T, K, r, tca, x, g,
                                                                                   pa);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  skinny_tn_kernel<RT><<<dim3((N + 127) / 128, p.splits_b), kThreads, 0, stream>>>(T, N, r, tcb, dy,
                                                                                   uu, pb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  skinny_reduce_kernel<<<(K * r + kThreads - 1) / kThreads, kThreads, 0, stream>>>(
      pa, p.splits_a, K, r, RT * 16, 1.0f, 0, dA);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  skinny_reduce_kernel<<<(N * r + kThreads - 1) / kThreads, kThreads, 0, stream>>>(
      pb, p.splits_b, N, r, RT * 16, s, 1, dB);
  return hipGetLastError();
}

// dst += src over n bf16 elements (float32 add, one nearest-even rounding).
__global__ __launch_bounds__(256) void add_bf16_kernel(int64_t n, uint16_t* __restrict__ dst,
                                                       const uint16_t* __restrict__ src) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i + 8 <= n) {
    const uint4 a = *reinterpret_cast<const uint4*>(dst + i);
    const uint4 b = *reinterpret_cast<const uint4*>(src + i);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = pack_bf16x2(__uint_as_float(aw[q] << 16) + __uint_as_float(bw[q] << 16),
                         __uint_as_float(aw[q] & 0xFFFF0000u) + __uint_as_float(bw[q] & 0xFFFF0000u));
    *reinterpret_cast<uint4*>(dst + i) = uint4{o[0], o[1], o[2], o[3]};
  } else {
    for (int64_t k = i; k < n; ++k) dst[k] = to_bf16(bf16_to_f32(dst[k]) + bf16_to_f32(src[k]));
  }
}

hipError_t launch_u(int T, int K, int r, const uint16_t* x, const uint16_t* A, uint16_t* u,
                    hipStream_t stream) {
#define LNF4_U(RT_) \
  lora_u_kernel<RT_><<<(T + 63) / 64, kThreads, 0, stream>>>(T, K, r, x, A, u); \
  return hipGetLastError()
  switch (generic_rank_tiles(r)) {
    case 1: LNF4_U(1);
    case 2: LNF4_U(2);
    case 3: LNF4_U(3);
    case 4: LNF4_U(4);
    case 5: LNF4_U(5);
    case 6: LNF4_U(6);
    case 7: LNF4_U(7);
    case 8: LNF4_U(8);
    case 12: LNF4_U(12);
    case 16: LNF4_U(16);
    default: return hipErrorInvalidValue;
  }
#undef LNF4_U
}

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// Token splits for a skinny reduction over `cols` columns: enough workgroups
// to fill the chip a few times over, each split a multiple of 64 tokens.
int choose_splits(int64_t T, int64_t cols) {
  const int64_t col_blocks = (cols + 127) / 128;
  int64_t want = (1024 + col_blocks - 1) / col_blocks;
  const int64_t max_splits = (T + 63) / 64;
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  // make every split a whole number of 64-token steps
  int64_t chunk = (T + want - 1) / want;
  chunk = ((chunk + 63) / 64) * 64;
  return static_cast<int>((T + chunk - 1) / chunk);
}

}  // namespace

BwdPlan plan_bwd(int64_t T, int64_t K, int64_t N, int r, bool allow_dq) {
  BwdPlan p{};
  p.fast = lora_dx_supported(r) && lora_skinny_supported(r) && fits_buffer(T, K, N);
  const int64_t rs = p.fast ? r : generic_rank_tiles(r) * 16;
  p.rp = static_cast<int>(((r + 31) / 32) * 32);
  if (p.fast) {
    p.splits_a = p.splits_b = skinny_splits(T, K, N);
  } else {
    p.splits_a = choose_splits(T, K);
    p.splits_b = choose_splits(T, N);
  }
  size_t off = 0;
  p.off_g = off;
  off = align256(off + static_cast<size_t>(T) * r * 2);
  p.off_u = off;
  off = align256(off + static_cast<size_t>(T) * r * 2);
  p.off_pa = off;
  off = align256(off + static_cast<size_t>(p.splits_a) * K * rs * 4);
  p.off_pb = off;
  off = align256(off + static_cast<size_t>(p.splits_b) * N * rs * 4);
  p.splitk = p.fast && lora_dx_splitk_supported(T, r);
  p.splits_x = 0;
  p.off_px = p.off_pg = off;
  if (p.splitk) {
    const DxSplitPlan d = plan_dx_splitk(T, K, N, r);
    p.splits_x = d.splits;
    off = align256(off + d.part_x_bytes);
    p.off_pg = off;
    off = align256(off + d.part_g_bytes);
  } else if (p.fast) {  // tiled dX, split over d_out when its tile grid is small
    const DxTiledSplit d = dx_tiled_split(T, K, N, r);
    if (d.splits > 1) {
      p.splits_x = d.splits;
      off = align256(off + static_cast<size_t>(d.splits) * T * K * 4);
      p.off_pg = off;
      off = align256(off + static_cast<size_t>(d.splits) * T * r * 4);
    } else if (!weight_staging() && dx_rw_supported(T, K, N, r)) {
      p.rwx = true;
      p.off_w = off;
      off = align256(off + dx_rw_bytes(K, N));
    } else if (allow_dq && dx_dq(T, K, N, r)) {
      p.dqx = true;
      p.off_w = off;
      off = align256(off + static_cast<size_t>(N) * K * 2);
    }
    // rank > 16 from 4096 tokens, unsplit, packed weight: G from a G pass
    p.gpass = p.splits_x <= 1 && !p.rwx && !p.dqx && r > 16 && T >= 4096 && N % 256 == 0;
  }
  p.bytes = off;
  return p;
}

hipError_t launch_lora_bwd(int T, int K, int N, int r, float s, const uint16_t* x,
                           const uint16_t* dy, const uint8_t* codes, const float* absmax,
                           const uint16_t* A, const uint16_t* B, const uint16_t* u_saved,
                           uint16_t* dx, uint16_t* dA, uint16_t* dB, void* workspace,
                           const BwdPlan& plan, hipStream_t stream, const SkinnyAdamW* adam) {
#define LNF4_BWD(RT_)                                                                              \
  return launch_bwd_rt<RT_>(T, K, N, r, s, x, dy, codes, absmax, A, B, u_saved, dx, dA, dB,        \
                            workspace, plan, stream, adam)
  switch (generic_rank_tiles(r)) {
    case 1: LNF4_BWD(1);
    case 2: LNF4_BWD(2);
    case 3: LNF4_BWD(3);
    case 4: LNF4_BWD(4);
    case 5: LNF4_BWD(5);
    case 6: LNF4_BWD(6);
    case 7: LNF4_BWD(7);
    case 8: LNF4_BWD(8);
    case 12: LNF4_BWD(12);
    case 16: LNF4_BWD(16);
    default: return hipErrorInvalidValue;
  }
#undef LNF4_BWD
}

// The rank-r gradients alone, from G and U the caller holds: the backward's own
// rank-r step (one launch and one reduce for r % 8 == 0, r <= 64; the generic
// split-T kernels otherwise), its partials at the start of the workspace.
GradPlan plan_grad_ab(int64_t T, int64_t K, int64_t N, int r) {
  GradPlan p{};
  p.fast = lora_skinny_supported(r) && fits_buffer(T, K, N);
  p.rs = p.fast ? r : generic_rank_tiles(r) * 16;
  if (p.fast) {
    p.splits_a = p.splits_b = skinny_splits(T, K, N);
  } else {
    p.splits_a = choose_splits(T, K);
    p.splits_b = choose_splits(T, N);
  }
  p.off_pb = align256(static_cast<size_t>(p.splits_a) * K * p.rs * 4);
  p.bytes = p.off_pb + align256(static_cast<size_t>(p.splits_b) * N * p.rs * 4);
  return p;
}

namespace {
template <int RT>
hipError_t launch_grad_ab_rt(int T, int K, int N, int r, float s, const uint16_t* x, const uint16_t* g,
                             const uint16_t* dy, const uint16_t* u, uint16_t* dA, uint16_t* dB, float* pa,
                             float* pb, const GradPlan& p, hipStream_t stream) {
  const int tca = (T + p.splits_a - 1) / p.splits_a;
  const int tcb = (T + p.splits_b - 1) / p.splits_b;
  skinny_tn_kernel<RT><<<dim3((K + 127) / 128, p.splits_a), kThreads, 0, stream>>>(T, K, r, tca, x, g, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  skinny_tn_kernel<RT><<<dim3((N + 127) / 128, p.splits_b), kThreads, 0, stream>>>(T, N, r, tcb, dy, u, pb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  skinny_reduce_kernel<<<(K * r + kThreads - 1) / kThreads, kThreads, 0, stream>>>(pa, p.splits_a, K, r, RT * 16,
                                                                                    1.0f, 0, dA);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  skinny_reduce_kernel<<<(N * r + kThreads - 1) / kThreads, kThreads, 0, stream>>>(pb, p.splits_b, N, r, RT * 16,
                                                                                    s, 1, dB);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_grad_ab(int T, int K, int N, int r, float s, const uint16_t* x, const uint16_t* g,
                          const uint16_t* dy, const uint16_t* u, uint16_t* dA, uint16_t* dB, void* workspace,
                          const GradPlan& p, hipStream_t stream) {
  float* pa = static_cast<float*>(workspace);
  float* pb = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.off_pb);
  if (p.fast) {
    DaOut da{};
    da.p[0] = dA;
    da.gw = r;
    return launch_lora_skinny(T, K, N, r, r, r, s, x, g, dy, u, pa, pb, p.splits_a, da, dB, stream);
  }
#define LNF4_GRAD(RT_) return launch_grad_ab_rt<RT_>(T, K, N, r, s, x, g, dy, u, dA, dB, pa, pb, p, stream)
  switch (generic_rank_tiles(r)) {
    case 1: LNF4_GRAD(1);
    case 2: LNF4_GRAD(2);
    case 3: LNF4_GRAD(3);
    case 4: LNF4_GRAD(4);
    case 5: LNF4_GRAD(5);
    case 6: LNF4_GRAD(6);
    case 7: LNF4_GRAD(7);
    case 8: LNF4_GRAD(8);
    case 12: LNF4_GRAD(12);
    case 16: LNF4_GRAD(16);
    default: return hipErrorInvalidValue;
  }
#undef LNF4_GRAD
}

// The fused dX takes G from a G pass (launch_gpass) at rank > 16 from 4096 tokens,
// when every d_out is a multiple of 256 and weights are not staged (measured on
// MI355X, Llama-3-8B q/k/v at r = 64: the in-loop G is 25 % more MFMA work in
// every one of the 16 column tiles of the tiled dX).
bool dx_gpass(int64_t T, int n, const int* N, int r) {
  if (n < 2 || r <= 16 || T < 4096 || weight_staging()) return false;
  for (int g = 0; g < n; ++g)
    if (N[g] % 256 != 0) return false;
  return true;
}

BwdMultiPlan plan_bwd_multi(int64_t T, int64_t K, int n, const int* N, int r) {
  BwdMultiPlan p{};
  p.n = n;
  p.R = n * r;
  bool fused = n > 1 && lora_dx_multi_supported(n, N, r) && lora_skinny_supported(r) &&
               !lora_dx_splitk_supported(T, r) &&
               static_cast<int64_t>(T) * p.R * 2 < (int64_t(1) << 31);
  for (int g = 0; g < n && fused; ++g) fused = fits_buffer(T, K, N[g]);
  p.fused = fused;
  size_t off = 0;
  if (fused) {
    p.off_g = off;
    off = align256(off + static_cast<size_t>(T) * p.R * 2);
    p.off_u = off;
    off = align256(off + static_cast<size_t>(n) * T * r * 2);
    // n r <= 64: one launch for every dA (one pass over x, rank n r) and every dB;
    // n r <= 192: one launch for every dA (the wide-rank kernel), one for every dB;
    // wider: one launch per projection for its dA and dB (G read as a column slice
    // of the side-by-side array). dB partials of the projections lie side by side.
    const bool one_pass = lora_skinny_supported(p.R);
    const bool wide = !one_pass && lora_skinny_wide_supported(p.R);
    const auto blocks = [](int64_t c) { return (c + 255) / 256; };
    int64_t nb = 0, nsum = 0;
    for (int g = 0; g < n; ++g) {
      nb += blocks(N[g]);
      nsum += N[g];
    }
    size_t pa = 0, pb = 0;
    if (one_pass) {
      p.splits_a = p.splits_b[0] = skinny_splits_blocks(T, blocks(K) + nb);
      pa = static_cast<size_t>(p.splits_a) * K * p.R * 4;
      pb = static_cast<size_t>(p.splits_a) * nsum * r * 4;
    } else if (wide) {
      p.splits_a = skinny_splits(T, K, 0);
      p.splits_b[0] = skinny_splits_blocks(T, nb);
      pa = static_cast<size_t>(p.splits_a) * K * p.R * 4;
      pb = static_cast<size_t>(p.splits_b[0]) * nsum * r * 4;
    } else {
      for (int g = 0; g < n; ++g) {
        const int sp = skinny_splits(T, K, N[g]);
        if (g == 0) p.splits_a = sp;
        else p.splits_b[g] = sp;
        pa = std::max(pa, static_cast<size_t>(sp) * K * r * 4);
        pb = std::max(pb, static_cast<size_t>(sp) * N[g] * r * 4);
      }
    }
    p.off_pa = off;
    off = align256(off + pa);
    p.off_pb = off;
    off = align256(off + pb);
    p.dq = true;
    for (int g = 0; g < n; ++g) p.dq = p.dq && dx_dq(T, K, N[g], r);
    for (int g = 0; g < n && p.dq; ++g) {
      p.off_w[g] = off;
      off = align256(off + static_cast<size_t>(N[g]) * K * 2);
    }
  } else {
    size_t single = 0;
    for (int g = 0; g < n; ++g) single = std::max(single, plan_bwd(T, K, N[g], r).bytes);
    p.off_single = off;
    off = align256(off + single);
    p.off_dxt = off;
    if (n > 1) off = align256(off + static_cast<size_t>(T) * K * 2);
  }
  p.bytes = off;
  return p;
}

hipError_t launch_lora_bwd_multi(int T, int K, int n, const int* N, int r, float s, const uint16_t* x,
                                 const uint16_t* const* dy, const uint8_t* const* codes,
                                 const float* const* absmax, const uint16_t* const* A,
                                 const uint16_t* const* B, const uint16_t* const* u_saved, uint16_t* dx,
                                 uint16_t* const* dA, uint16_t* const* dB, void* workspace,
                                 const BwdMultiPlan& p, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  hipError_t e = hipSuccess;
  if (!p.fused) {  // one backward per projection; dX accumulated
    uint16_t* dxt = reinterpret_cast<uint16_t*>(ws + p.off_dxt);
    for (int g = 0; g < n; ++g) {
      const uint16_t* u = u_saved == nullptr ? nullptr : u_saved[g];
      uint16_t* dxg = (dx != nullptr && g > 0) ? dxt : dx;
      e = launch_lora_bwd(T, K, N[g], r, s, x, dy[g], codes[g], absmax[g], A[g], B[g], u, dxg, dA[g], dB[g],
                          ws + p.off_single, plan_bwd(T, K, N[g], r), stream);
      if (e != hipSuccess) return e;
      if (dxg == dxt) {
        const int64_t total = static_cast<int64_t>(T) * K;
        add_bf16_kernel<<<static_cast<unsigned>((total / 8 + 255) / 256 + 1), 256, 0, stream>>>(total, dx, dxt);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
    }
    return hipSuccess;
  }
  DxTable tab{};
  tab.n = n;
  int steps = 0;
  for (int g = 0; g < n; ++g) {
    steps += N[g] / 64;
    tab.step_end[g] = steps;
    tab.N[g] = N[g];
    tab.dy[g] = dy[g];
    tab.codes[g] = codes[g];
    tab.absmax[g] = absmax[g];
    tab.A[g] = A[g];
    tab.B[g] = B[g];
    if (p.dq) {
      uint16_t* w = reinterpret_cast<uint16_t*>(ws + p.off_w[g]);
      if ((e = launch_nf4_dequantize(codes[g], absmax[g], N[g], K, true, w, stream)) != hipSuccess) return e;
      tab.wdq[g] = w;
    }
  }
  uint16_t* G = reinterpret_cast<uint16_t*>(ws + p.off_g);
  // rank > 16 from 4096 tokens (every d_out a multiple of 256): G = s dY_g B_g^T of
  // each projection in a pass of its own over dY_g (the U pass's kernel), so the
  // dX tiles skip the rank-wide MFMAs that every column tile would repeat
  const bool gpass = dx_gpass(T, n, N, r);
  if (gpass)
    for (int g = 0; g < n; ++g)
      if ((e = launch_gpass(T, N[g], r, s, dy[g], B[g], G + g * r, n * r, stream)) != hipSuccess) return e;
  if ((dx != nullptr || !gpass) && (e = launch_lora_dx_table(T, K, r, s, tab, dx, G, stream, gpass)) != hipSuccess)
    return e;
  const uint16_t* uu[kMaxProj];
  for (int g = 0; g < n; ++g) {
    uu[g] = u_saved == nullptr ? nullptr : u_saved[g];
    if (uu[g] == nullptr) {
      uint16_t* u = reinterpret_cast<uint16_t*>(ws + p.off_u) + static_cast<size_t>(g) * T * r;
      if ((e = launch_u(T, K, r, x, A[g], u, stream)) != hipSuccess) return e;
      uu[g] = u;
    }
  }
  float* pa = reinterpret_cast<float*>(ws + p.off_pa);
  float* pb = reinterpret_cast<float*>(ws + p.off_pb);
  DaOut da{};
  da.gw = r;
  const bool one_pass = lora_skinny_supported(p.R);
  if (one_pass || lora_skinny_wide_supported(p.R)) {
    for (int g = 0; g < n; ++g) da.p[g] = dA[g];
    // dA of every projection from one pass over x (G side by side); n r <= 64: in the
    // same launch as every dB, else (the wide-rank kernel) alone, then every dB in one
    // launch (each projection's partials at its own offset)
    SkinnyJob jobs[kMaxSkinnyJobs];
    int nj = 0;
    jobs[nj++] = SkinnyJob{x, G, pa, nullptr, K, p.R, p.R, true};
    if (!one_pass) {
      if ((e = launch_skinny_jobs(T, 1, jobs, p.splits_a, s, da, stream)) != hipSuccess) return e;
      nj = 0;
    }
    float* pbg = pb;
    const int sb = one_pass ? p.splits_a : p.splits_b[0];
    for (int g = 0; g < n; ++g) {
      jobs[nj++] = SkinnyJob{dy[g], uu[g], pbg, dB[g], N[g], r, r, false};
      pbg += static_cast<size_t>(sb) * r * N[g];
    }
    return launch_skinny_jobs(T, nj, jobs, sb, s, da, stream);
  }
  for (int g = 0; g < n && e == hipSuccess; ++g) {  // one pass per projection, G column slice g
    da.p[0] = dA[g];
    e = launch_lora_skinny(T, K, N[g], r, r, p.R, s, x, G + static_cast<size_t>(g) * r, dy[g], uu[g], pa, pb,
                           g == 0 ? p.splits_a : p.splits_b[g], da, dB[g], stream);
  }
  return e;
}

}  // namespace lnf4
