// Fused NF4-LoRA linear, forward, for up to 128 tokens: weight-streaming with the
// reduction split across workgroups (gfx950).
//
// With few tokens the forward is bound by reading the packed weight (0.5625 bytes
// per element) and by dequantizing it, not by the matrix products. The chain the
// kernel-fusion section of "Unsloth acceleration principles: CUDA kernel fusion
// and memory optimization" describes (base linear, LoRA down-projection, LoRA
// up-projection, add) runs in two launches:
//   * lora_fwd_splitk_kernel: workgroup (64 weight rows, one d_in chunk of the
//     split), four waves of 16 weight rows each. The waves share the x chunk of
//     each 128-element reduction step, staged in LDS by direct-to-LDS loads
//     (XOR-swizzled for conflict-free fragment reads; a ring of two to four
//     buffers, so up to three steps are in flight; one barrier per step). Each
//     lane loads 16 bytes of codes (32 consecutive
//     reduction elements of one weight row) and dequantizes them straight into
//     four v_mfma_f32_16x16x32_bf16 B fragments, one step ahead of their use: the
//     weight never passes through LDS. Codes run three steps ahead. fp32 partial
//     products go to a workspace [split][T][d_out].
//     U = x A: the grid has one more workgroup per (U split, 16-wide rank block),
//     which stages the same x chunks and that block's 16 columns of A (read back
//     transposed) and accumulates its part of U; its four waves take one of the
//     four MFMA k-slices of each step each and sum their parts in LDS. Main
//     workgroups carry no U work, so they stay uniform. fp32 partial U goes to the
//     workspace [split][T][r].
//   * lora_fwd_splitk_reduce: sums the partials over the splits in a fixed order
//     (deterministic), rounds s U to bf16 as the tiled kernels do, adds
//     bf16(s U) B and stores bf16 y (and bf16 U for the backward).
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int kKThreads = 256;            // 4 waves x 16 weight rows
constexpr int kRowsPerWg = 64;
constexpr int kStep = 128;                // reduction elements per step
constexpr uint32_t kXOut = 0x7FFFFFF0u;   // a per-lane offset past every buffer range: reads zeros
constexpr int kMaxSplits = 16;            // bounds the partial traffic of narrow outputs
// Workgroups of lora_fwd_splitk_kernel<TB> resident per CU (registers and LDS, as
// the compiler reports them for gfx950): the split count fills one resident round.
constexpr int kResident[4] = {4, 4, 3, 2};  // TB = 1, 2, 4, 8

// TB: 16-token blocks (T <= 16 TB).
template <int TB>
struct SplitCfg {
  static constexpr int kXBytes = 16 * TB * kStep * 2;  // one x stage
  static constexpr int kABytes = kStep * 16 * 2;       // one A stage: 16 rank columns
  static constexpr int kStage = kXBytes + kABytes;
  // ring depth: four stages for one token block (small), else two, which keeps
  // several workgroups per CU
  static constexpr int kNB = TB == 1 ? 4 : 2;
  static constexpr int kURed = 4 * TB * 4 * 64 * 4;    // U parts of the four waves
  static constexpr int kBytes = kNB * kStage > kURed ? kNB * kStage : kURed;
  // Loads each wave issues per step: TB x copies (+ one A copy in U workgroups),
  // two code / scale loads (main workgroups only).
  static constexpr int kMainWait = kNB == 2 ? 2 : TB + 2;  // at the top of a step
  static constexpr int kUWait = (kNB - 2) * (TB + 1);
};

// Workgroups 0 .. ncb * splits - 1: (column block, split) of the base product;
// the next splits * ceil(r / 16): (split, rank block) of U.
template <int TB>
__global__ __launch_bounds__(kKThreads) void lora_fwd_splitk_kernel(
    int T, int K, int N, int r, int steps_per, int ncb, int splits, const uint16_t* __restrict__ x,
    const uint8_t* __restrict__ codes, const float* __restrict__ absmax, const uint16_t* __restrict__ A,
    float* __restrict__ part, float* __restrict__ upart) {
  using C = SplitCfg<TB>;
  // level pairs of every code byte, (q[b & 15], q[b >> 4]) at 8 b: first in LDS, so
  // a table address needs no base
  __shared__ __align__(1024) float lut[512];
  __shared__ __align__(16) unsigned char smem[C::kBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int nmain = ncb * splits;
  const bool urole = static_cast<int>(blockIdx.x) >= nmain;  // workgroup-uniform
  const int rj = (r + 15) / 16;
  const int ub = blockIdx.x - nmain;
  const int sp = urole ? ub / rj : blockIdx.x / ncb;
  const int cb = urole ? 0 : blockIdx.x % ncb;
  const int jb = urole ? ub % rj : 0;
  const int n0 = cb * kRowsPerWg;
  const int K2 = K / 2, KB = K / 64;
  const int nsteps = (K + kStep - 1) / kStep;
  const int st_begin = sp * steps_per;
  const int n_my = min(nsteps - st_begin, steps_per);  // >= 1 (the plan leaves no split empty)

  for (int e = tid; e < 256; e += kKThreads) {
    lut[2 * e] = nf4_level_reg(e & 15);
    lut[2 * e + 1] = nf4_level_reg(e >> 4);
  }

  const int rows_w = min(N - n0, kRowsPerWg);
  const auto rs_c = make_rsrc(codes + static_cast<size_t>(n0) * K2, static_cast<uint32_t>(rows_w) * K2);
  const auto rs_s = make_rsrc(absmax + static_cast<size_t>(n0) * KB, static_cast<uint32_t>(rows_w) * KB * 4);
  const auto rs_x = make_rsrc(x, static_cast<uint32_t>(T) * K * 2);
  const auto rs_a = make_rsrc(A, static_cast<uint32_t>(K) * r * 2);

  // Lane (l16, g) of wave w owns reduction elements 32 g .. 32 g + 31 of every
  // step: codes of weight row n0 + 16 w + l16, x of token rows 16 tb + l16. MFMA
  // k-slice q of a step uses elements 32 g + 8 q .. +7, in both operands.
  const int wrow = 16 * wave + l16;
  const uint32_t cvoff = static_cast<uint32_t>(wrow) * K2 + 16 * g;
  const uint32_t svoff = (static_cast<uint32_t>(wrow) * KB + (g >> 1)) * 4;
  // x stage: [16 TB rows][16 pieces of 8 elements], piece p of row t stored at
  // physical piece p ^ (t & 15). Copy i fills rows 4 i .. 4 i + 3 (1 KB); wave w
  // issues copies w, w + 4, ...; lane L lands on row 4 i + (L >> 4), physical
  // piece L & 15, and loads the logical piece stored there.
  uint32_t xvoff[TB];
  int xpiece[TB];
#pragma unroll
  for (int c = 0; c < TB; ++c) {
    const int t = 4 * (wave + 4 * c) + (lane >> 4);
    xpiece[c] = (lane & 15) ^ (t & 15);
    xvoff[c] = static_cast<uint32_t>(t) * K * 2 + 16 * xpiece[c];
  }
  const int x_lane = l16 * kStep * 2;
  // A stage (U workgroups): [kStep rows k][16 rank columns 16 jb ..] bf16, 32 bytes
  // a row, four 1 KB copies (one per wave); lane L of copy w covers row 32 w +
  // (L >> 1), half L & 1. Columns past r read zeros.
  const int arow = 32 * wave + (lane >> 1), ahalf = lane & 1;
  const bool acol_ok = 16 * jb + 8 * ahalf < r;
  // transposed A fragment: rows 32 g + 8 q + 4 h + (l16 >> 2) of the step, rank
  // columns 4 (l16 & 3) .. +3 of the block; lane l16 receives rank column l16
  const int a_lane = (32 * g + (l16 >> 2)) * 32 + 8 * (l16 & 3);

  auto buf = [&](int i) { return smem + (i % C::kNB) * C::kStage; };

  auto load_stage = [&](int i, unsigned char* st) {
    const int c0 = (st_begin + i) * kStep;
#pragma unroll
    for (int c = 0; c < TB; ++c) {
      const uint32_t off = c0 + 8 * xpiece[c] < K ? xvoff[c] + static_cast<uint32_t>(c0) * 2 : kXOut;
      buf_load16_lds(rs_x, st + (wave_u + 4 * c) * 1024, off, 0);
    }
    if (urole) {
      // rows past d_in fall outside the range of A and read zeros
      const uint32_t off = acol_ok ? static_cast<uint32_t>(c0 + arow) * r * 2 + 32 * jb + 16 * ahalf : kXOut;
      buf_load16_lds(rs_a, st + C::kXBytes + wave_u * 1024, off, 0);
    }
  };

  uint4 creg[4];
  float sreg[4];
  auto load_codes = [&](int i, int slot) {
    if (urole) return;
    const uint32_t c0 = static_cast<uint32_t>(st_begin + i) * kStep;
    creg[slot] = buf_load16(rs_c, cvoff + c0 / 2, 0);
    sreg[slot] = __uint_as_float(buf_load4(rs_s, svoff + c0 / 64 * 4, 0));
  };

  const unsigned char* lutb = reinterpret_cast<const unsigned char*>(lut);
  auto dequant8 = [&](uint32_t w, float a) {
    // each code byte (the lower element in its low nibble) addresses its pair of
    // levels: one 64-bit LDS read per two elements
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t ad = (j == 0 ? (w << 3) : (w >> (8 * j - 3))) & 0x7F8u;
      const float2 p = *reinterpret_cast<const float2*>(lutb + ad);
      v[2 * j] = p.x;
      v[2 * j + 1] = p.y;
    }
    uint4 o;
    o.x = pack_bf16x2(v[0] * a, v[1] * a);
    o.y = pack_bf16x2(v[2] * a, v[3] * a);
    o.z = pack_bf16x2(v[4] * a, v[5] * a);
    o.w = pack_bf16x2(v[6] * a, v[7] * a);
    return o;
  };
  // B fragments of step i from the codes in `slot`; zero for the half of a
  // half-filled last step that lies past d_in
  auto dequant_step = [&](int i, int slot, uint4* wf) {
    const bool valid = (st_begin + i) * kStep + 32 * g < K;
    const uint32_t cw[4] = {creg[slot].x, creg[slot].y, creg[slot].z, creg[slot].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      wf[q] = dequant8(cw[q], sreg[slot]);
      if (!valid) wf[q] = uint4{0u, 0u, 0u, 0u};
    }
  };

  f32x4_t acc[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // prologue, in issue order: stages 0 .. kNB - 2, codes of steps 0, 1, 2; then
  // the B fragments of step 0
  uint4 wf[2][4];
#pragma unroll
  for (int j = 0; j < C::kNB - 1; ++j) load_stage(j, buf(j));
  load_codes(0, 0);
  load_codes(1, 1);
  load_codes(2, 2);
  if (urole) wait_vmem_upto<C::kUWait>();  // stage 0 landed
  else wait_vmem_upto<2>();                // stages 0 .. kNB - 2, codes 0 and 1 landed
  __syncthreads();                         // level table visible
  if (!urole) dequant_step(0, 0, wf[0]);

  // Step i issues the stage of step i + kNB - 1 (into the buffer of step i - 1,
  // which every wave finished before this step's barrier), then the codes of step
  // i + 3. Loads retire in issue order, so at the top of step i the stage of step
  // i and the codes of step i + 1 have landed once at most kMainWait (main) or
  // kUWait (U) loads are outstanding. The loop is unrolled by four so the code
  // slots are compile-time.
  auto step = [&](int i, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;  // i % 4
    constexpr int b = slot & 1;                    // B-fragment set of step i
    const unsigned char* const cur = buf(i);
    if (urole) wait_vmem_upto<C::kUWait>();
    else wait_vmem_upto<C::kMainWait>();
    __syncthreads();
    load_stage(i + C::kNB - 1, buf(i + C::kNB - 1));
    if (urole) {
      // U part over k-slice q = w of this step
      const unsigned char* p = cur + C::kXBytes + a_lane + 8 * wave_u * 32;
      const uint2 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(p));
      const uint2 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(p + 4 * 32));
      const uint4 af = uint4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const uint4 xv = *reinterpret_cast<const uint4*>(cur + tb * 16 * kStep * 2 + x_lane +
                                                         (((4 * g + wave_u) ^ l16) << 4));
        acc[tb] = mfma16(xv, af, acc[tb]);
      }
      return;
    }
    load_codes(i + 3, (slot + 3) & 3);
    if (i + 1 < n_my) dequant_step(i + 1, (slot + 1) & 3, wf[b ^ 1]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const uint4 xv = *reinterpret_cast<const uint4*>(cur + tb * 16 * kStep * 2 + x_lane +
                                                         (((4 * g + q) ^ l16) << 4));
        acc[tb] = mfma16(xv, wf[b][q], acc[tb]);
      }
    }
  };
  for (int i = 0; i < n_my; i += 4) {
    step(i, std::integral_constant<int, 0>{});
    if (i + 1 < n_my) step(i + 1, std::integral_constant<int, 1>{});
    if (i + 2 < n_my) step(i + 2, std::integral_constant<int, 2>{});
    if (i + 3 < n_my) step(i + 3, std::integral_constant<int, 3>{});
  }
  // run-ahead loads (direct-to-LDS ones included) must land before LDS is reused
  wait_vmem();

  // C layout: lane (l16, g) holds column l16, rows 4 g + e of each 16 x 16 block
  if (!urole) {
    float* dst = part + static_cast<size_t>(sp) * T * N;
    const int n = n0 + wrow;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * tb + 4 * g + e;
        if (t < T && n < N) dst[static_cast<size_t>(t) * N + n] = acc[tb][e];
      }
    return;
  }
  // U: the four waves hold parts over disjoint k-slices; sum them in LDS
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [wave][tb][e][64]
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[((wave * TB + tb) * 4 + e) * 64 + lane] = acc[tb][e];
  __syncthreads();
  float* udst = upart + static_cast<size_t>(sp) * T * r;
  constexpr int kPer = TB * 4 * 64;
  for (int idx = tid; idx < kPer; idx += kKThreads) {
    const float v = red[idx] + red[kPer + idx] + red[2 * kPer + idx] + red[3 * kPer + idx];
    const int ln = idx & 63, e = (idx >> 6) & 3, tb = idx >> 8;
    const int t = 16 * tb + 4 * (ln >> 4) + e, j = 16 * jb + (ln & 15);
    if (t < T && j < r) udst[static_cast<size_t>(t) * r + j] = v;
  }
}

// y = bf16(sum_sp part[sp] + bf16(s sum_sp upart[sp]) B); u_save = bf16(sum_sp upart).
// Workgroup: 8 token rows x 128 output columns, 256 threads (4 columns of one row
// each). The few rows keep the U sums that every column block repeats small. The
// loads of every split's partial, of the U parts and of B are all issued before
// any is waited on: the kernel costs about two memory round trips.
constexpr int kRCols = 128, kRRows = 8, kRThreads = 256;

__global__ __launch_bounds__(kRThreads) void lora_fwd_splitk_reduce(
    int T, int N, int r, int S, float s, const float* __restrict__ part, const float* __restrict__ upart,
    const uint16_t* __restrict__ B, uint16_t* __restrict__ y, uint16_t* __restrict__ u_save) {
  __shared__ float su[kRRows][64];                  // bf16(s U) of the rows, as float
  __shared__ __align__(16) uint16_t bs[64][kRCols];  // B rows 0..r-1 of the column block
  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * kRCols, t0 = blockIdx.y * kRRows;
  const int tl = tid >> 5, c4 = (tid & 31) * 4;
  const int t = t0 + tl, n = n0 + c4;
  const bool mine = t < T && n < N;  // d_out % 8 == 0: a 4-column group is all in or all out
  float4 w[kMaxSplits];
#pragma unroll
  for (int q = 0; q < kMaxSplits; ++q)
    w[q] = mine && q < S ? *reinterpret_cast<const float4*>(part + (static_cast<size_t>(q) * T + t) * N + n)
                         : float4{0.f, 0.f, 0.f, 0.f};
  float uw[2][kMaxSplits];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = tid + kRThreads * h, ur = e >> 6, j = e & 63, ut = t0 + ur;
    const bool ok = j < r && ut < T;
#pragma unroll
    for (int q = 0; q < kMaxSplits; ++q)
      uw[h][q] = ok && q < S ? upart[(static_cast<size_t>(q) * T + ut) * r + j] : 0.f;
  }
  uint4 bv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = tid + kRThreads * k, j = e >> 4, c = (e & 15) * 8;
    bv[k] = j < r && n0 + c < N ? *reinterpret_cast<const uint4*>(B + static_cast<size_t>(j) * N + n0 + c)
                                : uint4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = tid + kRThreads * k, j = e >> 4, c = (e & 15) * 8;
    if (j < r) *reinterpret_cast<uint4*>(&bs[j][c]) = bv[k];
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = tid + kRThreads * h, ur = e >> 6, j = e & 63, ut = t0 + ur;
    float uv = 0.f;
#pragma unroll
    for (int q = 0; q < kMaxSplits; ++q) uv += uw[h][q];
    su[ur][j] = __uint_as_float(static_cast<uint32_t>(to_bf16(s * uv)) << 16);
    if (u_save != nullptr && blockIdx.x == 0 && j < r && ut < T)
      u_save[static_cast<size_t>(ut) * r + j] = to_bf16(uv);
  }
  __syncthreads();
  if (!mine) return;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < kMaxSplits; ++q) v[0] += w[q].x, v[1] += w[q].y, v[2] += w[q].z, v[3] += w[q].w;
  for (int j = 0; j < r; ++j) {
    const float u = su[tl][j];
    const uint2 b2 = *reinterpret_cast<const uint2*>(&bs[j][c4]);
    v[0] = fmaf(u, __uint_as_float(b2.x << 16), v[0]);
    v[1] = fmaf(u, __uint_as_float(b2.x & 0xFFFF0000u), v[1]);
    v[2] = fmaf(u, __uint_as_float(b2.y << 16), v[2]);
    v[3] = fmaf(u, __uint_as_float(b2.y & 0xFFFF0000u), v[3]);
  }
  uint2 o;
  o.x = pack_bf16x2(v[0], v[1]);
  o.y = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2*>(y + static_cast<size_t>(t) * N + n) = o;
}

template <int TB>
hipError_t launch_splitk_t(int T, int K, int N, int r, const SplitKPlan& p, const uint16_t* x,
                           const uint8_t* codes, const float* absmax, const uint16_t* A, float* part,
                           float* upart, hipStream_t stream) {
  const int blocks = (p.ncb + (r + 15) / 16) * p.splits;
  lora_fwd_splitk_kernel<TB><<<blocks, kKThreads, 0, stream>>>(T, K, N, r, p.steps_per, p.ncb, p.splits, x,
                                                              codes, absmax, A, part, upart);
  return hipGetLastError();
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

}  // namespace

bool lora_fwd_splitk_supported(int64_t T, int r) { return T >= 1 && T <= 128 && r % 8 == 0 && r <= 64; }

SplitKPlan plan_fwd_splitk(int T, int K, int N, int r) {
  SplitKPlan p{};
  p.ncb = (N + kRowsPerWg - 1) / kRowsPerWg;
  const int nsteps = (K + kStep - 1) / kStep;
  // Splits: every split adds ncb + ceil(r / 16) workgroups; as many as one
  // resident round holds, at most kMaxSplits.
  const int per_split = p.ncb + (r + 15) / 16;
  const int tbi = T <= 16 ? 0 : (T <= 32 ? 1 : (T <= 64 ? 2 : 3));
  int S = 256 * kResident[tbi] / per_split;
  S = S < 1 ? 1 : (S > kMaxSplits ? kMaxSplits : S);
  S = S > nsteps ? nsteps : S;
  p.steps_per = (nsteps + S - 1) / S;
  p.splits = (nsteps + p.steps_per - 1) / p.steps_per;  // every split non-empty
  p.part_bytes = align256(static_cast<size_t>(p.splits) * T * N * 4);
  p.bytes = p.part_bytes + align256(static_cast<size_t>(p.splits) * T * r * 4);
  return p;
}

hipError_t launch_lora_fwd_splitk(int T, int K, int N, int r, float s, const uint16_t* x,
                                  const uint8_t* codes, const float* absmax, const uint16_t* A,
                                  const uint16_t* B, uint16_t* y, uint16_t* u_save, void* workspace,
                                  hipStream_t stream) {
  const SplitKPlan p = plan_fwd_splitk(T, K, N, r);
  float* part = static_cast<float*>(workspace);
  float* upart = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + p.part_bytes);
  hipError_t e;
  if (T <= 16) e = launch_splitk_t<1>(T, K, N, r, p, x, codes, absmax, A, part, upart, stream);
  else if (T <= 32) e = launch_splitk_t<2>(T, K, N, r, p, x, codes, absmax, A, part, upart, stream);
  else if (T <= 64) e = launch_splitk_t<4>(T, K, N, r, p, x, codes, absmax, A, part, upart, stream);
  else e = launch_splitk_t<8>(T, K, N, r, p, x, codes, absmax, A, part, upart, stream);
  if (e != hipSuccess) return e;
  return launch_fwd_splitk_reduce(T, N, r, p.splits, s, part, upart, B, y, u_save, stream);
}

hipError_t launch_fwd_splitk_reduce(int T, int N, int r, int S, float s, const float* part,
                                    const float* upart, const uint16_t* B, uint16_t* y, uint16_t* u_save,
                                    hipStream_t stream) {
  const dim3 grid((N + kRCols - 1) / kRCols, (T + kRRows - 1) / kRRows);
  lora_fwd_splitk_reduce<<<grid, kRThreads, 0, stream>>>(T, N, r, S, s, part, upart, B, y, u_save);
  return hipGetLastError();
}

}  // namespace lnf4
