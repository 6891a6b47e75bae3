// Rank-r gradients of the fused NF4-LoRA linear (gfx950):
//     dA = x^T G            [d_in, r],  G = s dY B^T  (bf16, from the dX kernel)
//     dB = s U^T dY         [r, d_out], U = x A       (bf16, from the forward)
// Both are skinny products reduced over all T tokens; they are bound by reading
// x and dY once from HBM (the pages' "hand-written backward" of "Unlocking AI
// potential: Unsloth's algorithms and implementation", core-algorithms section).
//
// One launch computes split-T partial sums of both: workgroup (column block,
// token split) streams its [tokens x 256] slice of x (or dY) through a 4-stage
// direct-to-LDS pipeline, together with the matching [tokens x r] rows of G (or
// U), and accumulates out^T[j][c] = sum_t V[t][j] M[t][c] with
// v_mfma_f32_32x32x16_bf16. Both operands are stored in LDS in their natural
// row-major [t][*] layout and read with ds_read_b64_tr_b16, which yields the
// token-contiguous fragments the MFMA wants without transposed stores.
// A second kernel sums the partials in split order (deterministic), applies the
// scale and stores bf16 in each gradient's layout.
#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int kThreads = 256;  // 4 waves, 64 columns each
constexpr int BC = 256;        // columns per workgroup
constexpr int TT = 64;         // tokens per pipeline step
constexpr int kMElems = TT * BC;  // [64][256] bf16 = 32 KB, 32-byte units XOR-swizzled by row

// Element offset of (row t, column c) in an M stage: 32-byte units (16 columns)
// are XOR-ed with 2 (t & 3), so the four rows a 16-lane transposing read touches
// fall in distinct banks.
__device__ __forceinline__ int m_off(int t, int c) {
  return t * BC + ((((c >> 4) ^ (2 * (t & 3)))) << 4) + (c & 15);
}

template <int RU>
__global__ __launch_bounds__(kThreads) void skinny_partial_kernel(
    int T, int K, int N, int ra, int rb, int vsa, int cb_a, int t_per_split, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ dy, const uint16_t* __restrict__ u,
    float* __restrict__ part_a, float* __restrict__ part_b) {
  // V stages hold [64][r] bf16 contiguous (64 r * 2 bytes); fragment reads of the
  // padding ranks j >= r may run up to 64 bytes past a stage. Four stages fit the
  // 160 KB LDS for r <= 32, three for r <= 64.
  constexpr int kStages = RU <= 32 ? 4 : 3;
  __shared__ __align__(16) uint16_t ms[kStages][kMElems];
  __shared__ __align__(16) uint16_t vs[kStages][TT * RU + 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool job_a = static_cast<int>(blockIdx.x) < cb_a;
  const int cb = job_a ? blockIdx.x : blockIdx.x - cb_a;
  const int r = job_a ? ra : rb;      // rank of this job's V (the columns used)
  const int vstr = job_a ? vsa : rb;  // V row stride (elements): G may be a column slice
  const int C = job_a ? K : N;
  const uint16_t* M = job_a ? x : dy;
  const uint16_t* V = job_a ? g : u;
  float* part = job_a ? part_a : part_b;
  const int c0 = cb * BC;
  const int split = blockIdx.y;
  const int t_begin = split * t_per_split;
  const int t_end = min(T, t_begin + t_per_split);
  const int steps = (t_end - t_begin + TT - 1) / TT;

  // Rows past t_end belong to the next split: the ranges stop at t_end so they
  // read as zeros.
  const auto rs_m = make_rsrc(M + static_cast<size_t>(t_begin) * C,
                              static_cast<uint32_t>(t_end - t_begin) * C * 2);
  const auto rs_v = make_rsrc(V + static_cast<size_t>(t_begin) * vstr,
                              static_cast<uint32_t>(t_end - t_begin - 1) * vstr * 2 + r * 2);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // M stage: each wave fills 16 rows with eight 1 KB loads (2 rows each); lane i
  // lands on physical 16-byte piece i & 31 of row (i >> 5) and loads the logical
  // piece the swizzle maps there.
  uint32_t mvoff[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int t = wave * 16 + q * 2 + (lane >> 5);
    const int piece = lane & 31, unit = piece >> 1, half = piece & 1;
    const int lunit = unit ^ (2 * (t & 3));
    mvoff[q] = static_cast<uint32_t>(t) * C * 2 + (c0 + lunit * 16 + half * 8) * 2;
  }
  // V stage: [64][r] bf16 contiguous in LDS = r / 8 KB pieces (r % 8 == 0); lane
  // L of piece p brings elements 512 p + 8 L .. +7 of that block, i.e. token row
  // (512 p + 8 L) / r, columns (512 p + 8 L) % r of V (row stride vstr). Every
  // wave issues kVPW piece loads per step so all waves wait on the same vmcnt;
  // pieces past r / 8 use an out-of-range offset and only write zeros.
  constexpr int kVPW = RU / 32;
  const int v_pieces = r / 8;
  uint32_t vvoff[kVPW];
#pragma unroll
  for (int p = 0; p < kVPW; ++p) {
    const int piece = wave * kVPW + p, e = piece * 512 + lane * 8;
    vvoff[p] = piece < v_pieces ? static_cast<uint32_t>((e / r) * vstr + e % r) * 2 : 0x7FFFFFF0u;
  }
  auto issue = [&](int st) {
    const int stage = st % kStages;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      buf_load16_lds(rs_m, &ms[stage][(wave_u * 8 + q) * 512], mvoff[q], st * TT * C * 2);
#pragma unroll
    for (int p = 0; p < kVPW; ++p) {
      const int piece = wave_u * kVPW + p;
      buf_load16_lds(rs_v, &vs[stage][piece * 512], vvoff[p], st * TT * vstr * 2);
    }
  };

  static_assert(kStages == 3 || kStages == 4, "wait counts below assume 3 or 4 stages");
  // fragment addresses (transposing reads; 16-lane group g16, lane m16)
  const int g16 = lane >> 4, m16 = lane & 15;
  // A operand = V^T: rows j (M dim), reduction t. Lane m16 points at token row
  // 8 (g16 >> 1) + (m16 >> 2) (+4 for the second read), ranks 16 (g16 & 1) + 4 (m16 & 3).
  const int vt = 8 * (g16 >> 1) + (m16 >> 2);
  const int vj = 16 * (g16 & 1) + 4 * (m16 & 3);
  // B operand = M: columns c, reduction t; same pattern over this wave's columns
  const int mc = wave * 64 + 16 * (g16 & 1) + 4 * (m16 & 3);

  f32x16_t acc[RU / 32][2];
#pragma unroll
  for (int a = 0; a < RU / 32; ++a)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][j][e] = 0.f;

#pragma unroll
  for (int p = 0; p < kStages - 1; ++p)
    if (p < steps) issue(p);

  for (int st = 0; st < steps; ++st) {
    // step st has landed once at most (steps issued after it) * (8 + kVPW) loads remain
    constexpr int kPer = 8 + kVPW;
    const int ahead = min(kStages - 2, steps - 1 - st);
    if (kStages == 4 && ahead >= 2) wait_vmem_upto<2 * kPer>();
    else if (ahead == 1) wait_vmem_upto<kPer>();
    else wait_vmem();
    __syncthreads();  // step st visible to all waves; step st - 1 fully consumed
    if (st + kStages - 1 < steps) issue(st + kStages - 1);
    const int stage = st % kStages;
    const uint16_t* mst = ms[stage];
    const uint16_t* vst = vs[stage];
#pragma unroll
    for (int ks = 0; ks < TT / 16; ++ks) {
      const int t0 = ks * 16;
      uint4 af[RU / 32], bf[2];
#pragma unroll
      for (int a = 0; a < RU / 32; ++a) {
        const uint16_t* p = vst + (t0 + vt) * r + a * 32 + vj;
        const uint2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 4 * r);
        af[a] = uint4{lo.x, lo.y, hi.x, hi.y};
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = t0 + vt, c = mc + j * 32;
        const uint2 lo = lds_read_tr16(mst + m_off(t, c)), hi = lds_read_tr16(mst + m_off(t + 4, c));
        bf[j] = uint4{lo.x, lo.y, hi.x, hi.y};
      }
#pragma unroll
      for (int a = 0; a < RU / 32; ++a)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[a][j] = mfma32(af[a], bf[j], acc[a][j]);
    }
  }

  // partial[split][j][c]: lane column c = l & 31 of each 32-column tile
#pragma unroll
  for (int a = 0; a < RU / 32; ++a)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = c0 + wave * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int jr = a * 32 + mfma32_row(e, lane);
        if (jr < r && c < C) part[(static_cast<size_t>(split) * r + jr) * C + c] = acc[a][j][e];
      }
    }
}

// Sum of p[sp * stride], sp = 0 .. splits - 1, in split order. The loads go out in
// independent batches of eight (a plain loop pays one memory latency per split:
// 13-16 us at 64 splits); the additions keep their order, so the bits do not change.
__device__ __forceinline__ float sum_splits(const float* __restrict__ p, int splits, size_t stride) {
  float sum = 0.f;
  int sp = 0;
  for (; sp + 8 <= splits; sp += 8) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = p[static_cast<size_t>(sp + q) * stride];
#pragma unroll
    for (int q = 0; q < 8; ++q) sum += v[q];
  }
  for (; sp < splits; ++sp) sum += p[static_cast<size_t>(sp) * stride];
  return sum;
}

// dA[c][j] = sum_split part_a[split][j][c], columns j split into projections of
// da.gw ranks (dA_g[c][j - g gw]);  dB[j][c] = s sum_split part_b[split][j][c]
__global__ __launch_bounds__(256) void skinny_reduce2_kernel(const float* __restrict__ part_a,
                                                             const float* __restrict__ part_b,
                                                             int splits, int K, int N, int ra, int rb,
                                                             float s, const DaOut da,
                                                             uint16_t* __restrict__ dB) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t na = static_cast<int64_t>(K) * ra;
  if (idx < na) {
    const int j = static_cast<int>(idx / K), c = static_cast<int>(idx - static_cast<int64_t>(j) * K);
    const float sum = sum_splits(part_a + static_cast<size_t>(j) * K + c, splits, static_cast<size_t>(ra) * K);
    const int g = j / da.gw, jj = j - g * da.gw;
    da.p[g][static_cast<size_t>(c) * da.gw + jj] = to_bf16(sum);
  } else if (idx < na + static_cast<int64_t>(N) * rb) {
    const int64_t i2 = idx - na;
    const int j = static_cast<int>(i2 / N), c = static_cast<int>(i2 - static_cast<int64_t>(j) * N);
    const float sum = sum_splits(part_b + static_cast<size_t>(j) * N + c, splits, static_cast<size_t>(rb) * N);
    dB[static_cast<size_t>(j) * N + c] = to_bf16(s * sum);
  }
}

}  // namespace

bool lora_skinny_supported(int r) { return r % 8 == 0 && r <= 64; }

// Token splits: about one workgroup per CU in total, each split a whole number
// of 64-token steps.
int skinny_splits(int64_t T, int64_t K, int64_t N) {
  const int64_t blocks = (K + BC - 1) / BC + (N + BC - 1) / BC;
  int64_t want = (256 + blocks - 1) / blocks;
  const int64_t max_splits = (T + TT - 1) / TT;
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  int64_t per = (T + want - 1) / want;
  per = ((per + TT - 1) / TT) * TT;
  return static_cast<int>((T + per - 1) / per);
}

hipError_t launch_lora_skinny(int T, int K, int N, int ra, int rb, int vsa, float s, const uint16_t* x,
                              const uint16_t* g, const uint16_t* dy, const uint16_t* u,
                              float* part_a, float* part_b, int splits, const DaOut& da,
                              uint16_t* dB, hipStream_t stream) {
  int per = (T + splits - 1) / splits;
  per = ((per + TT - 1) / TT) * TT;
  const int cb_a = (K + BC - 1) / BC, cb_b = (N + BC - 1) / BC;
  const dim3 grid(cb_a + cb_b, splits);
  if ((K > 0 ? ra : 0) <= 32 && (N > 0 ? rb : 0) <= 32)
    skinny_partial_kernel<32><<<grid, kThreads, 0, stream>>>(T, K, N, ra, rb, vsa, cb_a, per, x, g, dy, u,
                                                             part_a, part_b);
  else
    skinny_partial_kernel<64><<<grid, kThreads, 0, stream>>>(T, K, N, ra, rb, vsa, cb_a, per, x, g, dy, u,
                                                             part_a, part_b);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = static_cast<int64_t>(K) * ra + static_cast<int64_t>(N) * rb;
  skinny_reduce2_kernel<<<static_cast<unsigned>((total + 255) / 256), 256, 0, stream>>>(
      part_a, part_b, splits, K, N, ra, rb, s, da, dB);
  return hipGetLastError();
}

}  // namespace lnf4
