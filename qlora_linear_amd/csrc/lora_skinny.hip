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
#include <algorithm>

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

// Jobs of one launch: job i reduces M_i^T V_i over the tokens, workgroups
// cb_end[i - 1] .. cb_end[i] - 1 (x the token splits) taking its 256-column blocks.
// With one token split and no optimizer step (`direct`), each workgroup stores its
// sums as the reduce would (job 0 may be dA: into da, unscaled; every other job
// bf16(s sum) into out) and no reduce is launched.
struct SkinnyTab {
  int n;
  int cb_end[kMaxSkinnyJobs];
  const uint16_t* M[kMaxSkinnyJobs];  // [T][C] (x or dY)
  const uint16_t* V[kMaxSkinnyJobs];  // [T][vstr], r columns used (G or U)
  float* part[kMaxSkinnyJobs];        // [splits][r][C] fp32
  int C[kMaxSkinnyJobs], r[kMaxSkinnyJobs], vstr[kMaxSkinnyJobs];
  int direct, first_a;
  float s;
  uint16_t* out[kMaxSkinnyJobs];
  DaOut da;
};

template <int RU>
__global__ __launch_bounds__(kThreads) void skinny_partial_kernel(int T, int t_per_split, const SkinnyTab tab) {
  // V stages hold [64][r] bf16 contiguous (64 r * 2 bytes); fragment reads of the
  // padding ranks j >= r may run up to 64 bytes past a stage. Four stages fit the
  // 160 KB LDS for r <= 32, three for r <= 128, two above (the side-by-side G of
  // several projections, up to 192 ranks).
  constexpr int kStages = RU <= 32 ? 4 : (RU <= 128 ? 3 : 2);
  __shared__ __align__(16) uint16_t ms[kStages][kMElems];
  __shared__ __align__(16) uint16_t vs[kStages][TT * RU + 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // this workgroup's job (uniform; constant table indices, so the fields stay in
  // scalar registers)
  const int bid = blockIdx.x;
  const uint16_t* M = tab.M[0];
  const uint16_t* V = tab.V[0];
  float* part = tab.part[0];
  uint16_t* out = tab.out[0];
  bool is_a = tab.first_a != 0;
  int C = tab.C[0], r = tab.r[0], vstr = tab.vstr[0], cb = bid;
#pragma unroll
  for (int i = 1; i < kMaxSkinnyJobs; ++i)
    if (i < tab.n && bid >= tab.cb_end[i - 1]) {
      M = tab.M[i];
      V = tab.V[i];
      part = tab.part[i];
      out = tab.out[i];
      is_a = false;
      C = tab.C[i];
      r = tab.r[i];  // rank of this job's V (the columns used)
      vstr = tab.vstr[i];  // V row stride (elements): G may be a column slice
      cb = bid - tab.cb_end[i - 1];
    }
  const int c0 = cb * BC;
  const int split = blockIdx.y;
  const int t_begin = split * t_per_split;
  const int t_end = min(T, t_begin + t_per_split);
  const int steps = (t_end - t_begin + TT - 1) / TT;

  // Rows past t_end belong to the next split: each step's descriptors start at the
  // step's first row (scalar arithmetic, scalar offset 0) and stop at t_end, so the
  // lane offsets hold only rows within the step and rows past t_end read zeros.
  const int nrows = t_end - t_begin;
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
    vvoff[p] = piece < v_pieces ? static_cast<uint32_t>((e / r) * vstr + e % r) * 2 : kOutOfRange;
  }
  auto issue = [&](int st) {
    const int stage = st % kStages, left = nrows - st * TT;  // >= 1 rows from the step on
    const size_t row0 = static_cast<size_t>(t_begin) + st * TT;
    const auto rs_m = make_rsrc(M + row0 * C, static_cast<uint32_t>(left) * C * 2);
    const auto rs_v = make_rsrc(V + row0 * vstr, static_cast<uint32_t>(left - 1) * vstr * 2 + r * 2);
#pragma unroll
    for (int q = 0; q < 8; ++q) buf_load16_lds(rs_m, &ms[stage][(wave_u * 8 + q) * 512], mvoff[q], 0);
#pragma unroll
    for (int p = 0; p < kVPW; ++p) {
      const int piece = wave_u * kVPW + p;
      buf_load16_lds(rs_v, &vs[stage][piece * 512], vvoff[p], 0);
    }
  };

  static_assert(kStages >= 2 && kStages <= 4, "wait counts below assume 2 to 4 stages");
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
  if constexpr (RU <= 128) {
    if (tab.direct) {  // uniform: the one split's sums, rounded as the reduce rounds (0 + sum)
      // The workgroup's block goes through the (now idle) M stages so that it leaves
      // in 16-byte stores: dA as [256 columns][RU + 8], each column's ranks
      // contiguous like dA's rows; dB as [RU][256 + 8], like dB's rows.
      constexpr int kAS = RU + 8, kBS = BC + 8;
      static_assert(BC * kAS <= kStages * kMElems && RU * kBS <= kStages * kMElems, "staging fits");
      uint16_t* ot = &ms[0][0];
      __syncthreads();  // every wave is done with the last stage
#pragma unroll
      for (int a = 0; a < RU / 32; ++a)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int cl = wave * 64 + j * 32 + (lane & 31);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int jr = a * 32 + mfma32_row(e, lane);
            const float sum = 0.f + acc[a][j][e];
            if (is_a) ot[cl * kAS + jr] = to_bf16(sum);
            else ot[jr * kBS + cl] = to_bf16(tab.s * sum);
          }
        }
      __syncthreads();
      if (is_a) {  // 8 ranks of one column per store; r and the projection width are multiples of 8
        const int gw = tab.da.gw, q8 = r / 8;
        for (int q = tid; q < BC * q8; q += kThreads) {
          const int cl = q / q8, jr = 8 * (q - cl * q8), c = c0 + cl;
          if (c >= C) continue;
          const int g = jr / gw, jj = jr - g * gw;
          uint16_t* dst = tab.da.p[g] + static_cast<size_t>(c) * gw + jj;
          if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(ot + cl * kAS + jr);
          } else {
            for (int e = 0; e < 8; ++e) dst[e] = ot[cl * kAS + jr + e];
          }
        }
      } else {  // 8 columns of one rank row per store where whole and aligned, else one by one
        for (int q = tid; q < r * (BC / 8); q += kThreads) {
          const int jr = q / (BC / 8), cl = 8 * (q - jr * (BC / 8)), c = c0 + cl;
          if (c >= C) continue;
          uint16_t* dst = out + static_cast<size_t>(jr) * C + c;
          if (c + 8 <= C && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(ot + jr * kBS + cl);
          } else {
            for (int e = 0; e < 8 && c + e < C; ++e) dst[e] = ot[jr * kBS + cl + e];
          }
        }
      }
      return;
    }
  }
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

// Sums of the jobs' partials in split order, elements el_end[i - 1] .. el_end[i] - 1
// for job i ([r][C] of it). Job 0 may be dA (first_a): column j of its sum goes to
// projection j / da.gw, dA_g[c][j - g gw], unscaled; every other job stores
// out[j][c] = bf16(s sum) (dB).
struct SkinnyRed {
  int n, first_a;
  int64_t el_end[kMaxSkinnyJobs];
  const float* part[kMaxSkinnyJobs];
  int C[kMaxSkinnyJobs], r[kMaxSkinnyJobs];
  uint16_t* out[kMaxSkinnyJobs];
};

__global__ __launch_bounds__(256) void skinny_reduce2_kernel(const SkinnyRed red, int64_t total, int splits,
                                                             float s, const DaOut da) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const float* part = red.part[0];
  int C = red.C[0], r = red.r[0];
  uint16_t* out = red.out[0];
  int64_t li = idx;
  bool is_a = red.first_a != 0;
#pragma unroll
  for (int i = 1; i < kMaxSkinnyJobs; ++i)
    if (i < red.n && idx >= red.el_end[i - 1]) {
      part = red.part[i];
      C = red.C[i];
      r = red.r[i];
      out = red.out[i];
      li = idx - red.el_end[i - 1];
      is_a = false;
    }
  const int j = static_cast<int>(li / C), c = static_cast<int>(li - static_cast<int64_t>(j) * C);
  const float sum = sum_splits(part + static_cast<size_t>(j) * C + c, splits, static_cast<size_t>(r) * C);
  if (is_a) {
    const int g = j / da.gw, jj = j - g * da.gw;
    da.p[g][static_cast<size_t>(c) * da.gw + jj] = to_bf16(sum);
  } else {
    out[static_cast<size_t>(j) * C + c] = to_bf16(s * sum);
  }
}

// The same reduction for one projection (ra = rb = r), with the AdamW step of A and
// B applied to the float32 sums instead of storing dA and dB: the gradient never
// goes to HBM. A's state is indexed like A [K][r], B's like B [r][N].
__global__ __launch_bounds__(256) void skinny_reduce2_adamw_kernel(const float* __restrict__ part_a,
                                                                   const float* __restrict__ part_b,
                                                                   int splits, int K, int N, int r, float s,
                                                                   const AdamState sa, const AdamState sb,
                                                                   const AdamWArgs h) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t na = static_cast<int64_t>(K) * r;
  AdamState st;
  size_t e;
  float g;
  if (idx < na) {
    const int j = static_cast<int>(idx / K), c = static_cast<int>(idx - static_cast<int64_t>(j) * K);
    g = sum_splits(part_a + static_cast<size_t>(j) * K + c, splits, static_cast<size_t>(r) * K);
    st = sa;
    e = static_cast<size_t>(c) * r + j;
  } else if (idx < na + static_cast<int64_t>(N) * r) {
    const int64_t i2 = idx - na;
    const int j = static_cast<int>(i2 / N), c = static_cast<int>(i2 - static_cast<int64_t>(j) * N);
    g = __fmul_rn(s, sum_splits(part_b + static_cast<size_t>(j) * N + c, splits, static_cast<size_t>(r) * N));
    st = sb;
    e = static_cast<size_t>(j) * N + c;
  } else {
    return;
  }
  float p = st.p[e], m = st.m[e], v = st.v[e];
  adamw_elem(h, g, p, m, v);
  st.p[e] = p;
  st.m[e] = m;
  st.v[e] = v;
  st.w[e] = to_bf16(p);
}

}  // namespace

bool lora_skinny_supported(int r) { return r % 8 == 0 && r <= 64; }
bool lora_skinny_wide_supported(int r) { return r % 8 == 0 && r <= 192; }

// Token splits, each a whole number of 64-token steps. The partial-sum kernel holds
// one workgroup per CU (its LDS stages), so a grid of blocks x splits workgroups
// takes ceil(blocks splits / 256) rounds, each of `per` tokens plus about three
// steps' worth of fixed cost (pipeline fill, partial-sum stores): the split count
// minimizes that (ties: fewer splits, fewer partials to reduce). A grid just past
// 256 workgroups would otherwise run a second round for a few of them.
int skinny_splits(int64_t T, int64_t K, int64_t N) {
  return skinny_splits_blocks(T, (K + BC - 1) / BC + (N + BC - 1) / BC);
}

int skinny_splits_blocks(int64_t T, int64_t blocks) {
  if (blocks < 1) blocks = 1;
  const int64_t max_splits = std::min<int64_t>(std::max<int64_t>((T + TT - 1) / TT, 1), 256);
  int64_t best = 1, best_cost = -1;
  for (int64_t want = 1; want <= max_splits; ++want) {
    const int64_t per = ((std::max<int64_t>((T + want - 1) / want, 1) + TT - 1) / TT) * TT;
    const int64_t sp = std::max<int64_t>((T + per - 1) / per, 1);
    const int64_t cost = ((blocks * sp + 255) / 256) * (per + 3 * TT);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = sp;
    }
  }
  return static_cast<int>(best);
}

hipError_t launch_skinny_jobs(int T, int n, const SkinnyJob* jobs, int splits, float s, const DaOut& da,
                              hipStream_t stream, const SkinnyAdamW* adam) {
  if (n < 1 || n > kMaxSkinnyJobs || splits < 1) return hipErrorInvalidValue;
  int per = (T + splits - 1) / splits;
  per = ((per + TT - 1) / TT) * TT;
  SkinnyTab tab{};
  SkinnyRed red{};
  tab.n = red.n = n;
  red.first_a = jobs[0].is_a ? 1 : 0;
  int cbs = 0, rmax = 0;
  int64_t els = 0;
  for (int i = 0; i < n; ++i) {
    const SkinnyJob& j = jobs[i];
    if (j.C < 1 || j.r < 1 || j.r % 8 != 0 || j.vstr < j.r || (i > 0 && j.is_a)) return hipErrorInvalidValue;
    cbs += (j.C + BC - 1) / BC;
    els += static_cast<int64_t>(j.r) * j.C;
    tab.cb_end[i] = cbs;
    tab.M[i] = j.M;
    tab.V[i] = j.V;
    tab.part[i] = j.part;
    tab.C[i] = red.C[i] = j.C;
    tab.r[i] = red.r[i] = j.r;
    tab.vstr[i] = j.vstr;
    red.el_end[i] = els;
    red.part[i] = j.part;
    red.out[i] = j.out;
    rmax = std::max(rmax, j.r);
  }
  const dim3 grid(cbs, splits);
  // one token split, no optimizer step, ranks up to 128 (the staging of the
  // workgroup's block fits the M stages): no partials and no reduce launch
  tab.direct = splits == 1 && adam == nullptr && rmax <= 128;
  tab.first_a = red.first_a;
  tab.s = s;
  tab.da = da;
  for (int i = 0; i < n; ++i) tab.out[i] = jobs[i].out;
  if (rmax <= 32)
    skinny_partial_kernel<32><<<grid, kThreads, 0, stream>>>(T, per, tab);
  else if (rmax <= 64)
    skinny_partial_kernel<64><<<grid, kThreads, 0, stream>>>(T, per, tab);
  else if (rmax <= 128)
    skinny_partial_kernel<128><<<grid, kThreads, 0, stream>>>(T, per, tab);
  else if (rmax <= 192)
    skinny_partial_kernel<192><<<grid, kThreads, 0, stream>>>(T, per, tab);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || tab.direct) return e;
  if (adam != nullptr) {  // one projection: dA (job 0) and dB (job 1) of one rank
    if (n != 2 || !jobs[0].is_a || jobs[0].r != jobs[1].r) return hipErrorInvalidValue;
    skinny_reduce2_adamw_kernel<<<static_cast<unsigned>((els + 255) / 256), 256, 0, stream>>>(
        jobs[0].part, jobs[1].part, splits, jobs[0].C, jobs[1].C, jobs[0].r, s, adam->a, adam->b, adam->h);
    return hipGetLastError();
  }
  skinny_reduce2_kernel<<<static_cast<unsigned>((els + 255) / 256), 256, 0, stream>>>(red, els, splits, s, da);
  return hipGetLastError();
}

hipError_t launch_lora_skinny(int T, int K, int N, int ra, int rb, int vsa, float s, const uint16_t* x,
                              const uint16_t* g, const uint16_t* dy, const uint16_t* u,
                              float* part_a, float* part_b, int splits, const DaOut& da,
                              uint16_t* dB, hipStream_t stream, const SkinnyAdamW* adam) {
  SkinnyJob jobs[2];
  int n = 0;
  if (K > 0) jobs[n++] = SkinnyJob{x, g, part_a, nullptr, K, ra, vsa, true};
  if (N > 0) jobs[n++] = SkinnyJob{dy, u, part_b, dB, N, rb, rb, false};
  if (n == 0) return hipSuccess;
  return launch_skinny_jobs(T, n, jobs, splits, s, da, stream, adam);
}

}  // namespace lnf4
