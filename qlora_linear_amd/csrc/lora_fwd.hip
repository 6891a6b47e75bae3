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
//     each wave owning a 128 x 64 sub-tile of 4 x 2 v_mfma_f32_32x32x16_bf16
//     accumulators. A large M-tile amortizes the in-loop dequantization: every
//     weight element is dequantized T/256 times over the whole GEMM.
//   * When 256 x 256 tiles would leave CUs idle (a few thousand tokens or fewer
//     over a narrow d_out), the same kernel runs 128 x 128 tiles: 256 threads in
//     2 x 2 waves of 64 x 64 (2 x 2 accumulators), half the LDS, so two
//     workgroups share a CU and the grid has four times as many tiles.
//   * K-loop in steps of 64 = one NF4 block, so every weight row has exactly one
//     absmax per step. LDS holds two stages (x tile, dequantized weight tile,
//     A slice), XOR-swizzled for conflict-free 16-byte fragment reads; while the
//     MFMAs consume one stage, the next stage's x is stored and its packed codes
//     (already in registers) are dequantized into the other: level lookup in an
//     LDS table, multiply by the row's absmax, round to bf16.
//   * U = x A is accumulated in the same loop from the same x tile: each wave
//     owns 32 token rows of U (16 x 16 x 32 MFMAs for r <= 16, else 32 x 32 x 16).
//   * Epilogue: bf16(s U) and B go through LDS, one more MFMA pass over the rank
//     dimension adds (s U) B into the accumulators, and bf16 y is stored.
//   * When even 128 x 128 tiles leave CUs idle (a few hundred tokens over a
//     narrow d_out), a single projection's K-loop is split across workgroups:
//     each writes fp32 partial products (and partial U) to a workspace and the
//     split-K reduce adds bf16(s U) B and stores y.
//   * With many token tiles (8 of 128 rows or 16 of 256) the in-loop
//     dequantization would be repeated that many times per weight element: the
//     call then dequantizes the weight once into the workspace (bf16, the same
//     values) and the kernel stages bf16 weight tiles like x (DQ instances).
//     There, from 4096 tokens at rank > 16, U = x A comes from a separate pass
//     and the tile kernel (RU = 0) only reads bf16(s U) in its epilogue: the
//     in-loop U is recomputed by every column tile.
//   * Several projections of the same x (q/k/v or gate/up: the multi-projection
//     fusion) share one launch: the column tiles of all projections form one
//     grid, each tile reads its projection's weight, A, B and output from a small
//     table passed by value, and the tile order keeps a token tile's x hot in L2
//     across projections. A single projection is a one-entry table.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int BK = 64;
constexpr int kAStride = 72;  // A^T slice rows: 64 bf16 + 16 B pad (conflict-free b128 reads)

// Square output tile of edge BT (256 or 128): 2 x (BT / 64) waves, each owning
// BT / 2 token rows x 64 columns.
template <int BT>
struct FwdTile {
  static constexpr int kThreads = 2 * BT;
  static constexpr int kWN = BT / 64;          // waves along d_out
  static constexpr int kFM = BT / 64;          // 32-row fragments per wave along tokens
  static constexpr int kTileElems = BT * 64;   // one bf16 [BT][64] tile
  // workgroups per CU the register budget is sized for (LDS allows two at 128)
  static constexpr int kMinBlocks = BT == 128 ? 2 : 1;
};


// BT: tile edge; RU: U columns accumulated in the K-loop (16 for r <= 16, else r
// rounded up to 32); RE: rank padded to the 16-wide reduction step of the
// epilogue MFMA.
//
// LDS (static, so the compiler can prove the direct-to-LDS loads into one stage
// never alias reads of the other): level table, two stages of x [BT][64],
// dequantized weight [BT][64] and A^T slice [RU][64], all bf16 and swizzled.
//
// Split mode (part != nullptr, one projection): workgroup b runs tile b % tiles
// over K-steps [steps_per (b / tiles), ...) and writes fp32 partial products to
// part [split][T][N] and, from the first column tile, fp32 partial U to upart
// [split][T][r]; no epilogue.
//
// DQ: the weight was dequantized beforehand into tab.wdq (bf16 [N][K], the same
// values the in-loop dequantization produces), and its tiles are staged like x:
// direct-to-LDS loads into the same swizzled layout, no codes, no level lookups.
template <int BT, int RU, int RE, bool DQ>
__global__ __launch_bounds__(FwdTile<BT>::kThreads, FwdTile<BT>::kMinBlocks) void lora_fwd_kernel(
    int T, int K, int r, float s, const uint16_t* __restrict__ x, const ProjTable tab, int steps_per,
    float* __restrict__ part, float* __restrict__ upart) {
  using Tl = FwdTile<BT>;
  constexpr int kThreads = Tl::kThreads, BM = BT, BN = BT, kFM = Tl::kFM, kHalf = BT / 2;
  constexpr int kTileElems = Tl::kTileElems;
  __shared__ __align__(1024) float lut[16];  // first in LDS: level addresses need no base
  __shared__ __align__(16) uint16_t xs0[kTileElems];
  __shared__ __align__(16) uint16_t xs1[kTileElems];
  __shared__ __align__(16) uint16_t ws0[kTileElems];
  __shared__ __align__(16) uint16_t ws1[kTileElems];
  __shared__ __align__(16) uint16_t as0[RU > 0 ? RU * kAStride : 8];
  __shared__ __align__(16) uint16_t as1[RU > 0 ? RU * kAStride : 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Tl::kWN, wn = wave % Tl::kWN;  // 2 x kWN waves, BT / 2 x 64 each
  const int l32 = lane & 31, lh = lane >> 5;
  const int mt = (T + BM - 1) / BM, nt_all = tab.tile_end[tab.n - 1];
  const int tiles = mt * nt_all;
  const int tile_id = blockIdx.x % tiles, sp = blockIdx.x / tiles;
  int tm, tn;
  tile_coords(xcd_remap(tile_id, tiles), mt, nt_all, 4, tm, tn);
  int gp = 0;  // this tile's projection (wave-uniform)
  while (gp + 1 < tab.n && tn >= tab.tile_end[gp]) ++gp;
  if (gp > 0) tn -= tab.tile_end[gp - 1];
  const int N = tab.N[gp];
  const uint8_t* __restrict__ codes = tab.codes[gp];
  const float* __restrict__ absmax = tab.absmax[gp];
  const uint16_t* __restrict__ A = tab.A[gp];
  const uint16_t* __restrict__ B = tab.B[gp];
  uint16_t* __restrict__ y = tab.y[gp];
  uint16_t* __restrict__ u_save = tab.u[gp];
  const int m0 = tm * BM, n0 = tn * BN;
  const int K2 = K / 2, KB = K / BK;
  const int kbeg = sp * steps_per;                 // first K-step of this workgroup
  const int nsteps = min(KB - kbeg, steps_per);    // >= 1

  if (tid < 16) lut[tid] = nf4_level_reg(tid);
  // A^T slice rows r .. RU-1 stay zero in both stages
  for (int e = r * kAStride + tid; e < RU * kAStride; e += kThreads) {
    as0[e] = 0;
    as1[e] = 0;
  }

  // ---- global -> LDS / register staging of one K-step (buffer loads) ------------
  // Buffer resources cover this tile's rows only: loads of rows past T (x) or N
  // (weights) return zeros, and the per-step advance is a uniform scalar offset.
  // (shifted to the workgroup's first K-step; row strides are unchanged)
  const int rows_x = min(T - m0, BM), rows_w = min(N - n0, BN);
  const auto rs_x = make_rsrc(x + static_cast<size_t>(m0) * K + kbeg * BK,
                              static_cast<uint32_t>(rows_x) * K * 2 - kbeg * BK * 2);
  const auto rs_c = make_rsrc(codes + static_cast<size_t>(n0) * K2 + kbeg * 32,
                              static_cast<uint32_t>(rows_w) * K2 - kbeg * 32);
  const auto rs_s = make_rsrc(absmax + static_cast<size_t>(n0) * KB + kbeg,
                              (static_cast<uint32_t>(rows_w) * KB - kbeg) * 4);
  const auto rs_a = make_rsrc(A + static_cast<size_t>(kbeg) * BK * r,
                              static_cast<uint32_t>(K - kbeg * BK) * r * 2);
  const uint16_t* wdq = DQ ? tab.wdq[gp] : x;
  const auto rs_w = make_rsrc(wdq + (DQ ? static_cast<size_t>(n0) * K + kbeg * BK : 0),
                              DQ ? static_cast<uint32_t>(rows_w) * K * 2 - kbeg * BK * 2 : 0u);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // x: wave w fills rows 32 w .. 32 w + 31 with four 1 KB direct-to-LDS loads
  // (BT / 32 waves cover the tile)
  // (8 rows each). Lane i lands on physical chunk i & 7 of its row, so it loads
  // the logical chunk that the swizzle maps there.
  uint32_t xvoff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = (wave * 4 + q) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    xvoff[q] = static_cast<uint32_t>(row) * K * 2 + chunk * 16;
  }
  // Every step index passed to a load is clamped to this workgroup's last step:
  // the run-ahead loads of the last steps (one and two past the end) then read
  // that step again (unused) and never address past the operands.
  const int klast = nsteps - 1;
  auto load_x_lds = [&](int kt, uint16_t* stage) {
    kt = min(kt, klast);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      buf_load16_lds(rs_x, stage + (wave_u * 4 + q) * 512, xvoff[q], kt * BK * 2);
  };
  // DQ: weight rows have x's row stride (K), so x's lane offsets serve them
  auto load_w_lds = [&](int kt, uint16_t* stage) {
    kt = min(kt, klast);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      buf_load16_lds(rs_w, stage + (wave_u * 4 + q) * 512, xvoff[q], kt * BK * 2);
  };
  // codes: row tid>>1 (< BT), 16 bytes (32 codes) at half tid&1 of the block; one absmax
  const int crow = tid >> 1, chalf = tid & 1;
  const uint32_t cvoff = static_cast<uint32_t>(crow) * K2 + chalf * 16;
  const uint32_t svoff = static_cast<uint32_t>(crow) * KB * 4;
  // A slice: the 64 x r block of A is contiguous; 8-element chunks tid + kThreads i
  // (r % 8 == 0 on this path)
  constexpr int kAPer = (64 * RU / 8 + kThreads - 1) / kThreads;
  // Register sets for step s live in slot s & 1, so the prefetch of step kt + 2
  // and the dequantization of step kt + 1 use different registers with no copies.
  uint4 creg[2], areg[2][kAPer > 0 ? kAPer : 1];
  float sreg[2];
  auto load_codes = [&](int kt, int slot) {
    kt = min(kt, klast);
    creg[slot] = buf_load16(rs_c, cvoff, kt * 32);
    sreg[slot] = __uint_as_float(buf_load4(rs_s, svoff, kt * 4));
  };
  // (chunks past the slice's 8 r read zeros: at the last step they would lie past A)
  auto load_a = [&](int kt, int slot) {
    kt = min(kt, klast);
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int ch = tid + kThreads * i;
      areg[slot][i] = buf_load16(rs_a, ch < 8 * r ? ch * 16 : kOutOfRange, kt * BK * r * 2);
    }
  };

  // Loop-invariant LDS element offsets. Every fragment row this lane reads has
  // the same swizzle key ((row >> 1) & 7 depends only on lane & 31), so one chunk
  // offset per k-slice serves all of its A and B fragments.
  const int fkey = (l32 >> 1) & 7;
  int choff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) choff[ks] = ((2 * ks + lh) ^ fkey) << 3;
  const int a_off = (wm * kHalf + l32) * 64;  // + i * 2048
  const int b_off = (wn * 64 + l32) * 64;   // + j * 2048
  const int ua_off = a_off + wn * 2048;
  // Rank 64: row block i of the wave's BT / 2 x rows is block (i + wn) % kFM of
  // its slab, so block 0 is the 32 rows whose U this wave accumulates and U takes the
  // main x fragment instead of a read of its own (measured: 6 % faster at r = 64,
  // slower at r <= 32, where the extra address arithmetic costs more than the
  // read). choff[ks] = choff[0] ^ (ks << 4), so each block keeps one address
  // register (its row offset has no bits below 6).
  constexpr bool kRot = RU == 64;
  int xb[kFM];
#pragma unroll
  for (int i = 0; i < kFM; ++i) xb[i] = ((wm * kHalf + ((i + wn) % kFM) * 32 + l32) * 64) | choff[0];
  auto blk = [&](int i) { return kRot ? ((i + wn) % kFM) : i; };  // row block of fragment i
  const int ub_off = l32 * kAStride;        // + u * 32 * kAStride
  // r <= 16: 16 x 16 x 32 fragments of U rows wm * BT / 2 + wn * 32 + 16 rb + (lane & 15)
  constexpr bool kU16 = RU == 16;
  const int l16 = lane & 15, lq = lane >> 4;
  const int ua16_off = (wm * kHalf + wn * 32 + l16) * 64;  // + rb * 1024
  int choff16[2];
#pragma unroll
  for (int kq = 0; kq < 2; ++kq) choff16[kq] = ((4 * kq + lq) ^ (l16 >> 1)) << 3;
  const int ub16_off = l16 * kAStride + 8 * lq;         // + kq * 32
  const int wkey = (crow >> 1) & 7;
  int ws_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) ws_off[q] = crow * 64 + (((chalf * 4 + q) ^ wkey) << 3);

  // Dequantize the 8 codes of one dword (one NF4 block, scale a) to 8 bf16 and
  // store them as one 16-byte chunk. Level addresses (4 * code) come from two
  // byte planes: even codes (w << 2) & 0x3C.., odd codes (w >> 2) & 0x3C...
  const unsigned char* lutb = reinterpret_cast<const unsigned char*>(lut);
  auto lookup = [&](uint32_t w, float* v) {
    uint32_t ev = (w << 2) & 0x3C3C3C3Cu, od = (w >> 2) & 0x3C3C3C3Cu;
    // keep the two planes: otherwise each address is rebuilt as shift + mask
    asm volatile("" : "+v"(ev), "+v"(od));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = *reinterpret_cast<const float*>(lutb + __builtin_amdgcn_ubfe(ev, 8 * j, 8));
      v[2 * j + 1] = *reinterpret_cast<const float*>(lutb + __builtin_amdgcn_ubfe(od, 8 * j, 8));
    }
  };
  auto finish_store = [&](const float* lv, float a, uint16_t* dst) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = lv[j] * a;
    uint4 o;
    o.x = pack_bf16x2(v[0], v[1]);
    o.y = pack_bf16x2(v[2], v[3]);
    o.z = pack_bf16x2(v[4], v[5]);
    o.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(dst) = o;
  };
  auto dequant_store = [&](uint32_t w, float a, uint16_t* dst) {
    float lv[8];
    lookup(w, lv);
    finish_store(lv, a, dst);
  };
  // Thread c < 8 r owns 8 consecutive j of one k of the A slice (r % 8 == 0) and
  // writes them transposed: rows j0 .. j0 + 7 of the padded A^T tile, one address
  // register plus immediate row offsets.
  int a_dst[kAPer > 0 ? kAPer : 1];
#pragma unroll
  for (int i = 0; i < kAPer; ++i) {
    const int c = tid + kThreads * i, e = c * 8, kk = e / r, j0 = e - kk * r;
    a_dst[i] = j0 * kAStride + kk;
  }
  auto store_a = [&](uint16_t* as, const uint4* arr) {
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      if (tid + kThreads * i < 8 * r) {
        const uint32_t v[4] = {arr[i].x, arr[i].y, arr[i].z, arr[i].w};
#pragma unroll
        for (int h = 0; h < 8; ++h)
          as[a_dst[i] + h * kAStride] = static_cast<uint16_t>(v[h >> 1] >> (16 * (h & 1)));
      }
    }
  };

  f32x16_t acc[kFM][2];
  f32x16_t uacc[RU / 32 > 0 ? RU / 32 : 1];
  f32x4_t uacc16[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
#pragma unroll
  for (int u = 0; u < (RU / 32 > 0 ? RU / 32 : 1); ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) uacc[u][e] = 0.f;

  // prologue: step 0 into stage 0, step 1 into registers
  load_x_lds(0, xs0);
  if constexpr (DQ) load_w_lds(0, ws0);
  else load_codes(0, 0);
  load_a(0, 0);
  wait_vmem();
  __syncthreads();  // lut, zeroed A^T rows and x of step 0 visible
  {
    if constexpr (!DQ) {
      const uint32_t cw[4] = {creg[0].x, creg[0].y, creg[0].z, creg[0].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) dequant_store(cw[q], sreg[0], ws0 + ws_off[q]);
    }
    store_a(as0, areg[0]);
  }
  if constexpr (!DQ) load_codes(1, 1);  // clamped: a one-step tile loads step 0 again (unused)
  load_a(1, 1);
  __syncthreads();

  // One K-step. `cur` is a compile-time stage index (the loop is unrolled by two)
  // so every LDS address below is a loop-invariant register plus an immediate.
  // The step is branch-free: on the last step the next-stage work lands in the
  // unused stage (the clamped loads re-read the last step, unused), which keeps
  // the whole step one basic block for the scheduler. Fragments of k-slice
  // ks + 1 and the level lookups of code dword ks + 1 are issued one slice ahead
  // of their use.
  struct Frag {
    uint4 a[kFM], b[2], au, bu[RU / 32 > 0 ? RU / 32 : 1], au16[2], bu16;
  };
  auto kstep = [&](int kt, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value;
    const uint16_t* xc = cur ? xs1 : xs0;
    const uint16_t* wc = cur ? ws1 : ws0;
    const uint16_t* ac = cur ? as1 : as0;
    uint16_t* xn = cur ? xs0 : xs1;
    uint16_t* wnx = cur ? ws0 : ws1;
    uint16_t* an = cur ? as0 : as1;
    load_x_lds(kt + 1, xn);
    constexpr int nslot = cur ^ 1;  // registers of step kt + 1
    if constexpr (DQ) load_w_lds(kt + 1, wnx);
    else load_codes(kt + 2, cur);
    load_a(kt + 2, cur);
    // DQ: keep the next stage's loads at the top of the step (left to itself the
    // scheduler sinks them below most of the MFMAs, and the end-of-step wait then
    // exposes their whole latency)
    if constexpr (DQ) __builtin_amdgcn_sched_barrier(0);
    const uint32_t cw[4] = {creg[nslot].x, creg[nslot].y, creg[nslot].z, creg[nslot].w};
    const float ar = sreg[nslot];
    // re-declared opaque every step: one register per block, the slice bits
    // flipped per read, rather than one hoisted register per (block, slice)
    int xbs[kFM];
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
      xbs[i] = xb[i];
      if constexpr (kRot) asm volatile("" : "+v"(xbs[i]));
    }
    auto read_frag = [&](Frag& f, int ks) {
#pragma unroll
      for (int i = 0; i < kFM; ++i)
        f.a[i] = kRot ? *reinterpret_cast<const uint4*>(xc + (xbs[i] ^ (ks << 4)))
                      : *reinterpret_cast<const uint4*>(xc + a_off + i * 2048 + choff[ks]);
#pragma unroll
      for (int j = 0; j < 2; ++j) f.b[j] = *reinterpret_cast<const uint4*>(wc + b_off + j * 2048 + choff[ks]);
      if constexpr (kU16) {
        if (ks & 1) {  // one 32-wide k-slice of U per two 16-wide MFMA slices
          f.au16[0] = *reinterpret_cast<const uint4*>(xc + ua16_off + choff16[ks >> 1]);
          f.au16[1] = *reinterpret_cast<const uint4*>(xc + ua16_off + 1024 + choff16[ks >> 1]);
          f.bu16 = *reinterpret_cast<const uint4*>(ac + ub16_off + (ks >> 1) * 32);
        }
      } else if constexpr (RU > 0) {
        if constexpr (!kRot) f.au = *reinterpret_cast<const uint4*>(xc + ua_off + choff[ks]);
#pragma unroll
        for (int u = 0; u < RU / 32; ++u)
          f.bu[u] = *reinterpret_cast<const uint4*>(ac + ub_off + u * 32 * kAStride + (2 * ks + lh) * 8);
      }
    };
    Frag fr[2];
    float lv[2][8];
    read_frag(fr[0], 0);
    if constexpr (!DQ) lookup(cw[0], lv[0]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      Frag& f = fr[ks & 1];
      if (ks < 3) {
        read_frag(fr[(ks + 1) & 1], ks + 1);
        if constexpr (!DQ) lookup(cw[ks + 1], lv[(ks + 1) & 1]);
      }
#pragma unroll
      for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(f.a[i], f.b[j], acc[i][j]);
      if constexpr (kU16) {
        if (ks & 1) {
          uacc16[0] = mfma16(f.au16[0], f.bu16, uacc16[0]);
          uacc16[1] = mfma16(f.au16[1], f.bu16, uacc16[1]);
        }
      } else if constexpr (RU > 0) {
#pragma unroll
        for (int u = 0; u < RU / 32; ++u) uacc[u] = mfma32(kRot ? f.a[0] : f.au, f.bu[u], uacc[u]);
      }
      if constexpr (!DQ) finish_store(lv[ks & 1], ar, wnx + ws_off[ks]);
      if (ks == 3) store_a(an, areg[nslot]);
    }
    // x (and, DQ, the weight) of the next stage has landed in LDS (the codes,
    // absmax and A loads of step kt + 2, issued after it, may still be in flight)
    wait_vmem_upto<(DQ ? 0 : 2) + kAPer>();
    __syncthreads();
  };
  for (int kt = 0; kt < nsteps; kt += 2) {
    kstep(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < nsteps) kstep(kt + 1, std::integral_constant<int, 1>{});
  }

  if (part != nullptr) {  // split mode: fp32 partials, no epilogue
    wait_vmem();          // run-ahead loads land before the workgroup ends
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + wm * kHalf + blk(i) * 32 + mfma32_row(e, lane);
          if (row < T && col < N) part[(static_cast<size_t>(sp) * T + row) * N + col] = acc[i][j][e];
        }
      }
    if (tn != 0) return;
    float* ud = upart + static_cast<size_t>(sp) * T * r;
#pragma unroll
    for (int u = 0; u < RU / 32; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * kHalf + wn * 32 + mfma32_row(e, lane), col = u * 32 + l32;
        if (col < r && row < T) ud[static_cast<size_t>(row) * r + col] = uacc[u][e];
      }
    if constexpr (kU16) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + wm * kHalf + wn * 32 + rb * 16 + 4 * lq + e;
          if (l16 < r && row < T) ud[static_cast<size_t>(row) * r + l16] = uacc16[rb][e];
        }
    }
    return;
  }

  // ---- epilogue: acc += bf16(s U) B ---------------------------------------------
  // Rank-wide tiles: rows of RE bf16, padded to RE + 8 (conflict-free 16-byte
  // reads) when that fits a [BT][64] buffer, else swizzled like the main tiles.
  constexpr int ES = RE + 8;
  constexpr bool kPad = BT * ES <= kTileElems;
  auto ep = [](int row, int col) {  // element offset of (row, col)
    if constexpr (kPad) return row * ES + col;
    else return swz64(row, col >> 3) + (col & 7);
  };
  uint16_t* us = xs0;  // [BT][RE] bf16(s U)
  uint16_t* bt = ws0;  // [BT][RE] B^T tile
#pragma unroll
  for (int u = 0; u < RU / 32; ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = wm * kHalf + wn * 32 + mfma32_row(e, lane), col = u * 32 + l32;
      const float uv = uacc[u][e];
      if (col < RE) us[ep(row, col)] = to_bf16(s * uv);
      if (u_save != nullptr && tn == 0 && col < r && m0 + row < T)
        u_save[static_cast<size_t>(m0 + row) * r + col] = to_bf16(uv);
    }
  if constexpr (kU16) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = wm * kHalf + wn * 32 + rb * 16 + 4 * lq + e;
        const float uv = uacc16[rb][e];
        us[ep(row, l16)] = to_bf16(s * uv);
        if (u_save != nullptr && tn == 0 && l16 < r && m0 + row < T)
          u_save[static_cast<size_t>(m0 + row) * r + l16] = to_bf16(uv);
      }
  }
  if constexpr (RU == 0) {  // bf16(s U) of this tile's rows, written by the U pass
    const uint16_t* ug = tab.usg[gp];
    for (int e = tid; e < BT * (RE / 8); e += kThreads) {
      const int row = e / (RE / 8), c8 = 8 * (e - row * (RE / 8));
      uint4 v = {0u, 0u, 0u, 0u};
      if (c8 < r && m0 + row < T) v = *reinterpret_cast<const uint4*>(ug + static_cast<size_t>(m0 + row) * r + c8);
      *reinterpret_cast<uint4*>(us + ep(row, c8)) = v;
    }
  }
  for (int e = tid; e < BT * RE; e += kThreads) {
    const int j = e / BT, c = e % BT;
    bt[ep(c, j)] = (j < r && n0 + c < N) ? B[static_cast<size_t>(j) * N + n0 + c] : uint16_t(0);
  }
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < RE / 16; ++ks) {
    uint4 a[kFM], b[2];
#pragma unroll
    for (int i = 0; i < kFM; ++i)
      a[i] = *reinterpret_cast<const uint4*>(us + ep(wm * kHalf + blk(i) * 32 + l32, ks * 16 + lh * 8));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b[j] = *reinterpret_cast<const uint4*>(bt + ep(wn * 64 + j * 32 + l32, ks * 16 + lh * 8));
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
  }
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * kHalf + blk(i) * 32 + mfma32_row(e, lane);
        if (row < T && col < N) y[static_cast<size_t>(row) * N + col] = to_bf16(acc[i][j][e]);
      }
    }
}

template <int BT, int RU, int RE>
hipError_t launch_fwd_t(int T, int K, int r, float s, const uint16_t* x, const ProjTable& tab, int splits,
                        int steps_per, float* part, float* upart, bool dq, hipStream_t stream) {
  const int tiles = ((T + BT - 1) / BT) * tab.tile_end[tab.n - 1];
  if (dq)
    lora_fwd_kernel<BT, RU, RE, true><<<tiles * splits, FwdTile<BT>::kThreads, 0, stream>>>(
        T, K, r, s, x, tab, steps_per, part, upart);
  else
    lora_fwd_kernel<BT, RU, RE, false><<<tiles * splits, FwdTile<BT>::kThreads, 0, stream>>>(
        T, K, r, s, x, tab, steps_per, part, upart);
  return hipGetLastError();
}

template <int BT>
hipError_t launch_fwd_rank(int T, int K, int r, float s, const uint16_t* x, const ProjTable& tab, int splits,
                           int steps_per, float* part, float* upart, bool dq, hipStream_t stream) {
  switch ((r + 15) / 16) {
    case 1: return launch_fwd_t<BT, 16, 16>(T, K, r, s, x, tab, splits, steps_per, part, upart, dq, stream);
    case 2: return launch_fwd_t<BT, 32, 32>(T, K, r, s, x, tab, splits, steps_per, part, upart, dq, stream);
    case 3: return launch_fwd_t<BT, 64, 48>(T, K, r, s, x, tab, splits, steps_per, part, upart, dq, stream);
    default: return launch_fwd_t<BT, 64, 64>(T, K, r, s, x, tab, splits, steps_per, part, upart, dq, stream);
  }
}

// U = x A on its own, for the large-token forward at rank > 16 (the tile kernel
// then takes RU = 0 and reads bf16(s U) in its epilogue): the in-loop U is
// recomputed by every column tile, which at rank 32 / 64 costs 15 / 24 % of the
// loop. One workgroup per 32 token rows; wave w accumulates d_in quarter w with
// 32 x 32 x 16 MFMAs straight from global memory (x rows and rows of A^T, 16 bytes
// per lane), and wave 0 adds the four partials in a fixed order. Rows past T and
// rank rows past r lie outside the buffer ranges and read zeros.
template <int RU>
__global__ __launch_bounds__(256) void lora_u_pass_kernel(int T, int K, int r, float s,
                                                          const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ at,
                                                          uint16_t* __restrict__ us_out,
                                                          uint16_t* __restrict__ u_save) {
  constexpr int NU = RU / 32;
  __shared__ float red[3 * NU * 16 * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, lh = lane >> 5;
  const int m0 = blockIdx.x * 32;
  const int rows = min(T - m0, 32);
  const int kq = K / 4;  // d_in % 64 == 0: whole 16-wide slices per wave
  const auto rs_x = make_rsrc(x + static_cast<size_t>(m0) * K, static_cast<uint32_t>(rows) * K * 2);
  const auto rs_a = make_rsrc(at, static_cast<uint32_t>(r) * K * 2);
  const uint32_t xoff = static_cast<uint32_t>(l32) * K * 2 + (wave * kq + 8 * lh) * 2;
  uint32_t aoff[NU];
  f32x16_t acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    aoff[u] = static_cast<uint32_t>(u * 32 + l32) * K * 2 + (wave * kq + 8 * lh) * 2;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[u][e] = 0.f;
  }
#pragma unroll 8
  for (int k = 0; k < kq; k += 16) {
    const uint4 xa = buf_load16(rs_x, xoff, k * 2);
#pragma unroll
    for (int u = 0; u < NU; ++u) acc[u] = mfma32(xa, buf_load16(rs_a, aoff[u], k * 2), acc[u]);
  }
  if (wave > 0) {
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[(((wave - 1) * NU + u) * 16 + e) * 64 + lane] = acc[u][e];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float v = acc[u][e] + red[((0 * NU + u) * 16 + e) * 64 + lane] + red[((1 * NU + u) * 16 + e) * 64 + lane] +
                      red[((2 * NU + u) * 16 + e) * 64 + lane];
      const int row = m0 + mfma32_row(e, lane), col = u * 32 + l32;
      if (row < T && col < r) {
        us_out[static_cast<size_t>(row) * r + col] = to_bf16(s * v);
        if (u_save != nullptr) u_save[static_cast<size_t>(row) * r + col] = to_bf16(v);
      }
    }
}

// at [r][K] = A^T (A [K][r]), one element per thread.
__global__ __launch_bounds__(256) void transpose_a_kernel(const uint16_t* __restrict__ a, int K, int r,
                                                          uint16_t* __restrict__ at) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(K) * r) return;
  const int j = static_cast<int>(i / K), k = static_cast<int>(i - static_cast<int64_t>(j) * K);
  at[i] = a[static_cast<size_t>(k) * r + j];
}

hipError_t launch_u_pass(int T, int K, int r, float s, const uint16_t* x, const uint16_t* A, uint16_t* at,
                         uint16_t* us_out, uint16_t* u_save, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(K) * r;
  transpose_a_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(A, K, r, at);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned grid = static_cast<unsigned>((T + 31) / 32);
  if (r <= 32)
    lora_u_pass_kernel<32><<<grid, 256, 0, stream>>>(T, K, r, s, x, at, us_out, u_save);
  else
    lora_u_pass_kernel<64><<<grid, 256, 0, stream>>>(T, K, r, s, x, at, us_out, u_save);
  return hipGetLastError();
}

// The DQ tile kernel with U from the U pass (RU = 0), epilogue width by rank.
template <int BT>
hipError_t launch_fwd_ug(int T, int K, int r, float s, const uint16_t* x, const ProjTable& tab, hipStream_t stream) {
  const int tiles = ((T + BT - 1) / BT) * tab.tile_end[tab.n - 1];
  const int steps = K / BK;
  constexpr int kT = FwdTile<BT>::kThreads;
  switch ((r + 15) / 16) {
    case 2: lora_fwd_kernel<BT, 0, 32, true><<<tiles, kT, 0, stream>>>(T, K, r, s, x, tab, steps, nullptr, nullptr); break;
    case 3: lora_fwd_kernel<BT, 0, 48, true><<<tiles, kT, 0, stream>>>(T, K, r, s, x, tab, steps, nullptr, nullptr); break;
    default: lora_fwd_kernel<BT, 0, 64, true><<<tiles, kT, 0, stream>>>(T, K, r, s, x, tab, steps, nullptr, nullptr); break;
  }
  return hipGetLastError();
}

// Tile edge from a round count: a grid of 256 x 256 tiles runs in rounds of 256
// (one per CU), one of 128 x 128 tiles in rounds of 512 (two per CU; 256 at rank
// > 32, whose LDS allows one). Measured on MI355X (4096 -> 4096, 5120 -> 5120 and
// 8192 -> 28672, 64 to 8192 tokens), a full round of 128 tiles costs about 3/4 of
// a round of 256 tiles at rank <= 32 and 2/3 at rank 64, with the same outputs
// either way (each output accumulates in the same order).
int fwd_tile_edge(int64_t T, int cols256, int cols128, int r) {
  const int64_t rounds256 = ((T + 255) / 256 * cols256 + 255) / 256;
  const int slots128 = r <= 32 ? 512 : 256;
  const int64_t rounds128 = ((T + 127) / 128 * cols128 + slots128 - 1) / slots128;
  const bool small = r <= 32 ? 3 * rounds128 < 4 * rounds256 : 2 * rounds128 < 3 * rounds256;
  return small ? 128 : 256;
}

// K-splits of the tiled forward of one projection. The split costs a pass over
// S T N fp32 partials plus the reduce's rereads of B, so it pays where the tile
// grid leaves most resident slots idle (128 x 128 tiles: two per CU at rank <=
// 32): filling at most 32 % of them, or 50 % when the main loop dominates (rank
// > 32, or d_in >= 16384). Measured on MI355X at 160 .. 2048 tokens over q_proj,
// Qwen-14B, the 70B gate and down and k/v shapes, the rule splits exactly where
// splitting was faster. From 4096 tokens nothing splits: the partials grow with T
// while the unsplit dequantize-then-GEMM path runs at the same speed (k/v at rank
// 64, 8192 tokens: 157 us split, 149 us unsplit), and unsplit projections can share
// one multi-projection launch (q/k/v: 650 -> 500 us). S fills the slots, at most
// four ways and at least eight 64-element steps per split (1 = no split).
struct TiledSplit {
  int bt, splits, steps_per;
};
TiledSplit tiled_split(int64_t T, int64_t K, int64_t N, int r) {
  TiledSplit p{};
  p.bt = fwd_tile_edge(T, static_cast<int>((N + 255) / 256), static_cast<int>((N + 127) / 128), r);
  const int64_t tiles = (T + p.bt - 1) / p.bt * ((N + p.bt - 1) / p.bt);
  const int64_t slots = 256 * (p.bt == 128 && r <= 32 ? 2 : 1);
  const int KB = static_cast<int>(K / BK);
  const bool long_main = r > 32 || K >= 16384;
  const bool idle = 100 * tiles <= 32 * slots || (long_main && 2 * tiles <= slots);
  int S = static_cast<int>(slots / tiles);
  S = S > 4 ? 4 : S;
  S = S > KB / 8 ? KB / 8 : S;
  S = idle && S >= 2 && T < 4096 ? S : 1;
  p.steps_per = (KB + S - 1) / S;
  p.splits = (KB + p.steps_per - 1) / p.steps_per;  // every split non-empty
  return p;
}

// Dequantize-then-GEMM: the in-loop dequantization is repeated by every token tile
// (T / tile edge times per weight element). Once there are enough of them,
// dequantizing the whole weight once into the workspace (bf16 [N][K], one pass at
// HBM speed: 2.56 bytes per weight) and staging bf16 tiles like x costs less: from
// 8 token tiles of 128 rows (T >= 1024) or 16 of 256 rows (T >= 4096). Measured on
// MI355X: 4096 -> 4096 at 8192 tokens 295 -> 261 us, at 1024 tokens (128-row
// tiles) 71 -> 65 us; the 70B gate at 1024 tokens (4 tiles of 256 rows) runs
// 15 % faster in-loop (586 -> 496 us), and 256-row grids at 2048 tokens are within
// +-5 % either way. Same values: the dequantization rounds exactly as the in-loop
// one.
// Taken only with weight staging on (lora_nf4_set_weight_staging).
bool fwd_dq(int64_t T, int bt) { return weight_staging() && T >= (bt == 256 ? 4096 : 1024); }
// Rank > 16 on that path from 4096 tokens also takes the U pass (A^T [r][K] and
// bf16(s U) [T][r] follow each projection's weight in the workspace). Measured on
// MI355X, forward at 8192 tokens, in-loop U -> U pass: 4096 -> 4096 r = 32
// 288 -> 270 us, r = 64 338 -> 290 us; 4096 -> 14336 r = 64 1172 -> 925 us;
// 4096 -> 1024 r = 64 145 -> 134 us. At 2048 tokens it is even and at 1024 slower
// (72 -> 84 us at r = 32): the U pass runs T / 32 workgroups.
bool fwd_ug(int64_t T, int r) { return r > 16 && T >= 4096; }
size_t dq_bytes(int64_t T, int64_t K, int64_t N, int r) {
  const auto al = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
  size_t b = al(static_cast<size_t>(N) * K * 2);
  if (fwd_ug(T, r)) b += al(static_cast<size_t>(r) * K * 2) + al(static_cast<size_t>(T) * r * 2);
  return b;
}

// From 4096 tokens on 256 x 256 tiles the register-dequantizing kernel
// (lora_fwd_rw.hip) replaces dequantize-then-GEMM: the weight stays packed in HBM,
// each tile dequantizes its 256 x 64 block of a step once, into MFMA fragments.
// At rank 16 the kernel computes U = x A itself (no workspace). Otherwise U comes
// from the U pass (lora_upass.hip; A^T and bf16(s U) in the workspace): one pass
// over x for all projections when their ranks sum to at most 256, else one per
// projection.
bool fwd_rw(int64_t T, int64_t K, int bt, int r) { return !weight_staging() && bt == 256 && fwd_rw_supported(T, K, r); }
size_t rw_bytes(int64_t T, int64_t K, int n, int r) {
  if (fwd_rw_inloop_u(r)) return 0;
  return n * r <= 256 ? upass_table_bytes(T, K, n, r) : n * upass_table_bytes(T, K, 1, r);
}
hipError_t launch_rw_with_upass(int T, int K, int r, float s, const uint16_t* x, ProjTable& tab, void* workspace,
                                hipStream_t stream) {
  if (fwd_rw_inloop_u(r)) return launch_fwd_rw(T, K, r, s, x, tab, stream);
  unsigned char* w = static_cast<unsigned char*>(workspace);
  const int groups = tab.n * r <= 256 ? 1 : tab.n;  // U passes
  const int per = tab.n / groups;                   // projections per pass
  for (int p = 0; p < groups; ++p) {
    UpassTable ut{};
    ut.n = per;
    for (int g = 0; g < per; ++g) {
      ut.A[g] = tab.A[p * per + g];
      ut.u[g] = tab.u[p * per + g];
    }
    const hipError_t e = launch_upass(T, K, r, s, x, ut, w, stream);
    if (e != hipSuccess) return e;
    for (int g = 0; g < per; ++g) tab.usg[p * per + g] = ut.us + g * r;
    w += upass_table_bytes(T, K, per, r);
  }
  tab.us_stride = per * r;
  return launch_fwd_rw(T, K, r, s, x, tab, stream);
}

size_t tiled_split_bytes(int64_t T, int64_t N, int r, int splits) {
  if (splits <= 1) return 0;
  const size_t a = (static_cast<size_t>(splits) * T * N * 4 + 255) & ~static_cast<size_t>(255);
  return a + ((static_cast<size_t>(splits) * T * r * 4 + 255) & ~static_cast<size_t>(255));
}

// tab.N and the pointers are set; the column-tile prefix sums follow the tile edge.
// A single projection whose tile grid leaves CUs idle runs split (workspace).
hipError_t launch_fwd_table(int T, int K, int r, float s, const uint16_t* x, ProjTable& tab,
                            void* workspace, hipStream_t stream) {
  int cols256 = 0, cols128 = 0;
  for (int g = 0; g < tab.n; ++g) {
    cols256 += (tab.N[g] + 255) / 256;
    cols128 += (tab.N[g] + 127) / 128;
  }
  const int bt = fwd_tile_edge(T, cols256, cols128, r);
  int tiles = 0;
  for (int g = 0; g < tab.n; ++g) {
    tiles += (tab.N[g] + bt - 1) / bt;
    tab.tile_end[g] = tiles;
  }
  TiledSplit sp{bt, 1, K / BK};
  if (tab.n == 1 && workspace != nullptr) sp = tiled_split(T, K, tab.N[0], r);
  if (sp.splits == 1 && fwd_rw(T, K, bt, r)) return launch_rw_with_upass(T, K, r, s, x, tab, workspace, stream);
  // the weights of every projection dequantized one after another into the workspace
  const bool dq = workspace != nullptr && sp.splits == 1 && fwd_dq(T, bt);
  const bool ug = dq && fwd_ug(T, r);
  if (dq) {
    unsigned char* w = static_cast<unsigned char*>(workspace);
    for (int g = 0; g < tab.n; ++g) {
      hipError_t e = launch_nf4_dequantize(tab.codes[g], tab.absmax[g], tab.N[g], K, true, w, stream);
      if (e != hipSuccess) return e;
      tab.wdq[g] = reinterpret_cast<const uint16_t*>(w);
      if (ug) {
        uint16_t* at = reinterpret_cast<uint16_t*>(w + ((static_cast<size_t>(tab.N[g]) * K * 2 + 255) & ~size_t(255)));
        uint16_t* usg = at + (((static_cast<size_t>(r) * K * 2 + 255) & ~size_t(255)) / 2);
        e = launch_u_pass(T, K, r, s, x, tab.A[g], at, usg, tab.u[g], stream);
        if (e != hipSuccess) return e;
        tab.usg[g] = usg;
      }
      w += dq_bytes(T, K, tab.N[g], r);
    }
  }
  if (ug) return bt == 256 ? launch_fwd_ug<256>(T, K, r, s, x, tab, stream) : launch_fwd_ug<128>(T, K, r, s, x, tab, stream);
  float* part = nullptr;
  float* upart = nullptr;
  if (sp.splits > 1) {
    part = static_cast<float*>(workspace);
    upart = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) +
                                     ((static_cast<size_t>(sp.splits) * T * tab.N[0] * 4 + 255) & ~static_cast<size_t>(255)));
  }
  const hipError_t e =
      bt == 256 ? launch_fwd_rank<256>(T, K, r, s, x, tab, sp.splits, sp.steps_per, part, upart, dq, stream)
                : launch_fwd_rank<128>(T, K, r, s, x, tab, sp.splits, sp.steps_per, part, upart, dq, stream);
  if (e != hipSuccess || sp.splits <= 1) return e;
  return launch_fwd_splitk_reduce(T, tab.N[0], r, sp.splits, s, part, upart, tab.B[0], tab.y[0], tab.u[0], stream);
}

}  // namespace

namespace {
// Few tokens: the one-launch weight-streaming kernel when its 16-row workgroups
// fit one round of the CUs (T <= 32, d_out <= 4096), else the split-K kernel and
// its reduce (measured on MI355X: the reduce costs a few microseconds of latency,
// which one round of streaming workgroups beats).
bool fwd_uses_splitk(int64_t T, int64_t K, int64_t N, int r) {
  if (r % 8 != 0 || r > 64 || !fits_buffer(T, K, N) || !lora_fwd_splitk_supported(T, r)) return false;
  return !(lora_fwd_stream_supported(T, r) && (N + 15) / 16 <= 256);
}
// One launch for several projections unless one of them would run a path of its
// own (few tokens, or a K-split tiled forward): the fused launch then gives the
// same values as separate calls, in the same summation order.
bool fwd_multi_tiled(int64_t T, int64_t K, int n_proj, const int* N, int r) {
  bool tiled = r % 8 == 0 && r <= 64 && n_proj <= kMaxProj && !lora_fwd_stream_supported(T, r);
  for (int g = 0; g < n_proj; ++g)
    tiled = tiled && fits_buffer(T, K, N[g]) && !fwd_uses_splitk(T, K, N[g], r) &&
            tiled_split(T, K, N[g], r).splits == 1;
  return tiled;
}
}  // namespace

size_t fwd_workspace_bytes(int64_t T, int64_t K, int64_t N, int r) {
  if (fwd_uses_splitk(T, K, N, r))
    return plan_fwd_splitk(static_cast<int>(T), static_cast<int>(K), static_cast<int>(N), r).bytes;
  if (r % 8 != 0 || r > 64 || !fits_buffer(T, K, N) || lora_fwd_stream_supported(T, r)) return 0;
  const TiledSplit ts = tiled_split(T, K, N, r);
  if (ts.splits == 1 && fwd_rw(T, K, ts.bt, r)) return rw_bytes(T, K, 1, r);
  if (ts.splits == 1 && fwd_dq(T, ts.bt)) return dq_bytes(T, K, N, r);
  return tiled_split_bytes(T, N, r, ts.splits);
}

// Tile edge of one launch over several projections (their column tiles form one
// grid), as launch_fwd_table chooses it.
int table_edge(int64_t T, int n_proj, const int* N, int r) {
  int cols256 = 0, cols128 = 0;
  for (int g = 0; g < n_proj; ++g) {
    cols256 += (N[g] + 255) / 256;
    cols128 += (N[g] + 127) / 128;
  }
  return fwd_tile_edge(T, cols256, cols128, r);
}

size_t fwd_multi_workspace_bytes(int64_t T, int64_t K, int n_proj, const int* N, int r) {
  if (fwd_multi_tiled(T, K, n_proj, N, r)) {
    if (fwd_rw(T, K, table_edge(T, n_proj, N, r), r)) return rw_bytes(T, K, n_proj, r);
    size_t b = 0;
    for (int g = 0; fwd_dq(T, table_edge(T, n_proj, N, r)) && g < n_proj; ++g) b += dq_bytes(T, K, N[g], r);
    return b;
  }
  size_t b = 0;
  for (int g = 0; g < n_proj; ++g) {
    const size_t bg = fwd_workspace_bytes(T, K, N[g], r);
    b = bg > b ? bg : b;
  }
  return b;
}

hipError_t launch_lora_fwd(int T, int K, int N, int r, float s, const uint16_t* x,
                           const uint8_t* codes, const float* absmax, const uint16_t* A,
                           const uint16_t* B, uint16_t* y, uint16_t* u_save, void* workspace,
                           hipStream_t stream) {
  if (r % 8 != 0 || r > 64 || !fits_buffer(T, K, N))
    return launch_lora_fwd_generic(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
  if (fwd_uses_splitk(T, K, N, r))
    return launch_lora_fwd_splitk(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, workspace, stream);
  if (lora_fwd_stream_supported(T, r))
    return launch_lora_fwd_stream(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
  ProjTable tab{};
  tab.n = 1;
  tab.N[0] = N;
  tab.codes[0] = codes;
  tab.absmax[0] = absmax;
  tab.A[0] = A;
  tab.B[0] = B;
  tab.y[0] = y;
  tab.u[0] = u_save;
  return launch_fwd_table(T, K, r, s, x, tab, workspace, stream);
}

hipError_t launch_lora_fwd_multi(int T, int K, int n_proj, const int* N, int r, float s,
                                 const uint16_t* x, const uint8_t* const* codes,
                                 const float* const* absmax, const uint16_t* const* A,
                                 const uint16_t* const* B, uint16_t* const* y,
                                 uint16_t* const* u_save, void* workspace, hipStream_t stream) {
  if (!fwd_multi_tiled(T, K, n_proj, N, r)) {  // each projection on its own path
    for (int g = 0; g < n_proj; ++g) {
      const hipError_t e = launch_lora_fwd(T, K, N[g], r, s, x, codes[g], absmax[g], A[g], B[g], y[g],
                                           u_save == nullptr ? nullptr : u_save[g], workspace, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  ProjTable tab{};
  tab.n = n_proj;
  for (int g = 0; g < n_proj; ++g) {
    tab.N[g] = N[g];
    tab.codes[g] = codes[g];
    tab.absmax[g] = absmax[g];
    tab.A[g] = A[g];
    tab.B[g] = B[g];
    tab.y[g] = y[g];
    tab.u[g] = u_save == nullptr ? nullptr : u_save[g];
  }
  const int bt = table_edge(T, n_proj, N, r);
  return launch_fwd_table(T, K, r, s, x, tab, fwd_rw(T, K, bt, r) || fwd_dq(T, bt) ? workspace : nullptr, stream);
}

}  // namespace lnf4
