// Fused NF4-LoRA linear, backward input gradient (gfx950):
//     G  = s dY B^T                      (bf16, also written out for dA)
//     dX = dY deq(Wt) + G A^T
// The pages replace autograd with hand-written backward kernels ("Unlocking AI
// potential: Unsloth's algorithms and implementation", core-algorithms section).
//
// Work decomposition mirrors the forward kernel: 256 x 256 dX tile (tokens x
// d_in) per 512-thread workgroup, 8 waves of 128 x 64, v_mfma_f32_32x32x16_bf16,
// reduction over d_out in steps of 64; or, when those tiles would leave CUs idle,
// 128 x 128 tiles per 256-thread workgroup (4 waves of 64 x 64), half the LDS.
// The base weight is used transposed here (the reduction runs along its rows), so
// its 64 x BT tile is dequantized into
// LDS in its natural row-major orientation with 16-byte stores and read back with
// ds_read_b64_tr_b16, which hands each lane a column of four consecutive rows:
// exactly the MFMA B fragment. The same dY tile accumulates G = s dY B^T for the
// epilogue (16 x 16 x 32 MFMAs for r <= 16, else 32 x 32 x 16), which adds G A^T
// with one more MFMA pass over the rank.
//
// Several projections of one input (q/k/v, gate/up) sum their input gradients:
//     dX = sum_g (dY_g D_g + G_g A_g^T),   G_g = s dY_g B_g^T.
// The reduction then runs over the concatenated d_out of all projections (the
// table switches the dY, weight and B operands at each projection's first step).
// At the end of a projection's steps its G_g is flushed, bf16, into columns
// g r .. g r + r - 1 of g_out [T][n r] and the accumulator restarts; every
// column tile writes the same bits there. The epilogue reads the tile's rows back
// and adds [G_0 .. G_n-1] [A_0 .. A_n-1]^T in one MFMA pass over n r.
//
// DQ instances: at large token counts each weight tile is read by many token
// tiles, so the weight is dequantized once beforehand into bf16 [N][K] (the same
// bf16(level x absmax) values) and the kernel loads its 64 x BT tiles straight
// into LDS like the dY tiles, unpadded: the 16-byte piece p of row n sits at
// piece p ^ 4 (n & 3), which keeps the four rows of a transposing read on
// distinct banks. The arithmetic, and so every output bit, is the same.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int BK = 64;
// Row n of the dequantized weight tile starts at n kDStride + dshift(n). The row
// stride (BT + 32 bf16) is 64 bytes past a multiple of 256, so the four rows of
// one transposing read, and the two column halves a 32-lane group reads, fall on
// distinct banks; rows four apart are shifted by 16 bytes per group of four,
// which spreads the 16-byte dequantization stores of a 16-lane group over all 64
// banks.
__device__ __forceinline__ int dshift(int n) { return 8 * ((n >> 2) & 3); }
constexpr int kBStride = 72;  // B slice rows: 64 bf16 + 16 B pad

// Square dX tile of edge BT (256 or 128): 2 x (BT / 64) waves, each owning
// BT / 2 token rows x 64 d_in columns.
template <int BT>
struct DxTile {
  static constexpr int kThreads = 2 * BT;
  static constexpr int kWN = BT / 64;         // waves along d_in
  static constexpr int kFM = BT / 64;         // 32-row fragments per wave along tokens
  static constexpr int kTileElems = BT * 64;  // dY tile [BT][64]
  static constexpr int kDStride = BT + 32;    // deq weight tile rows
  static constexpr int kDElems = 64 * kDStride;
  static constexpr int kRuns = BT / 32;       // 32-column runs of one weight row
  static constexpr int kMinBlocks = BT == 128 ? 2 : 1;
};

// RU = 0: G is already in g_out (the G pass); the K loop forms dY deq(W) alone and
// the epilogue reads G back.
// Split mode (part_x != nullptr, one projection): workgroup b runs tile b % tiles
// over d_out steps [steps_per (b / tiles), ...) and writes fp32 partial dX to
// part_x [split][T][K] and, from the first column tile, fp32 partial dY B^T to
// part_g [split][T][r]; no epilogue.
template <int BT, int RU, int RE, bool MULTI, bool DQ>
__global__ __launch_bounds__(DxTile<BT>::kThreads, DxTile<BT>::kMinBlocks) void lora_dx_kernel(
    int T, int K, int r, float s, const DxTable tab, uint16_t* __restrict__ dx,
    uint16_t* __restrict__ g_out, int steps_per, float* __restrict__ part_x, float* __restrict__ part_g) {
  using Tl = DxTile<BT>;
  constexpr int kThreads = Tl::kThreads, BM = BT, BN = BT, kFM = Tl::kFM, kHalf = BT / 2;
  constexpr int kTileElems = Tl::kTileElems, kDStride = Tl::kDStride;
  constexpr int kDElems = DQ ? 64 * BT : Tl::kDElems;  // DQ: unpadded [64][BT]
  __shared__ __align__(1024) float lut[16];  // first in LDS: level addresses need no base
  __shared__ __align__(16) uint16_t ys0[kTileElems];
  __shared__ __align__(16) uint16_t ys1[kTileElems];
  __shared__ __align__(16) uint16_t ds0[kDElems];
  __shared__ __align__(16) uint16_t ds1[kDElems];
  __shared__ __align__(16) uint16_t bs0[(RU > 0 ? RU : 1) * kBStride];
  __shared__ __align__(16) uint16_t bs1[(RU > 0 ? RU : 1) * kBStride];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Tl::kWN, wn = wave % Tl::kWN;  // 2 x kWN waves, BT / 2 x 64 each
  const int l32 = lane & 31, lh = lane >> 5;
  const int mt = (T + BM - 1) / BM, kt_tiles = (K + BN - 1) / BN;
  const int tiles = mt * kt_tiles;
  const int tile_id = blockIdx.x % tiles, sp = blockIdx.x / tiles;
  int tm, tk;
  tile_coords(xcd_remap(tile_id, tiles), mt, kt_tiles, 4, tm, tk);
  const int m0 = tm * BM, k0 = tk * BN;
  const int K2 = K / 2, KB = K / 64;
  const int NS_all = tab.step_end[tab.n - 1];  // reduction steps over all d_out
  const int sbeg = sp * steps_per;              // this workgroup's first step (0 unless split)
  const int NS = min(NS_all, sbeg + steps_per);  // one past its last step
  const int R = tab.n * r;  // g_out row length

  if (tid < 16) lut[tid] = nf4_level_reg(tid);

  // ---- buffer resources: out-of-range loads return zeros ------------------------
  // Every load takes a descriptor whose base is advanced to its step by scalar
  // arithmetic (scalar offset 0), and whose byte count ends with its operand's
  // range for this tile: the lane offset holds only the position within the step,
  // so rows past T or d_out lie past the range and read zeros, and no load reaches
  // past its operand. Step indices are clamped to the projection's last step, so
  // the run-ahead loads past the end re-read that step (unused).
  // Several projections: each load stream (dY one step ahead; codes, absmax and
  // B two steps ahead) keeps its projection's bases and offsets in registers and
  // moves to the next projection when its step crosses a boundary (steps advance
  // by one, every projection has at least one), so the loop reads the table only
  // at those crossings. Steps past the end stay in the last projection.
  const int rows_t = min(T - m0, BM);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // dY: wave w fills rows 32 w .. 32 w + 31 of the [BT][64] tile, swizzled
  const int N0 = tab.N[0];
  uint32_t yvoff[4];
  auto set_yvoff = [&](int Ng) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = (wave * 4 + q) * 8 + (lane >> 3);
      yvoff[q] = static_cast<uint32_t>(row) * Ng * 2 + ((lane & 7) ^ ((row >> 1) & 7)) * 16;
    }
  };
  set_yvoff(N0);
  const uint16_t* y_ptr = tab.dy[0] + static_cast<size_t>(m0) * N0;
  uint32_t y_bytes = static_cast<uint32_t>(rows_t) * N0 * 2;
  // DQ weight tile: wave w fills 1 KB pieces 4 w .. 4 w + 3 of the [64][BT] stage;
  // lane l of piece c lands at element 512 c + 8 l (row n, 16-byte piece p') and
  // loads piece p' ^ 4 (n & 3) of that weight row. Rows past d_out lie outside the
  // range and read zeros; columns past d_in only reach dX columns that are not stored.
  uint32_t wvoff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = (wave * 4 + q) * 512 + lane * 8, n = e / BT, pp = (e % BT) / 8;
    wvoff[q] = static_cast<uint32_t>(n) * K * 2 + ((pp ^ (4 * (n & 3))) * 16);
  }
  const uint16_t* w_ptr = DQ ? tab.wdq[0] + k0 : nullptr;
  uint32_t w_bytes = DQ ? static_cast<uint32_t>((static_cast<size_t>(N0) * K - k0) * 2) : 0u;
  int y_g = 0, y_beg = 0, y_end = tab.step_end[0], y_N = N0;
  int y_ls = 0;  // the clamped step (within its projection) of the last load_y_lds
  auto load_y_lds = [&](int st, uint16_t* stage) {
    if constexpr (MULTI) {
      if (st >= y_end && y_g + 1 < tab.n) {
        ++y_g;
        y_beg = y_end;
        y_end = tab.step_end[y_g];
        y_N = tab.N[y_g];
        y_ptr = tab.dy[y_g] + static_cast<size_t>(m0) * y_N;
        y_bytes = static_cast<uint32_t>(rows_t) * y_N * 2;
        set_yvoff(y_N);
        if constexpr (DQ) {
          w_ptr = tab.wdq[y_g] + k0;
          w_bytes = static_cast<uint32_t>((static_cast<size_t>(y_N) * K - k0) * 2);
        }
      }
    }
    y_ls = min(st, y_end - 1) - y_beg;
    const auto rs_y = make_rsrc(y_ptr + y_ls * BK, y_bytes - y_ls * BK * 2);
    // On the step with d_out's last columns, chunks past d_out read the next row's
    // dY (the tile's last row reads zeros there): they meet weight rows past d_out,
    // which read zeros, so they add nothing (a non-finite value there could only
    // reach a dX that already holds the non-finite products of its own row).
#pragma unroll
    for (int q = 0; q < 4; ++q) buf_load16_lds(rs_y, stage + (wave_u * 4 + q) * 512, yvoff[q], 0);
  };
  // the weight tile of the step load_y_lds was last called with
  auto load_w_lds = [&](uint16_t* stage) {
    const auto rs_w = make_rsrc(w_ptr + static_cast<size_t>(y_ls) * BK * K,
                                w_bytes - static_cast<uint32_t>(y_ls) * BK * K * 2);
#pragma unroll
    for (int q = 0; q < 4; ++q) buf_load16_lds(rs_w, stage + (wave_u * 4 + q) * 512, wvoff[q], 0);
  };
  // weight codes: one of the 64 rows of the step, 32 columns (one half of an NF4
  // block) at one of the BT / 32 runs of the tile. Thread bits, 256 x 256 tiles:
  // [1:0] low run, [3:2] low row group, [4] high run, [6:5] high row group, [8:7]
  // row within the group of four; 128 x 128 tiles: [1:0] run, [3:2] low row
  // group, [5:4] high row group, [7:6] row within the group. Each 16 lanes then
  // store to distinct banks.
  const int run = BT == 256 ? (tid & 3) | (((tid >> 4) & 1) << 2) : (tid & 3);
  const int nl = BT == 256 ? 4 * (((tid >> 2) & 3) | (((tid >> 5) & 3) << 2)) + ((tid >> 7) & 3)
                           : 4 * (((tid >> 2) & 3) | (((tid >> 4) & 3) << 2)) + ((tid >> 6) & 3);
  const uint32_t cvoff = static_cast<uint32_t>(nl) * K2 + run * 16;
  const uint32_t svoff = (static_cast<uint32_t>(nl) * KB + (run >> 1)) * 4;
  // B slice: row j = tid >> 3 (+ kThreads / 8 per further load, < RU), 8 columns
  // at chunk tid & 7; columns past d_out are zeroed here (rows past r read zeros)
  constexpr int kBPer = (RU * 8 + kThreads - 1) / kThreads;
  const int bj = tid >> 3, bch = tid & 7;
  uint4 creg[2], breg[2][kBPer > 0 ? kBPer : 1];
  float sreg[2];
  // 2 + kBPer loads per thread and step, so every wave can wait on the same vmcnt.
  const uint8_t* c_ptr = tab.codes[0] + k0 / 2;
  uint32_t c_bytes = static_cast<uint32_t>(static_cast<size_t>(N0) * K2 - k0 / 2);
  const float* s_ptr = tab.absmax[0] + k0 / 64;
  uint32_t s_bytes = static_cast<uint32_t>((static_cast<size_t>(N0) * KB - k0 / 64) * 4);
  const uint16_t* b_ptr = tab.B[0];
  uint32_t b_bytes = static_cast<uint32_t>(r) * N0 * 2;
  uint32_t bvoff = static_cast<uint32_t>(bj) * N0 * 2 + bch * 16;
  int w_g = 0, w_beg = 0, w_end = tab.step_end[0], w_N = N0;
  auto load_regs = [&](int st, int slot) {
    if constexpr (MULTI) {
      if (st >= w_end && w_g + 1 < tab.n) {
        ++w_g;
        w_beg = w_end;
        w_end = tab.step_end[w_g];
        w_N = tab.N[w_g];
        if constexpr (!DQ) {
          c_ptr = tab.codes[w_g] + k0 / 2;
          c_bytes = static_cast<uint32_t>(static_cast<size_t>(w_N) * K2 - k0 / 2);
          s_ptr = tab.absmax[w_g] + k0 / 64;
          s_bytes = static_cast<uint32_t>((static_cast<size_t>(w_N) * KB - k0 / 64) * 4);
        }
        b_ptr = tab.B[w_g];
        b_bytes = static_cast<uint32_t>(r) * w_N * 2;
        bvoff = static_cast<uint32_t>(bj) * w_N * 2 + bch * 16;
      }
    }
    const int ls = min(st, w_end - 1) - w_beg;
    if constexpr (!DQ) {
      const uint32_t cstep = static_cast<uint32_t>(ls) * 64 * K2, sstep = static_cast<uint32_t>(ls) * 64 * KB;
      creg[slot] = buf_load16(make_rsrc(c_ptr + cstep, c_bytes - cstep), cvoff, 0);
      sreg[slot] = __uint_as_float(buf_load4(make_rsrc(s_ptr + sstep, s_bytes - sstep * 4), svoff, 0));
    }
    const auto rs_b = make_rsrc(b_ptr + ls * BK, b_bytes - ls * BK * 2);
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const uint4 v = buf_load16(rs_b, bvoff + i * (kThreads / 8) * w_N * 2, 0);
      breg[slot][i] = (ls * BK + bch * 8 < w_N) ? v : uint4{0u, 0u, 0u, 0u};
    }
  };

  const int fkey = (l32 >> 1) & 7;
  int choff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) choff[ks] = ((2 * ks + lh) ^ fkey) << 3;
  const int a_off = (wm * kHalf + l32) * 64;  // + i * 2048
  const int ga_off = a_off + wn * 2048;     // this wave's 32 rows of G
  // transposed weight fragment: 16-lane group g, lane m within it
  const int g16 = lane >> 4, m16 = lane & 15;
  // rows 8 (g16 >> 1) + (m16 >> 2) (+ 4 for the second read): row groups 2 (g16 >> 1)
  // and 2 (g16 >> 1) + 1, so the second read sits one group shift further
  const int d_off = ((g16 >> 1) * 8 + (m16 >> 2)) * kDStride + dshift((g16 >> 1) * 8) + wn * 64 +
                    (g16 & 1) * 16 + 4 * (m16 & 3);
  // DQ layout: the same rows and columns, column half j at its swizzled piece
  int dq_off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    dq_off[j] = ((g16 >> 1) * 8 + (m16 >> 2)) * BT +
                (((wn * 8 + j * 4 + (g16 & 1) * 2 + ((m16 & 3) >> 1)) ^ (4 * (m16 >> 2))) * 8) + 4 * (m16 & 1);
  const int gb_off = l32 * kBStride + lh * 8;  // + u * 32 * kBStride + ks * 16
  // r <= 16: 16 x 16 x 32 fragments of G rows wm * BT / 2 + wn * 32 + 16 rb + (lane & 15)
  constexpr bool kG16 = RU == 16;
  const int l16 = lane & 15, lq = lane >> 4;
  const int ga16_off = (wm * kHalf + wn * 32 + l16) * 64;  // + rb * 1024
  int choff16[2];
#pragma unroll
  for (int kq = 0; kq < 2; ++kq) choff16[kq] = ((4 * kq + lq) ^ (l16 >> 1)) << 3;
  const int gb16_off = l16 * kBStride + 8 * lq;         // + kq * 32

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
  const int dw_off = nl * kDStride + dshift(nl) + run * 32;  // + q * 8
  auto store_b = [&](uint16_t* bs, const uint4* v) {
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int j = bj + i * (kThreads / 8);
      if (j < RU) *reinterpret_cast<uint4*>(bs + j * kBStride + bch * 8) = v[i];
    }
  };

  f32x16_t acc[kFM][2];
  f32x16_t gacc[RU / 32 > 0 ? RU / 32 : 1];
  f32x4_t gacc16[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
#pragma unroll
  for (int u = 0; u < RU / 32; ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) gacc[u][e] = 0.f;

  // prologue: step 0 into stage 0, step 1 into registers
  load_y_lds(sbeg, ys0);
  if constexpr (DQ) load_w_lds(ds0);
  load_regs(sbeg, 0);
  wait_vmem();
  __syncthreads();  // lut and dY of step 0 visible
  {
    if constexpr (!DQ) {
      const uint32_t cw[4] = {creg[0].x, creg[0].y, creg[0].z, creg[0].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float lv[8];
        lookup(cw[q], lv);
        finish_store(lv, sreg[0], ds0 + dw_off + q * 8);
      }
    }
    store_b(bs0, breg[0]);
  }
  load_regs(sbeg + 1, 1);
  __syncthreads();

  struct Frag {
    uint4 a[kFM], b[2], ga, gb[RU / 32 > 0 ? RU / 32 : 1], ga16[2], gb16;
  };
  auto kstep = [&](int st, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr int nslot = cur ^ 1;
    const uint16_t* yc = cur ? ys1 : ys0;
    const uint16_t* dc = cur ? ds1 : ds0;
    const uint16_t* bc = cur ? bs1 : bs0;
    uint16_t* yn = cur ? ys0 : ys1;
    uint16_t* dn = cur ? ds0 : ds1;
    uint16_t* bn = cur ? bs0 : bs1;
    load_y_lds(st + 1, yn);
    if constexpr (DQ) load_w_lds(dn);
    load_regs(st + 2, cur);
    // DQ: keep the next stage's loads at the top of the step
    if constexpr (DQ) __builtin_amdgcn_sched_barrier(0);
    const uint32_t cw[4] = {creg[nslot].x, creg[nslot].y, creg[nslot].z, creg[nslot].w};
    const float ar = sreg[nslot];
    auto read_frag = [&](Frag& f, int ks) {
#pragma unroll
      for (int i = 0; i < kFM; ++i) f.a[i] = *reinterpret_cast<const uint4*>(yc + a_off + i * 2048 + choff[ks]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (DQ) {
          const uint16_t* p = dc + dq_off[j] + ks * 16 * BT;
          const uint2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 4 * BT);
          f.b[j] = uint4{lo.x, lo.y, hi.x, hi.y};
        } else {
          const uint16_t* p = dc + d_off + ks * 16 * kDStride + j * 32;
          const uint2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 4 * kDStride + 8);
          f.b[j] = uint4{lo.x, lo.y, hi.x, hi.y};
        }
      }
      if constexpr (kG16) {
        if (ks & 1) {  // one 32-wide k-slice of G per two 16-wide MFMA slices
          f.ga16[0] = *reinterpret_cast<const uint4*>(yc + ga16_off + choff16[ks >> 1]);
          f.ga16[1] = *reinterpret_cast<const uint4*>(yc + ga16_off + 1024 + choff16[ks >> 1]);
          f.gb16 = *reinterpret_cast<const uint4*>(bc + gb16_off + (ks >> 1) * 32);
        }
      } else {
        f.ga = *reinterpret_cast<const uint4*>(yc + ga_off + choff[ks]);
#pragma unroll
        for (int u = 0; u < RU / 32; ++u)
          f.gb[u] = *reinterpret_cast<const uint4*>(bc + gb_off + u * 32 * kBStride + ks * 16);
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
      if constexpr (kG16) {
        if (ks & 1) {
          gacc16[0] = mfma16(f.ga16[0], f.gb16, gacc16[0]);
          gacc16[1] = mfma16(f.ga16[1], f.gb16, gacc16[1]);
        }
      } else {
#pragma unroll
        for (int u = 0; u < RU / 32; ++u) gacc[u] = mfma32(f.ga, f.gb[u], gacc[u]);
      }
      if constexpr (!DQ) finish_store(lv[ks & 1], ar, dn + dw_off + ks * 8);
      if (ks == 3) store_b(bn, breg[nslot]);
    }
    // dY (and the DQ weight) of the next stage has landed (the step st + 2 register
    // loads issued after it may still be in flight)
    wait_vmem_upto<(DQ ? 0 : 2) + kBPer>();
    __syncthreads();
  };
  // Several projections: at the end of projection g's steps, store bf16(s G_g)
  // for this wave's rows into g_out columns g r .. and restart the accumulator.
  // The lane's first row is made opaque here and every other row is that plus a
  // constant times R (uniform): otherwise the compiler hoists the 32 loop-invariant
  // row addresses out of the K-loop and keeps them live through it (spills).
  int gseg = 0, gend = tab.step_end[0];
  auto flush = [&](int st) {
    if constexpr (!MULTI) return;
    if (st + 1 != gend) return;
    const size_t col0 = static_cast<size_t>(gseg) * r;
    if constexpr (RU / 32 > 0) {
      int lrow = m0 + wm * kHalf + wn * 32 + 4 * lh;  // row of element 0 of this lane
      asm volatile("" : "+v"(lrow));
      uint16_t* gp = g_out + static_cast<size_t>(lrow) * R + col0 + l32;
#pragma unroll
      for (int u = 0; u < RU / 32; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int dr = 8 * (e >> 2) + (e & 3);  // mfma32_row(e, lane) - 4 (lane >> 5)
          if (u * 32 + l32 < r && lrow + dr < T) gp[static_cast<size_t>(dr) * R + u * 32] = to_bf16(s * gacc[u][e]);
          gacc[u][e] = 0.f;
        }
    }
    if constexpr (kG16) {
      int lrow = m0 + wm * kHalf + wn * 32 + 4 * lq;
      asm volatile("" : "+v"(lrow));
      uint16_t* gp = g_out + static_cast<size_t>(lrow) * R + col0 + l16;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int dr = rb * 16 + e;
          if (l16 < r && lrow + dr < T) gp[static_cast<size_t>(dr) * R] = to_bf16(s * gacc16[rb][e]);
          gacc16[rb][e] = 0.f;
        }
    }
    ++gseg;
    if (gseg < tab.n) gend = tab.step_end[gseg];
  };
  for (int st = sbeg; st < NS; st += 2) {
    kstep(st, std::integral_constant<int, 0>{});
    flush(st);
    if (st + 1 < NS) {
      kstep(st + 1, std::integral_constant<int, 1>{});
      flush(st + 1);
    }
  }

  if (part_x != nullptr) {  // split mode: fp32 partials, no epilogue
    wait_vmem();            // run-ahead loads land before the workgroup ends
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = k0 + wn * 64 + j * 32 + l32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + wm * kHalf + i * 32 + mfma32_row(e, lane);
          if (row < T && col < K) part_x[(static_cast<size_t>(sp) * T + row) * K + col] = acc[i][j][e];
        }
      }
    if (tk != 0) return;
    float* gd = part_g + static_cast<size_t>(sp) * T * r;
#pragma unroll
    for (int u = 0; u < RU / 32; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * kHalf + wn * 32 + mfma32_row(e, lane), col = u * 32 + l32;
        if (col < r && row < T) gd[static_cast<size_t>(row) * r + col] = gacc[u][e];
      }
    if constexpr (kG16) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + wm * kHalf + wn * 32 + rb * 16 + 4 * lq + e;
          if (l16 < r && row < T) gd[static_cast<size_t>(row) * r + l16] = gacc16[rb][e];
        }
    }
    return;
  }

  // ---- epilogue: acc += bf16(G) A^T ----------------------------------------------
  constexpr int ES = RE + 8;
  constexpr bool kPad = BT * ES <= kTileElems;
  auto ep = [](int row, int col) {
    if constexpr (kPad) return row * ES + col;
    else return swz64(row, col >> 3) + (col & 7);
  };
  uint16_t* gs = ys0;  // [BT][RE] bf16(G), G = s dY B^T (projections side by side)
  uint16_t* at = ys1;  // [BT][RE] rows k of A (A is [d_in, r] row-major), projections side by side
  // one MFMA pass over RE rank columns: acc += gs at^T
  auto lora_pass = [&]() {
#pragma unroll
    for (int ks = 0; ks < RE / 16; ++ks) {
      uint4 a[kFM], b[2];
#pragma unroll
      for (int i = 0; i < kFM; ++i)
        a[i] = *reinterpret_cast<const uint4*>(gs + ep(wm * kHalf + i * 32 + l32, ks * 16 + lh * 8));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const uint4*>(at + ep(wn * 64 + j * 32 + l32, ks * 16 + lh * 8));
#pragma unroll
      for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    }
  };
  // A^T columns c0 .. c0 + RE - 1 of the side-by-side projections
  auto stage_at = [&](int c0) {
    for (int e = tid; e < BT * (RE / 8); e += kThreads) {
      const int c = e / (RE / 8), jc = c0 + 8 * (e - c * (RE / 8));
      const int g = jc / r, j0 = jc - g * r;  // r % 8 == 0: a chunk never straddles projections
      uint4 v = {0u, 0u, 0u, 0u};
      if (k0 + c < K && jc < R)
        v = *reinterpret_cast<const uint4*>(tab.A[g] + static_cast<size_t>(k0 + c) * r + j0);
      *reinterpret_cast<uint4*>(at + ep(c, jc - c0)) = v;
    }
  };
  if constexpr (MULTI || RU == 0) {  // G from g_out (stored at projection ends, or precomputed)
    if (dx == nullptr) return;
    __threadfence_block();  // this tile's G stores, before other waves read them back
    // n r may exceed RE: the rank columns are added RE at a time
    for (int c0 = 0; c0 < R; c0 += RE) {
      __syncthreads();  // previous pass (or the K-loop) done with gs and at
      for (int e = tid; e < BT * (RE / 8); e += kThreads) {
        const int row = e / (RE / 8), jc = c0 + 8 * (e - row * (RE / 8));
        uint4 v = {0u, 0u, 0u, 0u};
        if (jc < R && m0 + row < T)
          v = *reinterpret_cast<const uint4*>(g_out + static_cast<size_t>(m0 + row) * R + jc);
        *reinterpret_cast<uint4*>(gs + ep(row, jc - c0)) = v;
      }
      stage_at(c0);
      __syncthreads();
      lora_pass();
    }
  } else {
#pragma unroll
    for (int u = 0; u < RU / 32; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * kHalf + wn * 32 + mfma32_row(e, lane), col = u * 32 + l32;
        const uint16_t gv = to_bf16(s * gacc[u][e]);
        if (col < RE) gs[ep(row, col)] = gv;
        if (tk == 0 && col < r && m0 + row < T) g_out[static_cast<size_t>(m0 + row) * r + col] = gv;
      }
    if constexpr (kG16) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = wm * kHalf + wn * 32 + rb * 16 + 4 * lq + e;
          const uint16_t gv = to_bf16(s * gacc16[rb][e]);
          gs[ep(row, l16)] = gv;
          if (tk == 0 && l16 < r && m0 + row < T) g_out[static_cast<size_t>(m0 + row) * r + l16] = gv;
        }
    }
    stage_at(0);
    __syncthreads();
    if (dx == nullptr) return;
    lora_pass();
  }
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = k0 + wn * 64 + j * 32 + l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * kHalf + i * 32 + mfma32_row(e, lane);
        if (row < T && col < K) dx[static_cast<size_t>(row) * K + col] = to_bf16(acc[i][j][e]);
      }
    }
}

// Dispatch arguments: split mode when part_x != nullptr (single projection).
struct DxSplitArgs {
  int splits, steps_per;
  float* part_x;
  float* part_g;
};

template <int BT, int RU, int RE, bool MULTI>
hipError_t launch_dx_t(int T, int K, int r, float s, const DxTable& tab, uint16_t* dx, uint16_t* g_out,
                       const DxSplitArgs& a, hipStream_t stream) {
  const int tiles = ((T + BT - 1) / BT) * ((K + BT - 1) / BT);
  if (tab.wdq[0] != nullptr)
    lora_dx_kernel<BT, RU, RE, MULTI, true><<<tiles * a.splits, DxTile<BT>::kThreads, 0, stream>>>(
        T, K, r, s, tab, dx, g_out, a.steps_per, a.part_x, a.part_g);
  else
    lora_dx_kernel<BT, RU, RE, MULTI, false><<<tiles * a.splits, DxTile<BT>::kThreads, 0, stream>>>(
        T, K, r, s, tab, dx, g_out, a.steps_per, a.part_x, a.part_g);
  return hipGetLastError();
}

template <int BT>
hipError_t launch_dx_rank(int T, int K, int r, float s, const DxTable& tab, uint16_t* dx, uint16_t* g_out,
                          const DxSplitArgs& a, hipStream_t stream, bool g_ready = false) {
  const int R = tab.n * r;
  // G already in g_out: no G in the K loop (RU = 0)
  if (g_ready) {
    if (a.part_x != nullptr || r <= 16) return hipErrorInvalidValue;
    if (tab.n > 1) return launch_dx_t<BT, 0, 64, true>(T, K, r, s, tab, dx, g_out, a, stream);
    if (r <= 32) return launch_dx_t<BT, 0, 32, false>(T, K, r, s, tab, dx, g_out, a, stream);
    if (r <= 48) return launch_dx_t<BT, 0, 48, false>(T, K, r, s, tab, dx, g_out, a, stream);
    return launch_dx_t<BT, 0, 64, false>(T, K, r, s, tab, dx, g_out, a, stream);
  }
  if (tab.n == 1) {
    switch ((r + 15) / 16) {
      case 1: return launch_dx_t<BT, 16, 16, false>(T, K, r, s, tab, dx, g_out, a, stream);
      case 2: return launch_dx_t<BT, 32, 32, false>(T, K, r, s, tab, dx, g_out, a, stream);
      case 3: return launch_dx_t<BT, 64, 48, false>(T, K, r, s, tab, dx, g_out, a, stream);
      case 4: return launch_dx_t<BT, 64, 64, false>(T, K, r, s, tab, dx, g_out, a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  // several projections: RU from r, RE from n r (64 at most: wider sums take several passes)
  const int RE = R >= 64 ? 64 : ((R + 15) / 16) * 16;
  if (r <= 16) {
    switch (RE) {
      case 16: return launch_dx_t<BT, 16, 16, true>(T, K, r, s, tab, dx, g_out, a, stream);
      case 32: return launch_dx_t<BT, 16, 32, true>(T, K, r, s, tab, dx, g_out, a, stream);
      case 48: return launch_dx_t<BT, 16, 48, true>(T, K, r, s, tab, dx, g_out, a, stream);
      default: return launch_dx_t<BT, 16, 64, true>(T, K, r, s, tab, dx, g_out, a, stream);
    }
  }
  if (r <= 32) {
    if (RE == 48) return launch_dx_t<BT, 32, 48, true>(T, K, r, s, tab, dx, g_out, a, stream);
    return launch_dx_t<BT, 32, 64, true>(T, K, r, s, tab, dx, g_out, a, stream);
  }
  return launch_dx_t<BT, 64, 64, true>(T, K, r, s, tab, dx, g_out, a, stream);
}

// Tile edge from a round count: 256 x 256 tiles run one per CU; 128 x 128 tiles
// two per CU at rank <= 16 (one above, where the B slices push the LDS past half
// a CU). A full round of 128 tiles costs a fraction of a round of 256 tiles
// (measured on MI355X); the outputs are the same either way.
constexpr int kDxCost128Num = 3, kDxCost128Den = 4;  // rank <= 16
constexpr int kDxCost128NumR = 2, kDxCost128DenR = 3;  // rank > 16
int dx_tile_edge(int64_t T, int64_t K, int r) {
  const int64_t rounds256 = ((T + 255) / 256 * ((K + 255) / 256) + 255) / 256;
  const int slots128 = r <= 16 ? 512 : 256;
  const int64_t rounds128 = ((T + 127) / 128 * ((K + 127) / 128) + slots128 - 1) / slots128;
  const bool small = r <= 16 ? kDxCost128Num * rounds128 < kDxCost128Den * rounds256
                             : kDxCost128NumR * rounds128 < kDxCost128DenR * rounds256;
  return small ? 128 : 256;
}

}  // namespace

bool lora_dx_supported(int r) { return r % 8 == 0 && r <= 64; }

bool lora_dx_multi_supported(int n_proj, const int* N, int r) {
  if (n_proj < 1 || n_proj > kMaxProj || r % 8 != 0 || r > 64) return false;
  for (int g = 0; g < n_proj; ++g)
    if (N[g] % BK != 0) return false;
  return true;
}

hipError_t launch_lora_dx_table(int T, int K, int r, float s, const DxTable& tab, uint16_t* dx,
                                uint16_t* g_out, hipStream_t stream, bool g_ready) {
  const DxSplitArgs a{1, tab.step_end[tab.n - 1], nullptr, nullptr};
  if (dx_tile_edge(T, K, r) == 256) return launch_dx_rank<256>(T, K, r, s, tab, dx, g_out, a, stream, g_ready);
  return launch_dx_rank<128>(T, K, r, s, tab, dx, g_out, a, stream, g_ready);
}

// d_out splits of the tiled dX of one projection: the rule of the tiled forward's
// K-split with d_out as the reduction (slots: 128 x 128 tiles two per CU at rank
// <= 16), at most four ways and at least sixteen 64-row steps per split (a shorter
// d_out does not pay for the fp32 partials). A half-idle grid splits only for a long
// d_out, or at rank > 32 while strictly under half the slots (measured: 4096-wide
// dX at rank 64 and 128 tiles is slower split).
DxTiledSplit dx_tiled_split(int64_t T, int64_t K, int64_t N, int r) {
  DxTiledSplit p{};
  const int bt = dx_tile_edge(T, K, r);
  const int64_t tiles = (T + bt - 1) / bt * ((K + bt - 1) / bt);
  const int64_t slots = 256 * (bt == 128 && r <= 16 ? 2 : 1);
  const int NS = static_cast<int>((N + BK - 1) / BK);
  const bool half_idle = N >= 16384 ? 2 * tiles <= slots : r > 32 && 2 * tiles < slots;
  const bool idle = 100 * tiles <= 32 * slots || half_idle;
  int S = static_cast<int>(slots / tiles);
  S = S > 4 ? 4 : S;
  S = S > NS / 16 ? NS / 16 : S;
  S = idle && S >= 2 ? S : 1;
  p.steps_per = (NS + S - 1) / S;
  p.splits = (NS + p.steps_per - 1) / p.steps_per;  // every split non-empty
  return p;
}

// The tiled dX on a weight dequantized beforehand: from 1024 tokens on 128 x 128
// tiles and 4096 on 256 x 256 tiles (the forward's rule: there each weight tile
// is read by at least eight token tiles), with the bf16 weight within one buffer
// range. Taken only with weight staging on (lora_nf4_set_weight_staging).
bool dx_dq(int64_t T, int64_t K, int64_t N, int r) {
  return weight_staging() && T >= (dx_tile_edge(T, K, r) == 256 ? 4096 : 1024) &&
         N * K * 2 < (int64_t(1) << 31) - 1;
}

hipError_t launch_lora_dx(int T, int K, int N, int r, float s, const uint16_t* dy,
                          const uint8_t* codes, const float* absmax, const uint16_t* A,
                          const uint16_t* B, const uint16_t* wdq, uint16_t* dx, uint16_t* g_out, float* part_x,
                          float* part_g, hipStream_t stream, bool g_ready) {
  DxTable tab{};
  tab.n = 1;
  tab.step_end[0] = (N + BK - 1) / BK;
  tab.N[0] = N;
  tab.dy[0] = dy;
  tab.codes[0] = codes;
  tab.absmax[0] = absmax;
  tab.A[0] = A;
  tab.B[0] = B;
  tab.wdq[0] = wdq;
  const DxTiledSplit sp = part_x != nullptr ? dx_tiled_split(T, K, N, r) : DxTiledSplit{1, tab.step_end[0]};
  if (sp.splits <= 1) return launch_lora_dx_table(T, K, r, s, tab, dx, g_out, stream, g_ready);
  if (g_ready) return hipErrorInvalidValue;
  const DxSplitArgs a{sp.splits, sp.steps_per, part_x, part_g};
  const hipError_t e = dx_tile_edge(T, K, r) == 256 ? launch_dx_rank<256>(T, K, r, s, tab, dx, g_out, a, stream)
                                                    : launch_dx_rank<128>(T, K, r, s, tab, dx, g_out, a, stream);
  if (e != hipSuccess) return e;
  return launch_dx_splitk_reduce(T, K, r, sp.splits, s, part_x, part_g, A, dx, g_out, stream);
}

}  // namespace lnf4
