// Fused NF4-LoRA linear, backward input gradient for up to 128 tokens:
//     G  = s dY B^T,   dX = dY deq(Wt) + G A^T
// (the hand-written backward of "Unlocking AI potential: Unsloth's algorithms and
// implementation", core-algorithms section), split over the weight for weight
// streaming, with the reduction over d_out split across workgroups (gfx950).
//
//   * lora_dx_splitk_kernel: workgroup (128 d_in columns, one d_out slice), four
//     waves of 32 columns. Each 64-row step's packed codes (64 rows x 64 bytes),
//     the absmax of every wave's rows and the step's dY chunk go to LDS by
//     direct-to-LDS loads, in a ring of stages three steps ahead; one barrier per
//     step. The reduction runs along the weight's rows, so each lane takes its
//     column's codes with a 4-bit transposing read (ds_read_b64_tr_b4: within a
//     16-lane group, lane j receives column j of the 16 rows the group's lanes
//     address, row e in nibble e) and dequantizes them in registers (a 256-entry
//     table of level pairs, one per code byte, times each row's own absmax) into
//     v_mfma_f32_16x16x32_bf16 B fragments; no dequantized tile passes through
//     LDS. fp32 partial sums go to a workspace [slice][T][d_in]. Taken up to 32
//     tokens when each slice is at least eight steps long; otherwise
//     lora_dx_splitk_tile_kernel dequantizes each step's 64 x 128 tile into LDS
//     and reads it back transposed (ds_read_b64_tr_b16).
//     G: the grid has one more workgroup per (slice, 16-wide rank block), which
//     stages the same dY chunks and loads rows of B straight from global memory
//     (contiguous along d_out, as the MFMA operand needs); its wave w takes the
//     16-token blocks w, w + 4. fp32 partial G goes to [slice][T][r].
//   * lora_dx_splitk_reduce: sums the slices' partials in a fixed order
//     (deterministic), rounds G = s sum to bf16 like the tiled path, adds
//     bf16(G) A^T and stores dX and bf16 G (for dA).
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int kKThreads = 256;          // 4 waves x 32 d_in columns
constexpr int kCols = 128;              // d_in columns per workgroup
constexpr int kNS = 64;                 // d_out rows per step
constexpr uint32_t kOut = 0x7FFFFFF0u;  // a per-lane offset past every buffer range: reads zeros
constexpr int kMaxSplits = 16;
// Workgroups of lora_dx_splitk_kernel<TB> resident per CU (LDS and registers on
// gfx950): the slice count fills one resident round.
constexpr int kResidentTr = 4;                 // lora_dx_splitk_kernel<2>
constexpr int kResidentTile[3] = {3, 2, 2};  // lora_dx_splitk_tile_kernel<TB>, TB = 2, 4, 8
constexpr int kTrMinSteps = 8;  // slice length from which the transposing-code kernel is taken

// TB: 16-token blocks (T <= 16 TB, TB >= 2 so every wave issues the same number
// of dY copies per step). A stage: dY [16 TB][64] bf16, then (main workgroups)
// the codes [64 rows][64 bytes] of the step, whose 16-byte chunks are XOR-swizzled
// by (row >> 2) & 3 (a transposing read of 16 rows at one chunk then touches
// distinct banks), then the absmax of the step's rows for each wave's block
// [4 waves][64] floats.
template <int TB>
struct DxSplitCfg {
  static constexpr int kYBytes = 16 * TB * kNS * 2;
  static constexpr int kCBytes = kNS * 64;
  static constexpr int kABytes = 4 * kNS * 4;
  static constexpr int kStage = kYBytes + kCBytes + kABytes;
  static constexpr int kNB = TB <= 4 ? 4 : 2;         // ring of stages
  static constexpr int kCopies = 2 * TB;             // 1 KB dY copies per stage
  static constexpr int kPerWave = kCopies / 4;
  static constexpr int kBytes = kNB * kStage;
  // loads per wave and step in main workgroups: dY copies, codes, absmax; at the
  // top of step i, stage i has landed once the later stages' loads are all that
  // is outstanding
  static constexpr int kMainWait = (kNB - 3) * (kPerWave + 2);  // stages i and i + 1 landed
};

// Workgroups 0 .. kcb * splits - 1: (column block, slice); the next
// splits * ceil(r / 16): (slice, rank block) of G.
template <int TB>
__global__ __launch_bounds__(kKThreads, 4) void lora_dx_splitk_kernel(
    int T, int K, int N, int r, int rows_per_split, int kcb, int splits, const uint16_t* __restrict__ dy,
    const uint8_t* __restrict__ codes, const float* __restrict__ absmax, const uint16_t* __restrict__ B,
    float* __restrict__ part_x, float* __restrict__ part_g) {
  using C = DxSplitCfg<TB>;
  // level pairs of every code byte, (q[b & 15], q[b >> 4]) at 8 b: first in LDS, so
  // a table address needs no base
  __shared__ __align__(1024) float lut[512];
  __shared__ __align__(16) unsigned char smem[C::kBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int nmain = kcb * splits;
  const bool grole = static_cast<int>(blockIdx.x) >= nmain;  // workgroup-uniform
  const int rj = (r + 15) / 16;
  const int gb = blockIdx.x - nmain;
  // main workgroups: each XCD takes one contiguous range of (slice, column block)
  // ids, so the column blocks that share 128-byte lines of codes (two) and of
  // absmax (sixteen) run on one L2 at about the same time
  const int mid = grole ? 0 : xcd_remap(blockIdx.x, nmain);
  const int sp = grole ? gb / rj : mid / kcb;
  const int kb = grole ? 0 : mid % kcb;
  const int jb = grole ? gb % rj : 0;
  const int k0 = kb * kCols;
  const int nbeg = sp * rows_per_split;
  const int steps = (min(N, nbeg + rows_per_split) - nbeg + kNS - 1) / kNS;  // >= 1
  const int K2 = K / 2, KB = K / 64;

  for (int e = tid; e < 256; e += kKThreads) {
    lut[2 * e] = nf4_level_reg(e & 15);
    lut[2 * e + 1] = nf4_level_reg(e >> 4);
  }

  // Buffer resources over whole operands: rows past d_out (codes, absmax, B rows
  // read along d_out), token rows past T (dY) and rank rows past r (B) read as
  // zeros. Columns past d_out inside a dY or B row are masked explicitly.
  const auto rs_c = make_rsrc(codes, static_cast<uint32_t>(static_cast<size_t>(N) * K2));
  const auto rs_s = make_rsrc(absmax, static_cast<uint32_t>(static_cast<size_t>(N) * KB * 4));
  const auto rs_y = make_rsrc(dy, static_cast<uint32_t>(T) * N * 2);
  const auto rs_b = make_rsrc(B, static_cast<uint32_t>(r) * N * 2);

  // codes stage: wave w copies rows 16 w .. 16 w + 15 (1 KB); lane L lands on row
  // 16 w + (L >> 2), physical chunk L & 3, and loads the logical chunk stored there.
  // Columns past d_in (a last block of 128 with d_in % 128 == 64) read unrelated
  // in-range bytes; those columns are never stored.
  const int crow = 16 * wave + (lane >> 2);
  const uint32_t cvoff = static_cast<uint32_t>(nbeg + crow) * K2 + k0 / 2 + 16 * ((lane & 3) ^ ((crow >> 2) & 3));
  // absmax stage: wave w copies the step's 64 rows of its block (k0 + 32 w) / 64
  const uint32_t avoff = (static_cast<uint32_t>(nbeg + lane) * KB + (k0 + 32 * wave) / 64) * 4;
  const bool wval = k0 + 32 * wave < K;  // the wave's columns lie inside d_in
  // transposing code read for the wave's 16-column block c: lane (l16, g) addresses
  // row 16 g + l16, byte 16 w + 8 c of the row (logical chunk w, half c) and receives
  // column 32 w + 16 c + l16 of rows 16 g .. 16 g + 15 (nibble e = row 16 g + e)
  const int trow = 16 * g + l16;
  const int c_off = trow * 64 + 16 * (wave ^ ((trow >> 2) & 3));  // + 8 c
  // dY stage: [16 TB rows][8 pieces of 8 elements], piece p of row t stored at
  // physical piece p ^ ((t >> 1) & 7). Copy i fills rows 8 i .. 8 i + 7 (1 KB);
  // wave w issues copies w, w + 4, ...; lane L lands on row 8 i + (L >> 3),
  // physical piece L & 7, and loads the logical piece stored there.
  uint32_t yvoff[C::kPerWave];
  int ypiece[C::kPerWave];
#pragma unroll
  for (int c = 0; c < C::kPerWave; ++c) {
    const int t = 8 * (wave + 4 * c) + (lane >> 3);
    ypiece[c] = (lane & 7) ^ ((t >> 1) & 7);
    yvoff[c] = static_cast<uint32_t>(t) * N * 2 + 16 * ypiece[c];
  }
  // dY A fragment for k-slice q and token block tb: row 16 tb + l16. G workgroups:
  // logical piece 4 q + g (d_out rows 32 q + 8 g .. +7 of the step, matching their
  // B rows); main workgroups: piece 2 g + q (rows 16 g + 8 q .. +7, matching the
  // transposed codes)
  auto y_off = [&](int tb, int q) {
    const int t = 16 * tb + l16;
    return t * kNS + (((4 * q + g) ^ ((t >> 1) & 7)) << 3);
  };
  auto y_off_main = [&](int tb, int q) {
    const int t = 16 * tb + l16;
    return t * kNS + (((2 * g + q) ^ ((t >> 1) & 7)) << 3);
  };

  auto stage_of = [&](int i) { return smem + (i % C::kNB) * C::kStage; };
  // one stage: the dY chunk; main workgroups also the codes and the absmax
  auto load_stage = [&](int i) {
    unsigned char* st = stage_of(i);
    const int n = nbeg + i * kNS;
#pragma unroll
    for (int c = 0; c < C::kPerWave; ++c) {
      const uint32_t off = n + 8 * ypiece[c] < N ? yvoff[c] + static_cast<uint32_t>(n) * 2 : kOut;
      buf_load16_lds(rs_y, st + (wave_u + 4 * c) * 1024, off, 0);
    }
    if (grole) return;
    const uint32_t row = static_cast<uint32_t>(i) * kNS;
    buf_load16_lds(rs_c, st + C::kYBytes + wave_u * 1024, cvoff + row * K2, 0);
    buf_load4_lds(rs_s, st + C::kYBytes + C::kCBytes + wave_u * 256, avoff + row * KB * 4, 0);
  };
  // G workgroups: rows 16 jb + l16 of B, d_out columns of k-slice q: 32 q + 8 g .. +7
  uint4 breg[2][2];
  auto load_b = [&](int i, int slot) {
    if (!grole) return;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int n = nbeg + i * kNS + 32 * q + 8 * g;
      const uint32_t off = n < N ? static_cast<uint32_t>(16 * jb + l16) * N * 2 + n * 2 : kOut;
      breg[slot][q] = buf_load16(rs_b, off, 0);
    }
  };

  // B fragment from 8 transposed codes (one dword: rows 16 g + 8 q + 2 j and + 1 in
  // the low and high nibble of byte j) and those rows' absmax: each code byte reads
  // its pair of levels, and every element is multiplied by its own row's absmax
  const unsigned char* lutb = reinterpret_cast<const unsigned char*>(lut);
  auto dequant8 = [&](uint32_t w, const float* a) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t ad = (j == 0 ? (w << 3) : (w >> (8 * j - 3))) & 0x7F8u;
      const float2 p = *reinterpret_cast<const float2*>(lutb + ad);
      v[2 * j] = p.x;
      v[2 * j + 1] = p.y;
    }
    return uint4{pack_bf16x2(__fmul_rn(v[0], a[0]), __fmul_rn(v[1], a[1])),
                 pack_bf16x2(__fmul_rn(v[2], a[2]), __fmul_rn(v[3], a[3])),
                 pack_bf16x2(__fmul_rn(v[4], a[4]), __fmul_rn(v[5], a[5])),
                 pack_bf16x2(__fmul_rn(v[6], a[6]), __fmul_rn(v[7], a[7]))};
  };

  f32x4_t acc[TB][2];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[tb][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // G workgroups: token blocks wave and wave + 4 (a runtime block index would put
  // acc in scratch memory, so these accumulators are indexed by k only)
  f32x4_t gacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};

  // B fragments of one stage: this lane's 16 rows' absmax (a wave past d_in takes
  // zeros: its codes are unrelated bytes) and its two columns' transposed codes
  uint4 wf[2][2];
  auto dequant_stage = [&](const unsigned char* st, uint4 (*w)[2]) {
    const float* ap = reinterpret_cast<const float*>(st + C::kYBytes + C::kCBytes + wave_u * 256) + 16 * g;
    float a[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(ap + 4 * j);
      a[4 * j] = wval ? v.x : 0.f;
      a[4 * j + 1] = wval ? v.y : 0.f;
      a[4 * j + 2] = wval ? v.z : 0.f;
      a[4 * j + 3] = wval ? v.w : 0.f;
    }
    const unsigned char* cst = st + C::kYBytes + c_off;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint2 cc = lds_read_tr4(cst + 8 * c);
      w[c][0] = dequant8(cc.x, a);
      w[c][1] = dequant8(cc.y, a + 8);
    }
  };

  // prologue, in issue order: stages 0 .. kNB - 2, B rows of step 0 (G)
#pragma unroll
  for (int j = 0; j < C::kNB - 1; ++j) load_stage(j);
  load_b(0, 0);

  // Step i: at its top stage i has landed once at most the loads of the later
  // stages are outstanding (main); G workgroups (B rows issued one step ahead)
  // wait for all. The barrier makes stage i visible (and, at step 0, the level
  // table) and ends every wave's reads of step i - 1, whose buffer the stage of
  // step i + kNB - 1 then overwrites. Unrolled by four: compile-time slots.
  auto step = [&](int i, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;  // i % 4
    constexpr int b = slot & 1;
    const unsigned char* st = stage_of(i);
    const uint16_t* ycur = reinterpret_cast<const uint16_t*>(st);
    if (grole) wait_vmem();
    else wait_vmem_upto<C::kMainWait>();
    __syncthreads();
    load_stage(i + C::kNB - 1);
    if (grole) {
      load_b(i + 1, b ^ 1);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int tb = wave_u + 4 * k;
        if (tb < TB) {
#pragma unroll
          for (int q = 0; q < 2; ++q)
            gacc[k] = mfma16(*reinterpret_cast<const uint4*>(ycur + y_off(tb, q)), breg[b][q], gacc[k]);
        }
      }
      return;
    }
    (void)b;
    // the B fragments of step i were formed during step i - 1 (step 0: here); those
    // of step i + 1 are formed now, beside step i's MFMAs
    if (i == 0) dequant_stage(st, wf);
    uint4 wn[2][2];
    if (i + 1 < steps) dequant_stage(stage_of(i + 1), wn);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint4 yf[TB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) yf[tb] = *reinterpret_cast<const uint4*>(ycur + y_off_main(tb, q));
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[tb][c] = mfma16(yf[tb], wf[c][q], acc[tb][c]);
    }
    if (i + 1 < steps)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int q = 0; q < 2; ++q) wf[c][q] = wn[c][q];
  };
  for (int i = 0; i < steps; i += 4) {
    step(i, std::integral_constant<int, 0>{});
    if (i + 1 < steps) step(i + 1, std::integral_constant<int, 1>{});
    if (i + 2 < steps) step(i + 2, std::integral_constant<int, 2>{});
    if (i + 3 < steps) step(i + 3, std::integral_constant<int, 3>{});
  }
  wait_vmem();  // run-ahead loads (direct-to-LDS ones included) land before the workgroup ends

  // C layout: lane (l16, g) holds column l16, rows 4 g + e of each 16 x 16 block
  if (!grole) {
    float* dst = part_x + static_cast<size_t>(sp) * T * K;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * tb + 4 * g + e;
        if (t >= T) continue;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int k = k0 + 32 * wave + 16 * c + l16;
          if (k < K) dst[static_cast<size_t>(t) * K + k] = acc[tb][c][e];
        }
      }
    return;
  }
  float* gdst = part_g + static_cast<size_t>(sp) * T * r;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int tb = wave + 4 * k;
    if (tb >= TB) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * tb + 4 * g + e, j = 16 * jb + l16;
      if (t < T && j < r) gdst[static_cast<size_t>(t) * r + j] = gacc[k][e];
    }
  }
}

// The same product with the weight dequantized into LDS (one step ahead, half an
// NF4 block per thread, natural row-major layout) and read back transposed
// (ds_read_b64_tr_b16); taken where the transposing-code kernel measured slower
// (more than 32 tokens, or slices of fewer than eight steps).
constexpr int kDStride = kCols + 32;    // dequantized tile row pitch, bf16 (320 bytes)
// Row n of the dequantized tile starts at n kDStride + dshift(n): the pitch is 64
// bytes past a multiple of 256, so the four rows of one transposing read fall on
// distinct banks, and rows four apart shift by 16 bytes per group of four, which
// spreads the 16-byte dequantization stores of a 16-lane group over all banks
// (and the two 16-lane groups of a transposing read over disjoint banks).
__device__ __forceinline__ int dshift(int n) { return 8 * ((n >> 2) & 3); }

template <int TB>
struct DxTileCfg {
  static constexpr int kTile = kNS * kDStride * 2;  // bytes of one dequantized tile
  static constexpr int kYBytes = 16 * TB * kNS * 2;  // one dY stage [16 TB][64] bf16
  static constexpr int kCopies = 2 * TB;             // 1 KB direct-to-LDS copies per stage
  static constexpr int kPerWave = kCopies / 4;
  static constexpr int kBytes = 2 * kTile + 2 * kYBytes;
};

// Workgroups 0 .. kcb * splits - 1: (column block, slice); the next
// splits * ceil(r / 16): (slice, rank block) of G.
template <int TB>
__global__ __launch_bounds__(kKThreads) void lora_dx_splitk_tile_kernel(
    int T, int K, int N, int r, int rows_per_split, int kcb, int splits, const uint16_t* __restrict__ dy,
    const uint8_t* __restrict__ codes, const float* __restrict__ absmax, const uint16_t* __restrict__ B,
    float* __restrict__ part_x, float* __restrict__ part_g) {
  using C = DxTileCfg<TB>;
  __shared__ __align__(1024) float lut[16];  // first in LDS: level addresses need no base
  __shared__ __align__(16) unsigned char smem[C::kBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int nmain = kcb * splits;
  const bool grole = static_cast<int>(blockIdx.x) >= nmain;  // workgroup-uniform
  const int rj = (r + 15) / 16;
  const int gb = blockIdx.x - nmain;
  // main workgroups: each XCD takes one contiguous range of (slice, column block)
  // ids, so the column blocks that share 128-byte lines of codes (two) and of
  // absmax (sixteen) run on one L2 at about the same time
  const int mid = grole ? 0 : xcd_remap(blockIdx.x, nmain);
  const int sp = grole ? gb / rj : mid / kcb;
  const int kb = grole ? 0 : mid % kcb;
  const int jb = grole ? gb % rj : 0;
  const int k0 = kb * kCols;
  const int nbeg = sp * rows_per_split;
  const int steps = (min(N, nbeg + rows_per_split) - nbeg + kNS - 1) / kNS;  // >= 1
  const int K2 = K / 2, KB = K / 64;

  if (tid < 16) lut[tid] = nf4_level_reg(tid);

  // Buffer resources over whole operands: rows past d_out (codes, absmax, B rows
  // read along d_out), token rows past T (dY) and rank rows past r (B) read as
  // zeros. Columns past d_out inside a dY or B row are masked explicitly.
  const auto rs_c = make_rsrc(codes, static_cast<uint32_t>(static_cast<size_t>(N) * K2));
  const auto rs_s = make_rsrc(absmax, static_cast<uint32_t>(static_cast<size_t>(N) * KB * 4));
  const auto rs_y = make_rsrc(dy, static_cast<uint32_t>(T) * N * 2);
  const auto rs_b = make_rsrc(B, static_cast<uint32_t>(r) * N * 2);

  // codes: thread owns row nl of the step, columns k0 + 32 run .. +31 (16 bytes,
  // half an NF4 block). Thread bits [1:0] run, [3:2] low row group, [5:4] high row
  // group, [7:6] row within the group of four: each 16 lanes store to distinct banks.
  const int run = tid & 3;
  const int nl = 4 * (((tid >> 2) & 3) | (((tid >> 4) & 3) << 2)) + ((tid >> 6) & 3);
  const bool kval = k0 + 32 * run < K;
  const uint32_t cvoff = static_cast<uint32_t>(nbeg + nl) * K2 + (k0 + 32 * run) / 2;
  const uint32_t svoff = (static_cast<uint32_t>(nbeg + nl) * KB + (k0 + 32 * run) / 64) * 4;
  const int dw_off = nl * kDStride + dshift(nl) + 32 * run;  // + 8 i
  // transposed weight fragment for MFMA k-slice q (rows 32 q .. 32 q + 31 of the
  // step): lane (l16, g) reads rows 32 q + 8 g + 4 h + (l16 >> 2), columns
  // 32 wave + 16 c + 4 (l16 & 3) .. +3 and receives column 16 c + l16 of rows
  // 32 q + 8 g + 4 h .. +3
  const int d_row = 8 * g + (l16 >> 2);                     // + 32 q + 4 h
  const int d_col = 32 * wave + 4 * (l16 & 3);              // + 16 c
  auto d_off = [&](int q, int h) {
    const int n = 32 * q + d_row + 4 * h;
    return n * kDStride + dshift(n) + d_col;
  };
  // dY stage: [16 TB rows][8 pieces of 8 elements], piece p of row t stored at
  // physical piece p ^ ((t >> 1) & 7). Copy i fills rows 8 i .. 8 i + 7 (1 KB);
  // wave w issues copies w, w + 4, ...; lane L lands on row 8 i + (L >> 3),
  // physical piece L & 7, and loads the logical piece stored there.
  uint32_t yvoff[C::kPerWave];
  int ypiece[C::kPerWave];
#pragma unroll
  for (int c = 0; c < C::kPerWave; ++c) {
    const int t = 8 * (wave + 4 * c) + (lane >> 3);
    ypiece[c] = (lane & 7) ^ ((t >> 1) & 7);
    yvoff[c] = static_cast<uint32_t>(t) * N * 2 + 16 * ypiece[c];
  }
  // dY A fragment for k-slice q and token block tb: row 16 tb + l16, logical piece
  // 4 q + g (d_out rows 32 q + 8 g .. +7 of the step)
  auto y_off = [&](int tb, int q) {
    const int t = 16 * tb + l16;
    return t * kNS + (((4 * q + g) ^ ((t >> 1) & 7)) << 3);
  };

  uint16_t* const tile0 = reinterpret_cast<uint16_t*>(smem);
  uint16_t* const tile1 = reinterpret_cast<uint16_t*>(smem + C::kTile);
  uint16_t* const ybuf0 = reinterpret_cast<uint16_t*>(smem + 2 * C::kTile);
  uint16_t* const ybuf1 = reinterpret_cast<uint16_t*>(smem + 2 * C::kTile + C::kYBytes);

  auto load_stage = [&](int i, uint16_t* st) {
    const int n = nbeg + i * kNS;
#pragma unroll
    for (int c = 0; c < C::kPerWave; ++c) {
      const uint32_t off = n + 8 * ypiece[c] < N ? yvoff[c] + static_cast<uint32_t>(n) * 2 : kOut;
      buf_load16_lds(rs_y, st + (wave_u + 4 * c) * 512, off, 0);
    }
  };
  uint4 creg[4];
  float sreg[4];
  auto load_codes = [&](int i, int slot) {
    if (grole) return;
    const uint32_t row = static_cast<uint32_t>(i) * kNS;
    creg[slot] = buf_load16(rs_c, cvoff + row * K2, 0);
    sreg[slot] = __uint_as_float(buf_load4(rs_s, svoff + row * KB * 4, 0));
  };
  // G workgroups: rows 16 jb + l16 of B, d_out columns of k-slice q: 32 q + 8 g .. +7
  uint4 breg[2][2];
  auto load_b = [&](int i, int slot) {
    if (!grole) return;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int n = nbeg + i * kNS + 32 * q + 8 * g;
      const uint32_t off = n < N ? static_cast<uint32_t>(16 * jb + l16) * N * 2 + n * 2 : kOut;
      breg[slot][q] = buf_load16(rs_b, off, 0);
    }
  };

  const unsigned char* lutb = reinterpret_cast<const unsigned char*>(lut);
  auto dequant_store = [&](int slot, uint16_t* tile) {
    const uint32_t cw[4] = {creg[slot].x, creg[slot].y, creg[slot].z, creg[slot].w};
    // a block past d_in gets scale 0: its (in-range, unrelated) codes dequantize to zeros
    const float a = kval ? sreg[slot] : 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t ev = (cw[q] << 2) & 0x3C3C3C3Cu, od = (cw[q] >> 2) & 0x3C3C3C3Cu;
      // keep the two planes: otherwise each address is rebuilt as shift + mask
      asm volatile("" : "+v"(ev), "+v"(od));
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = *reinterpret_cast<const float*>(lutb + __builtin_amdgcn_ubfe(ev, 8 * j, 8));
        v[2 * j + 1] = *reinterpret_cast<const float*>(lutb + __builtin_amdgcn_ubfe(od, 8 * j, 8));
      }
      uint4 o;
      o.x = pack_bf16x2(v[0] * a, v[1] * a);
      o.y = pack_bf16x2(v[2] * a, v[3] * a);
      o.z = pack_bf16x2(v[4] * a, v[5] * a);
      o.w = pack_bf16x2(v[6] * a, v[7] * a);
      *reinterpret_cast<uint4*>(tile + dw_off + 8 * q) = o;
    }
  };

  f32x4_t acc[TB][2];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[tb][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // G workgroups: token blocks wave and wave + 4 (a runtime block index would put
  // acc in scratch memory, so these accumulators are indexed by k only)
  f32x4_t gacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};

  // prologue, in issue order: dY stage 0, codes (or B rows) of steps 0, 1, 2
  load_stage(0, ybuf0);
  load_codes(0, 0);
  load_codes(1, 1);
  load_codes(2, 2);
  load_b(0, 0);
  if (grole) wait_vmem();      // stage 0 and B rows of step 0 landed
  else wait_vmem_upto<4>();    // stage 0 and codes 0 landed
  __syncthreads();                 // level table visible
  if (!grole) dequant_store(0, tile0);

  // Step i: at its top the dY stage of step i and the codes of step i + 1 have
  // landed once at most the two loads issued after them are outstanding (main);
  // G workgroups (stage, then B rows, issued one step ahead) wait for all. The barrier makes the tile and stage of step i
  // visible and ends every wave's reads of step i - 1, whose buffers the stage
  // and tile of step i + 1 then overwrite. Unrolled by four: compile-time slots.
  auto step = [&](int i, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;  // i % 4
    constexpr int b = slot & 1;
    const uint16_t* tcur = b ? tile1 : tile0;
    const uint16_t* ycur = b ? ybuf1 : ybuf0;
    if (grole) wait_vmem();
    else wait_vmem_upto<2>();
    __syncthreads();
    load_stage(i + 1, b ? ybuf0 : ybuf1);
    if (grole) {
      load_b(i + 1, b ^ 1);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int tb = wave_u + 4 * k;
        if (tb < TB) {
#pragma unroll
          for (int q = 0; q < 2; ++q)
            gacc[k] = mfma16(*reinterpret_cast<const uint4*>(ycur + y_off(tb, q)), breg[b][q], gacc[k]);
        }
      }
      return;
    }
    load_codes(i + 3, (slot + 3) & 3);
    if (i + 1 < steps) dequant_store((slot + 1) & 3, b ? tile0 : tile1);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint4 yf[TB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) yf[tb] = *reinterpret_cast<const uint4*>(ycur + y_off(tb, q));
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint16_t* p = tcur + d_off(q, 0) + 16 * c;
        const uint2 lo = lds_read_tr16(p);
        const uint2 hi = lds_read_tr16(tcur + d_off(q, 1) + 16 * c);
        const uint4 wfr = uint4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[tb][c] = mfma16(yf[tb], wfr, acc[tb][c]);
      }
    }
  };
  for (int i = 0; i < steps; i += 4) {
    step(i, std::integral_constant<int, 0>{});
    if (i + 1 < steps) step(i + 1, std::integral_constant<int, 1>{});
    if (i + 2 < steps) step(i + 2, std::integral_constant<int, 2>{});
    if (i + 3 < steps) step(i + 3, std::integral_constant<int, 3>{});
  }
  wait_vmem();  // run-ahead loads (direct-to-LDS ones included) land before the workgroup ends

  // C layout: lane (l16, g) holds column l16, rows 4 g + e of each 16 x 16 block
  if (!grole) {
    float* dst = part_x + static_cast<size_t>(sp) * T * K;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * tb + 4 * g + e;
        if (t >= T) continue;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int k = k0 + 32 * wave + 16 * c + l16;
          if (k < K) dst[static_cast<size_t>(t) * K + k] = acc[tb][c][e];
        }
      }
    return;
  }
  float* gdst = part_g + static_cast<size_t>(sp) * T * r;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int tb = wave + 4 * k;
    if (tb >= TB) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * tb + 4 * g + e, j = 16 * jb + l16;
      if (t < T && j < r) gdst[static_cast<size_t>(t) * r + j] = gacc[k][e];
    }
  }
}

// dX = sum_sp part_x[sp] + bf16(G) A^T, G = s sum_sp part_g[sp]; g_out = bf16(G).
// Workgroup: 8 token rows x 128 d_in columns, 256 threads (4 columns of one row
// each). All loads (every slice's partial, the G parts of the rows, the rows of A
// for the columns) are issued before any is waited on.
constexpr int kRCols = 128, kRRows = 8, kRThreads = 256, kAS = 64 + 8;  // A row pitch, bf16

__global__ __launch_bounds__(kRThreads) void lora_dx_splitk_reduce(
    int T, int K, int r, int S, float s, const float* __restrict__ part_x, const float* __restrict__ part_g,
    const uint16_t* __restrict__ A, uint16_t* __restrict__ dx, uint16_t* __restrict__ g_out) {
  __shared__ float gs[kRRows][64];                    // bf16(G) of the rows, as float
  __shared__ __align__(16) uint16_t as[kRCols * kAS];  // rows k0 .. k0 + 127 of A
  const int tid = threadIdx.x;
  const int k0 = blockIdx.x * kRCols, t0 = blockIdx.y * kRRows;
  const int tl = tid >> 5, c4 = (tid & 31) * 4;
  const int t = t0 + tl, k = k0 + c4;
  const bool mine = dx != nullptr && t < T && k < K;  // K % 64 == 0: 4 columns all in or all out
  float4 w[kMaxSplits];
#pragma unroll
  for (int q = 0; q < kMaxSplits; ++q)
    w[q] = mine && q < S ? *reinterpret_cast<const float4*>(part_x + (static_cast<size_t>(q) * T + t) * K + k)
                         : float4{0.f, 0.f, 0.f, 0.f};
  float gw[2][kMaxSplits];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = tid + kRThreads * h, gr = e >> 6, j = e & 63, gt = t0 + gr;
    const bool ok = j < r && gt < T;
#pragma unroll
    for (int q = 0; q < kMaxSplits; ++q)
      gw[h][q] = ok && q < S ? part_g[(static_cast<size_t>(q) * T + gt) * r + j] : 0.f;
  }
  // A rows: r / 8 pieces of 16 bytes per row (r % 8 == 0)
  uint4 av[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = tid + kRThreads * m, row = e >> 3, pc = e & 7;
    av[m] = 8 * pc < r && k0 + row < K ? *reinterpret_cast<const uint4*>(A + static_cast<size_t>(k0 + row) * r + 8 * pc)
                                       : uint4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = tid + kRThreads * m, row = e >> 3, pc = e & 7;
    *reinterpret_cast<uint4*>(as + row * kAS + 8 * pc) = av[m];
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = tid + kRThreads * h, gr = e >> 6, j = e & 63, gt = t0 + gr;
    float gv = 0.f;
#pragma unroll
    for (int q = 0; q < kMaxSplits; ++q) gv += gw[h][q];
    const uint16_t gb = to_bf16(s * gv);
    gs[gr][j] = bf16_to_f32(gb);
    if (blockIdx.x == 0 && j < r && gt < T) g_out[static_cast<size_t>(gt) * r + j] = gb;
  }
  __syncthreads();
  if (!mine) return;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < kMaxSplits; ++q) o[0] += w[q].x, o[1] += w[q].y, o[2] += w[q].z, o[3] += w[q].w;
  for (int j = 0; j < r; j += 8) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 a8 = *reinterpret_cast<const uint4*>(as + (c4 + c) * kAS + j);
      const uint32_t aw[4] = {a8.x, a8.y, a8.z, a8.w};
#pragma unroll
      for (int h = 0; h < 8; ++h)
        o[c] = fmaf(gs[tl][j + h], __uint_as_float((aw[h >> 1] >> (16 * (h & 1))) << 16), o[c]);
    }
  }
  uint2 packed;
  packed.x = pack_bf16x2(o[0], o[1]);
  packed.y = pack_bf16x2(o[2], o[3]);
  *reinterpret_cast<uint2*>(dx + static_cast<size_t>(t) * K + k) = packed;
}

template <int TB>
hipError_t launch_dx_splitk_t(int T, int K, int N, int r, const DxSplitPlan& p, const uint16_t* dy,
                              const uint8_t* codes, const float* absmax, const uint16_t* B, float* part_x,
                              float* part_g, hipStream_t stream) {
  const int blocks = (p.kcb + (r + 15) / 16) * p.splits;
  if (TB == 2 && p.tr)
    lora_dx_splitk_kernel<2><<<blocks, kKThreads, 0, stream>>>(T, K, N, r, p.rows_per_split, p.kcb, p.splits,
                                                              dy, codes, absmax, B, part_x, part_g);
  else
    lora_dx_splitk_tile_kernel<TB><<<blocks, kKThreads, 0, stream>>>(T, K, N, r, p.rows_per_split, p.kcb,
                                                                    p.splits, dy, codes, absmax, B, part_x,
                                                                    part_g);
  return hipGetLastError();
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

}  // namespace

bool lora_dx_splitk_supported(int64_t T, int r) { return T >= 1 && T <= 128 && r % 8 == 0 && r <= 64; }

DxSplitPlan plan_dx_splitk(int64_t T, int64_t K, int64_t N, int r) {
  DxSplitPlan p{};
  p.kcb = static_cast<int>((K + kCols - 1) / kCols);
  const int nsteps = static_cast<int>((N + kNS - 1) / kNS);
  const int tbi = T <= 32 ? 0 : (T <= 64 ? 1 : 2);
  const int per_split = p.kcb + (r + 15) / 16;
  // Slices: every slice adds per_split workgroups; as many as one resident round
  // holds, at most kMaxSplits. Up to 32 tokens the transposing-code kernel runs
  // when its slices are at least kTrMinSteps steps long.
  auto slice = [&](int resident, int& steps_per) {
    int S = 256 * resident / per_split;
    S = S < 1 ? 1 : (S > kMaxSplits ? kMaxSplits : S);
    S = S > nsteps ? nsteps : S;
    steps_per = (nsteps + S - 1) / S;
  };
  int steps_per = 0;
  p.tr = false;
  if (tbi == 0) {
    slice(kResidentTr, steps_per);
    p.tr = steps_per >= kTrMinSteps;
  }
  if (!p.tr) slice(kResidentTile[tbi], steps_per);
  p.rows_per_split = steps_per * kNS;
  p.splits = (nsteps + steps_per - 1) / steps_per;  // every slice non-empty
  p.part_x_bytes = align256(static_cast<size_t>(p.splits) * T * K * 4);
  p.part_g_bytes = align256(static_cast<size_t>(p.splits) * T * r * 4);
  return p;
}

hipError_t launch_lora_dx_splitk(int T, int K, int N, int r, float s, const uint16_t* dy,
                                 const uint8_t* codes, const float* absmax, const uint16_t* A,
                                 const uint16_t* B, uint16_t* dx, uint16_t* g_out, float* part_x,
                                 float* part_g, hipStream_t stream) {
  const DxSplitPlan p = plan_dx_splitk(T, K, N, r);
  hipError_t e;
  if (T <= 32) e = launch_dx_splitk_t<2>(T, K, N, r, p, dy, codes, absmax, B, part_x, part_g, stream);
  else if (T <= 64) e = launch_dx_splitk_t<4>(T, K, N, r, p, dy, codes, absmax, B, part_x, part_g, stream);
  else e = launch_dx_splitk_t<8>(T, K, N, r, p, dy, codes, absmax, B, part_x, part_g, stream);
  if (e != hipSuccess) return e;
  return launch_dx_splitk_reduce(T, K, r, p.splits, s, part_x, part_g, A, dx, g_out, stream);
}

hipError_t launch_dx_splitk_reduce(int T, int K, int r, int S, float s, const float* part_x,
                                   const float* part_g, const uint16_t* A, uint16_t* dx, uint16_t* g_out,
                                   hipStream_t stream) {
  const dim3 grid((K + kRCols - 1) / kRCols, (T + kRRows - 1) / kRRows);
  lora_dx_splitk_reduce<<<grid, kRThreads, 0, stream>>>(T, K, r, S, s, part_x, part_g, A, dx, g_out);
  return hipGetLastError();
}

}  // namespace lnf4
