// Fused NF4-LoRA linear, forward, with the NF4 weight dequantized into registers:
//     y = x deq(Wt)^T + s (x A) B                                         (gfx950)
//
// The kernel-fusion section of "Unsloth acceleration principles: CUDA kernel
// fusion and memory optimization" runs base linear, LoRA down-projection, LoRA
// up-projection and add as one pass whose inputs are staged once on chip. Here
// the 4-bit weight never exists in wider form outside registers:
//
//   * One 256 x 256 output tile per 512-thread workgroup (two waves per SIMD).
//     Wave w owns all 256 token rows x output columns 32 w .. 32 w + 31: 8
//     v_mfma_f32_32x32x16_bf16 accumulators (128 fp32 per lane). No two waves need
//     the same weight element, so each weight element of the tile is dequantized
//     exactly once per tile. (One wave per SIMD with 64 columns each measured
//     slower: a lone wave issues at most one instruction per cycle of its SIMD,
//     and the dequantization's VALU and LDS work then competes with its MFMAs.)
//   * K-steps of 64 = one NF4 block: each weight row has one absmax per step. A
//     lane owns one weight row per 32-column block and half of its step: 16
//     bytes of packed codes (32 NF4 values) loaded straight into registers two
//     steps ahead, dequantized one step ahead (a table of level pairs in LDS
//     indexed by code byte, multiply by the row's absmax, nearest-even bf16)
//     directly into the MFMA B fragments.
//     The reduction index inside a step is permuted so that those 32 values
//     are exactly the lane's fragments of the step's four 16-deep k-slices:
//     k-slice ks of lane half h holds the 8 elements 8 (4 h + ks) .. +7, and
//     the x fragments read from LDS use the same permutation.
//   * x tiles [256][64] bf16 (32 KB) move global -> LDS with direct-to-LDS loads
//     into a ring of four stages, three steps ahead; one workgroup barrier per
//     step (a raw s_barrier after a partial vmcnt wait: the loads of later
//     stages stay in flight across it).
//   * Rank 16: U = x A in the K loop. Wave w owns U rows 32 w .. 32 w + 31 (two
//     16 x 16 x 32 MFMAs per 32-deep half step, 1/16 of the tile's MFMA work);
//     the step's 64 rows of A (2 KB, contiguous in A) ride each x stage. Every
//     column tile of a token tile forms the same U; the first one stores
//     bf16(U). Other ranks: U from the U pass (bf16(s U) read in the epilogue),
//     whose extra accumulators would not fit beside the tile's 128.
//   * Epilogue: bf16(s U) and B^T go through LDS, one MFMA pass over the rank adds
//     (s U) B, and bf16 y is stored.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int kBT = 256;          // tile edge (tokens and output columns)
constexpr int kNJ = 1;            // 32-column blocks per wave: 8 waves of 256 x 32
constexpr int kWaves = 8 / kNJ;
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 4;        // x stages in LDS (loads run kStages - 1 steps ahead)
constexpr int kTileElems = kBT * 64;
constexpr int kGroupM = 2;        // token tiles swept together (x rows read once per XCD round)

// RE: rank padded to 16 (epilogue width). LU: U = x A computed in the K loop (rank
// 16 only), else bf16(s U) comes from the U pass.
template <int RE, bool LU>
__global__ __launch_bounds__(kThreads, 1) void lora_fwd_rw_kernel(int T, int K, int r, float s,
                                                                  const uint16_t* __restrict__ x,
                                                                  const ProjTable tab) {
  // Four distinct stage arrays, so the compiler can tell a stage's fragment reads
  // from the direct-to-LDS loads into the other stages.
  // level pairs of every code byte, (q[b & 15], q[b >> 4]) at 8 b: first in LDS, so
  // a table address needs no base
  __shared__ __align__(1024) float lut[512];
  // A stage: x [256][64], then (LU) the step's A slice [64][16] (k-major, as in A)
  constexpr int kAElems = LU ? 64 * 16 : 0;
  __shared__ __align__(16) uint16_t xs0[kTileElems + kAElems];
  __shared__ __align__(16) uint16_t xs1[kTileElems + kAElems];
  __shared__ __align__(16) uint16_t xs2[kTileElems + kAElems];
  __shared__ __align__(16) uint16_t xs3[kTileElems + kAElems];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int mt = (T + kBT - 1) / kBT, nt_all = tab.tile_end[tab.n - 1];
  const int tiles = mt * nt_all;
  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, tiles), mt, nt_all, kGroupM, tm, tn);
  int gp = 0;  // this tile's projection (wave-uniform)
  while (gp + 1 < tab.n && tn >= tab.tile_end[gp]) ++gp;
  if (gp > 0) tn -= tab.tile_end[gp - 1];
  const int N = tab.N[gp];
  const int m0 = tm * kBT, n0 = tn * kBT;
  const int K2 = K / 2, KB = K / 64, last = KB - 1;

  for (int e = tid; e < 256; e += kThreads) {
    lut[2 * e] = nf4_level(e & 15);
    lut[2 * e + 1] = nf4_level(e >> 4);
  }

  // ---- buffer resources: this tile's rows only; rows past T (x) or N (weight)
  // read zeros. Every K-step index passed to a load is clamped to the last step,
  // so no load addresses bytes past its operand's last step.
  const int rows_x = min(T - m0, kBT), rows_w = min(N - n0, kBT);
  const auto rs_x = make_rsrc(x + static_cast<size_t>(m0) * K, static_cast<uint32_t>(rows_x) * K * 2);
  const auto rs_c = make_rsrc(tab.codes[gp] + static_cast<size_t>(n0) * K2, static_cast<uint32_t>(rows_w) * K2);
  const auto rs_s = make_rsrc(tab.absmax[gp] + static_cast<size_t>(n0) * KB, static_cast<uint32_t>(rows_w) * KB * 4);

  // x: wave w fills rows kXR w .. kXR w + kXR - 1 with 1 KB direct-to-LDS loads of
  // 8 rows; lane i lands on physical chunk i & 7 of its row and loads the logical
  // chunk that the (row >> 1) & 7 XOR swizzle maps there. Rows 16 apart share the
  // swizzle, so two lane offsets serve all the loads (the rest is scalar).
  constexpr int kXR = kBT / kWaves, kXL = kXR / 8;  // rows and loads per wave
  uint32_t xvoff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = kXR * wave + 8 * q + (lane >> 3);
    xvoff[q] = static_cast<uint32_t>(row) * K * 2 + (((lane & 7) ^ ((row >> 1) & 7)) << 4);
  }
  const uint32_t xrow16 = static_cast<uint32_t>(16) * K * 2;  // bytes of 16 rows
  // A (LU): the step's rows of A are 2 KB contiguous; wave w loads bytes
  // 256 w .. 256 w + 255 of them, 4 per lane
  const auto rs_a = make_rsrc(tab.A[gp], static_cast<uint32_t>(K) * 32);
  const uint32_t avoff = 256 * static_cast<uint32_t>(wave) + 4 * static_cast<uint32_t>(lane);
  auto load_x = [&](int kt, uint16_t* stage) {
    const uint32_t soff = static_cast<uint32_t>(min(kt, last)) * 128;
#pragma unroll
    for (int q = 0; q < kXL; ++q)
      buf_load16_lds(rs_x, stage + (kXR * wave_u + 8 * q) * 64, xvoff[q & 1], soff + (q >> 1) * xrow16);
    if constexpr (LU) buf_load4_lds(rs_a, stage + kTileElems + 128 * wave_u, avoff, static_cast<uint32_t>(min(kt, last)) * 2048);
  };
  // codes: lane (column block j, row l32, half hh) loads 16 bytes of its row's step
  // and the row's absmax
  uint32_t cvoff[kNJ], svoff[kNJ];
#pragma unroll
  for (int j = 0; j < kNJ; ++j) {
    const int row = 32 * kNJ * wave + 32 * j + l32;
    cvoff[j] = static_cast<uint32_t>(row) * K2 + 16 * hh;
    svoff[j] = static_cast<uint32_t>(row) * KB * 4;
  }
  uint4 creg[2][kNJ];   // [step parity][j]
  float sreg[2][kNJ];
  auto load_codes = [&](int kt, int slot) {
    const uint32_t k = static_cast<uint32_t>(min(kt, last));
#pragma unroll
    for (int j = 0; j < kNJ; ++j) {
      creg[slot][j] = buf_load16(rs_c, cvoff[j], k * 32);
      sreg[slot][j] = __uint_as_float(buf_load4(rs_s, svoff[j], k * 4));
    }
  };

  // ---- dequantization of one code dword (8 consecutive k of one row) into a B
  // fragment: each code byte (two consecutive elements, the even one in the low
  // nibble) addresses its pair of levels in the table, 8 bytes at 8 b (one 64-bit
  // LDS read per two elements); each level is multiplied by the row's absmax
  // (fl32(q * a)) and the pair packed to nearest-even bf16.
  const unsigned char* lutb = reinterpret_cast<const unsigned char*>(lut);
  auto dequant = [&](uint32_t w, float a) -> uint4 {
    float v[8];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t ad = (b == 0 ? (w << 3) : (w >> (8 * b - 3))) & 0x7F8u;
      const float2 p = *reinterpret_cast<const float2*>(lutb + ad);
      v[2 * b] = p.x;
      v[2 * b + 1] = p.y;
    }
    return uint4{pack_bf16x2(__fmul_rn(v[0], a), __fmul_rn(v[1], a)), pack_bf16x2(__fmul_rn(v[2], a), __fmul_rn(v[3], a)),
                 pack_bf16x2(__fmul_rn(v[4], a), __fmul_rn(v[5], a)), pack_bf16x2(__fmul_rn(v[6], a), __fmul_rn(v[7], a))};
  };
  auto code_dword = [&](int slot, int j, int q) -> uint32_t {
    return q == 0 ? creg[slot][j].x : q == 1 ? creg[slot][j].y : q == 2 ? creg[slot][j].z : creg[slot][j].w;
  };
  // B fragments of the current step, [j][k-slice]; once k-slice ks's MFMAs have
  // read fragment (j, ks) it is overwritten with the next step's
  uint4 bfr[kNJ][4];
  auto dequant_dword = [&](int slot, int j, int q) { bfr[j][q] = dequant(code_dword(slot, j, q), sreg[slot][j]); };

  // ---- fragment offsets (elements) into an x stage. 32 x 32 x 16 A operand of
  // row block i, k-slice ks: row 32 i + l32, logical chunk 4 hh + ks.
  const int fkey = (l32 >> 1) & 7;
  int choff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) choff[ks] = l32 * 64 + (((4 * hh + ks) ^ fkey) << 3);
  f32x16_t acc[8][kNJ];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < kNJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  // ---- U (LU): wave w owns U rows 32 w .. 32 w + 31, two 16 x 16 x 32 MFMAs per
  // 32-deep half of a step. A operand: tile row 32 w + 16 rb + (lane & 15), logical
  // chunk 4 kh + (lane >> 4) of the x stage; B operand: column lane & 15 of the
  // same 8 k of the A slice, two transposing reads of 4 rows each.
  f32x4_t uacc[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int e = 0; e < 4; ++e) uacc[rb][e] = 0.f;
  int uxo[2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
    uxo[kh] = (32 * wave + (lane & 15)) * 64 + (((4 * kh + (lane >> 4)) ^ ((lane & 15) >> 1)) << 3);
  const int uao = kTileElems + (8 * (lane >> 4) + ((lane & 15) >> 2)) * 16 + 4 * (lane & 3);

  auto xst = [&](auto c) -> uint16_t* {
    constexpr int i = decltype(c)::value & 3;
    if constexpr (i == 0) return xs0;
    else if constexpr (i == 1) return xs1;
    else if constexpr (i == 2) return xs2;
    else return xs3;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  // ---- prologue: per virtual step t < 3: x(t), and codes(t) for t < 2 -- the issue
  // order of the steady state, so the end-of-step vmcnt bound holds from the first
  // step: every wave issues kLd = kXL + 2 kNJ loads per step, and between x(kt + 1)
  // and the end of step kt at least kVm = 2 kLd loads of later steps are issued.
  constexpr int kLd = kXL + (LU ? 1 : 0) + 2 * kNJ, kVm = 2 * kLd;
  load_x(0, xs0);
  load_codes(0, 0);
  load_x(1, xs1);
  load_codes(1, 1);
  load_x(2, xs2);
  __syncthreads();  // level table visible
#pragma unroll
  for (int j = 0; j < kNJ; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) dequant_dword(0, j, q);
  wait_vmem_upto<kVm>();  // x(0) has landed (after it: codes(0), x(1), codes(1), x(2): 2 kLd loads)
  __builtin_amdgcn_s_barrier();

  // One K-step: stage CUR of the ring; the step's loads go three steps ahead
  // (stage CUR + 3), its codes two ahead (register set CUR & 1), and the codes of
  // step kt + 1 (the other set) are dequantized slice by slice into the fragments
  // the step's MFMAs have just read.
  auto kstep = [&](int kt, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr int bs = cur & 1, nb = bs ^ 1;
    const uint16_t* xc = xst(cur_c);
    load_x(kt + 3, xst(std::integral_constant<int, cur + 3>{}));
    load_codes(kt + 2, bs);
    // the loads stay at the top of the step (left alone, the scheduler sinks them
    // to its end, where their latency is exposed at the next step's dequantization)
    __builtin_amdgcn_sched_barrier(0);
    // Per k-slice: the MFMAs of the slice, the x fragment reads of the next slice
    // and the dequantization of this slice's fragments for step kt + 1 (after the
    // MFMAs that read them), interleaved one MFMA, two LDS reads, three VALU
    // operations at a time (measured: the scheduler's own order exposes the LDS
    // latency; this pattern hides it and the barrier's wait).
    // x fragments: fragment i of k-slice ks + 1 is read as soon as the MFMAs of
    // slice ks have consumed fragment i (one set of 8 live)
    uint4 xa[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) xa[i] = *reinterpret_cast<const uint4*>(xc + choff[0] + i * 2048);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 ux, ua;
      if constexpr (LU) {  // U operands of (row block ks >> 1, k half ks & 1)
        const int rb = ks >> 1, kh = ks & 1;
        ux = *reinterpret_cast<const uint4*>(xc + uxo[kh] + rb * 1024);
        const uint2 lo = lds_read_tr16(xc + uao + kh * 512), hi = lds_read_tr16(xc + uao + kh * 512 + 64);
        ua = uint4{lo.x, lo.y, hi.x, hi.y};
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < kNJ; ++j) acc[i][j] = mfma32(xa[i], bfr[j][ks], acc[i][j]);
        if (ks < 3) xa[i] = *reinterpret_cast<const uint4*>(xc + choff[ks + 1] + i * 2048);
      }
      if constexpr (LU) uacc[ks >> 1] = mfma16(ux, ua, uacc[ks >> 1]);
#pragma unroll
      for (int j = 0; j < kNJ; ++j) dequant_dword(nb, j, ks);
#pragma unroll
      for (int m = 0; m < 8 * kNJ + (LU ? 1 : 0); ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three VALU
      }
    }
    wait_vmem_upto<kVm>();  // x(kt + 1) has landed
    __builtin_amdgcn_s_barrier();
    // keep the next step's work out of this one (bounds the live registers)
    __builtin_amdgcn_sched_barrier(0);
  };
  // d_in % 256 == 0: the loop body is four whole steps, one basic block
  for (int k0 = 0; k0 < KB; k0 += 4) {
    kstep(k0, I0{});
    kstep(k0 + 1, I1{});
    kstep(k0 + 2, I2{});
    kstep(k0 + 3, I3{});
  }
  wait_vmem();       // the run-ahead loads have landed before LDS is reused
  __syncthreads();

  // ---- epilogue: acc += bf16(s U) B ------------------------------------------------
  // Rank-wide tiles [256][RE] in stages 0 and 1: rows padded to RE + 8 (16-byte
  // fragment reads free of bank conflicts) when that fits a stage, else (RE = 64)
  // unpadded with the stage's chunk swizzle.
  constexpr int ES = RE + 8;
  constexpr bool kPad = kBT * ES <= kTileElems;
  auto ep = [](int row, int col) {  // element offset of (row, col)
    if constexpr (kPad) return row * ES + col;
    else return swz64(row, col >> 3) + (col & 7);
  };
  uint16_t* us = xs0;  // bf16(s U)
  uint16_t* bt = xs1;  // B^T tile
  if constexpr (LU) {  // bf16(s U) of the wave's rows; bf16(U) once per token tile
    uint16_t* ug = tn == 0 ? tab.u[gp] : nullptr;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 32 * wave + 16 * rb + 4 * (lane >> 4) + e, col = lane & 15;
        const float v = uacc[rb][e];
        us[ep(row, col)] = to_bf16(s * v);
        if (ug != nullptr && m0 + row < T) ug[static_cast<size_t>(m0 + row) * 16 + col] = to_bf16(v);
      }
  } else {  // bf16(s U) of this tile's rows, written by the U pass
    const uint16_t* ug = tab.usg[gp];
    for (int e = tid; e < kBT * (RE / 8); e += kThreads) {
      const int row = e / (RE / 8), c8 = 8 * (e - row * (RE / 8));
      uint4 v = {0u, 0u, 0u, 0u};
      if (c8 < r && m0 + row < T)
        v = *reinterpret_cast<const uint4*>(ug + static_cast<size_t>(m0 + row) * tab.us_stride + c8);
      *reinterpret_cast<uint4*>(us + ep(row, c8)) = v;
    }
  }
  {
    const uint16_t* B = tab.B[gp];
    for (int c = tid; c < kBT; c += kThreads) {
      const int n = n0 + c;
#pragma unroll
      for (int j = 0; j < RE; ++j) bt[ep(c, j)] = (j < r && n < N) ? B[static_cast<size_t>(j) * N + n] : uint16_t(0);
    }
  }
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < RE / 16; ++ks) {
    uint4 b[kNJ];
#pragma unroll
    for (int j = 0; j < kNJ; ++j)
      b[j] = *reinterpret_cast<const uint4*>(bt + ep(32 * kNJ * wave + 32 * j + l32, ks * 16 + hh * 8));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 a = *reinterpret_cast<const uint4*>(us + ep(32 * i + l32, ks * 16 + hh * 8));
#pragma unroll
      for (int j = 0; j < kNJ; ++j) acc[i][j] = mfma32(a, b[j], acc[i][j]);
    }
  }
  // y through LDS: rows 64 b .. 64 b + 63 of the tile in stage b, row-major [64][256]
  // bf16 with the 16-byte chunk index XORed by 4 (row >> 2 & 1) (the two row groups
  // an accumulator's lanes write at once then hit different banks); then each thread
  // stores whole 16-byte chunks, 32 threads per 512-byte row.
  __syncthreads();  // every wave is done with the rank-wide tiles
  auto put = [&](auto bc) {
    constexpr int b = decltype(bc)::value;
    uint16_t* st = xst(bc);
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < kNJ; ++j) {
        const int col = 32 * kNJ * wave + 32 * j + l32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int rl = 32 * ii + mfma32_row(e, lane);
          st[rl * 256 + ((((col >> 3) ^ (((rl >> 2) & 1) << 2))) << 3) + (col & 7)] = to_bf16(acc[2 * b + ii][j][e]);
        }
      }
  };
  put(I0{});
  put(I1{});
  put(I2{});
  put(I3{});
  __syncthreads();
  uint16_t* y = tab.y[gp];
  auto copy_out = [&](auto bc) {
    constexpr int b = decltype(bc)::value;
    const uint16_t* st = xst(bc);
#pragma unroll
    for (int q = 0; q < 64 * 32 / kThreads; ++q) {
      const int idx = q * kThreads + tid, rl = idx >> 5, ch = idx & 31;
      const uint4 v = *reinterpret_cast<const uint4*>(st + rl * 256 + ((ch ^ (((rl >> 2) & 1) << 2)) << 3));
      const int row = m0 + 64 * b + rl, col = n0 + 8 * ch;
      if (row < T && col < N) *reinterpret_cast<uint4*>(y + static_cast<size_t>(row) * N + col) = v;
    }
  };
  copy_out(I0{});
  copy_out(I1{});
  copy_out(I2{});
  copy_out(I3{});
}

}  // namespace

// Taken for 256 x 256 tile grids from 4096 tokens (where the tile grid fills the
// GPU at least twice over a 4096-wide output), r % 8 == 0, r <= 64, d_in % 256 == 0
// (whole groups of four K-steps).
bool fwd_rw_supported(int64_t T, int64_t K, int r) { return T >= 4096 && r % 8 == 0 && r <= 64 && K % 256 == 0; }
bool fwd_rw_inloop_u(int r) { return r == 16; }

hipError_t launch_fwd_rw(int T, int K, int r, float s, const uint16_t* x, const ProjTable& tab,
                         hipStream_t stream) {
  const int tiles = ((T + kBT - 1) / kBT) * tab.tile_end[tab.n - 1];
  switch ((r + 15) / 16) {
    case 1:
      if (fwd_rw_inloop_u(r)) lora_fwd_rw_kernel<16, true><<<tiles, kThreads, 0, stream>>>(T, K, r, s, x, tab);
      else lora_fwd_rw_kernel<16, false><<<tiles, kThreads, 0, stream>>>(T, K, r, s, x, tab);
      break;
    case 2: lora_fwd_rw_kernel<32, false><<<tiles, kThreads, 0, stream>>>(T, K, r, s, x, tab); break;
    case 3: lora_fwd_rw_kernel<48, false><<<tiles, kThreads, 0, stream>>>(T, K, r, s, x, tab); break;
    default: lora_fwd_rw_kernel<64, false><<<tiles, kThreads, 0, stream>>>(T, K, r, s, x, tab); break;
  }
  return hipGetLastError();
}

}  // namespace lnf4
