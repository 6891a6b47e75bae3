// Fused NF4-LoRA linear on 256 x 256 tiles with the NF4 weight dequantized into
// registers (gfx950), both directions of the linear:
//     forward  y  = x  deq(W)^T + bf16(s x A)  B          reduction over d_in
//     dX       dX = dY deq(W)   + bf16(s dY B^T) A^T      reduction over d_out
//
// The kernel-fusion section of "Unsloth acceleration principles: CUDA kernel
// fusion and memory optimization" runs base product, LoRA down-projection, LoRA
// up-projection and add as one pass whose inputs are staged once on chip. Here
// the 4-bit weight never exists in wider form outside registers:
//
//   * One 256 x 256 output tile per 512-thread workgroup (two waves per SIMD).
//     Wave w owns all 256 token rows x output columns 32 w .. 32 w + 31: 8
//     v_mfma_f32_32x32x16_bf16 accumulators (128 fp32 per lane). No two waves need
//     the same weight element, so each weight element of the tile is dequantized
//     exactly once per tile. (One wave per SIMD with 64 columns each, which halves
//     the token-fragment LDS reads, measured 357 against 277-286 us at q_proj,
//     8192 tokens, with bit-identical output: a lone wave per SIMD exposes every
//     barrier and load wait, and its dequantization competes with its MFMAs.)
//   * K-steps of 64 along the reduction. A lane owns one output column and half
//     of the step: 16 bytes of packed codes (32 NF4 values) loaded straight into
//     registers two steps ahead and dequantized one step ahead (a table of level
//     pairs in LDS indexed by code byte, multiply by the absmax, nearest-even
//     bf16) directly into the MFMA B fragments. The reduction index inside a step
//     is permuted so that those 32 values are exactly the lane's fragments of the
//     step's four 16-deep k-slices: k-slice ks of lane half h holds the 8
//     elements 8 (4 h + ks) .. +7, and the token-operand fragments read from LDS
//     use the same permutation.
//       - forward: the codes of output column n are row n of the packed weight
//         (blocks of 64 run along d_in = the reduction, so a step is one block
//         and one absmax per lane, loaded with the codes);
//       - dX: the codes of output column k, 32 consecutive d_out rows, come from
//         the packed weight transposed once per call (nf4_transpose_kernel:
//         codes^T [d_in][d_out / 2], same nibbles; absmax^T [d_in / 64][d_out]).
//         Every element of a lane's column has its own absmax; the wave's 64
//         values of a step ride the token-operand stage in LDS.
//   * Token-operand tiles [256][64] bf16 (x or dY, 32 KB) move global -> LDS with
//     direct-to-LDS loads into a ring of four stages, three steps ahead; one
//     workgroup barrier per step (a raw s_barrier after a partial vmcnt wait: the
//     loads of later stages stay in flight across it).
//   * Rank 16: the LoRA down-projection (U = x A, or G = dY B^T) in the same K
//     loop. Wave w owns its rows 32 w .. 32 w + 31 (two 16 x 16 x 32 MFMAs per
//     32-deep half step, 1/16 of the tile's MFMA work); the step's slice of A
//     (64 rows, 2 KB, contiguous in A) or B (16 rows x 64 columns) rides each
//     stage. Every column tile of a token tile forms the same U (G); the first
//     one stores it. Other ranks (forward only): U from the U pass, bf16(s U)
//     read in the epilogue (its accumulators would not fit beside the tile's 128).
//   * Epilogue: bf16(s U) (bf16(s G)) and the up-projection operand go through
//     LDS, one MFMA pass over the rank adds the LoRA term, and bf16 y (dX) is
//     stored.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int kBT = 256;          // tile edge (tokens and output columns)
constexpr int kWaves = 8;         // each 256 rows x 32 output columns
constexpr int kThreads = 64 * kWaves;
constexpr int kTileElems = kBT * 64;
constexpr int kGroupM = 2;        // token tiles swept together (token rows read once per XCD round)

// One output tile's operands. L: reduction length (d_in forward, d_out dX); ncols:
// output columns of the product.
struct RwTile {
  int T, L, ncols, m0, c0, r;
  float s;
  const uint16_t* xsrc;  // token operand [T][L] bf16 (x or dY)
  const uint8_t* wc;     // packed codes: one row of L / 2 bytes per output column
  const float* wa;       // forward: absmax [ncols][L / 64]; dX: absmax^T [ncols / 64][L]
  const uint16_t* lr;    // rank 16: forward A [L][16], dX B [16][L]
  const uint16_t* usg;   // other ranks: bf16(s U) rows at stride us_stride (forward)
  int us_stride;
  const uint16_t* eo;    // up-projection operand: forward B [r][ncols], dX A [ncols][r]
  uint16_t* out;         // [T][ncols]; null (dX): only `side` is stored
  uint16_t* side;        // rank 16: bf16(U) (forward) or bf16(s G) (dX), [T][16]; null: none
};

// DX: the dX orientation. RE: rank padded to 16 (epilogue width). LU: the rank-16
// down-projection in the K loop.
template <bool DX, int RE, bool LU>
__device__ __forceinline__ void rw_tile(const RwTile& t) {
  static_assert(!DX || LU, "dX takes the in-loop down-projection");
  // A stage: the token tile [256][64]; then (LU) the step's rank slice, 1024 bf16;
  // then (dX) the absmax of the NEXT step, 64 floats per wave. Four distinct
  // arrays, so the compiler can tell a stage's fragment reads from the
  // direct-to-LDS loads into the other stages.
  constexpr int kLElems = LU ? 1024 : 0;
  constexpr int kAOff = kTileElems + kLElems;  // element offset of the absmax floats
  constexpr int kStageElems = kAOff + (DX ? 2 * 64 * kWaves : 0);
  // level pairs of every code byte, (q[b & 15], q[b >> 4]) at 8 b: first in LDS,
  // so a table address needs no base
  __shared__ __align__(1024) float lut[512];
  __shared__ __align__(16) uint16_t xs0[kStageElems];
  __shared__ __align__(16) uint16_t xs1[kStageElems];
  __shared__ __align__(16) uint16_t xs2[kStageElems];
  __shared__ __align__(16) uint16_t xs3[kStageElems];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int T = t.T, L = t.L, m0 = t.m0, c0 = t.c0, r = t.r;
  const float s = t.s;
  const int L2 = L / 2, LB = L / 64, last = LB - 1;

  for (int e = tid; e < 256; e += kThreads) {
    lut[2 * e] = nf4_level_reg(e & 15);
    lut[2 * e + 1] = nf4_level_reg(e >> 4);
  }

  // ---- buffer resources: this tile's rows only; rows past T (tokens) or ncols
  // (weight) read zeros. Every K-step index passed to a load is clamped to the
  // last step, so no load addresses bytes past its operand's last step.
  const int rows_x = min(T - m0, kBT), rows_w = min(t.ncols - c0, kBT);
  const auto rs_x = make_rsrc(t.xsrc + static_cast<size_t>(m0) * L, static_cast<uint32_t>(rows_x) * L * 2);
  const auto rs_c = make_rsrc(t.wc + static_cast<size_t>(c0) * L2, static_cast<uint32_t>(rows_w) * L2);
  // forward: rows_w rows of LB floats; dX: the tile's four 64-column blocks, rows of L
  const auto rs_s = DX ? make_rsrc(t.wa + static_cast<size_t>(c0 / 64) * L, static_cast<uint32_t>(4) * L * 4)
                       : make_rsrc(t.wa + static_cast<size_t>(c0) * LB, static_cast<uint32_t>(rows_w) * LB * 4);
  const auto rs_l = make_rsrc(t.lr, static_cast<uint32_t>(L) * 32);  // A [L][16] or B [16][L]

  // token operand: wave w fills rows 32 w .. 32 w + 31 with four 1 KB direct-to-LDS
  // loads of 8 rows; lane i lands on physical chunk i & 7 of its row and loads the
  // logical chunk that the (row >> 1) & 7 XOR swizzle maps there. The row is in the
  // lane offset and only the step in the scalar offset, so rows past T lie past
  // the descriptor's range through the lane offset alone.
  constexpr int kXR = kBT / kWaves, kXL = kXR / 8;  // rows and loads per wave
  uint32_t xvoff[kXL];
#pragma unroll
  for (int q = 0; q < kXL; ++q) {
    const int row = kXR * wave + 8 * q + (lane >> 3);
    xvoff[q] = static_cast<uint32_t>(row) * L * 2 + (((lane & 7) ^ ((row >> 1) & 7)) << 4);
  }
  // rank slice (LU), 256 bytes per wave, 4 per lane. Forward: the step's 64 rows
  // of A are 2 KB contiguous; wave w takes bytes 256 w ... dX: wave w takes rows
  // j = 2 w, 2 w + 1 of B's 64 step columns, stored [16][64] with 16-byte chunks
  // XOR-swizzled by j & 7: lane i fills physical dword i & 31 of row 2 w + (i >> 5).
  uint32_t lvoff;
  if constexpr (DX) {
    const int j = 2 * wave + (lane >> 5), pd = lane & 31;
    lvoff = static_cast<uint32_t>(j) * L * 2 + ((((pd >> 2) ^ (j & 7)) << 4) | ((pd & 3) << 2));
  } else {
    lvoff = 256 * static_cast<uint32_t>(wave) + 4 * static_cast<uint32_t>(lane);
  }
  // dX absmax: wave w loads the 64 values of its 64-column block (c0 / 64 + w / 2)
  // for the step's 64 reduction rows, one per lane
  const uint32_t avoff = (static_cast<uint32_t>(wave >> 1) * L + lane) * 4;
  auto load_stage = [&](int kt, uint16_t* stage) {
    const uint32_t k = static_cast<uint32_t>(min(kt, last));
#pragma unroll
    for (int q = 0; q < kXL; ++q)
      buf_load16_lds(rs_x, stage + (kXR * wave_u + 8 * q) * 64, xvoff[q], k * 128);
    if constexpr (LU) buf_load4_lds(rs_l, stage + kTileElems + 128 * wave_u, lvoff, DX ? k * 128 : k * 2048);
    // the next step's absmax (its dequantization runs during this stage's step)
    if constexpr (DX) buf_load4_lds(rs_s, stage + kAOff + 128 * wave_u, avoff, static_cast<uint32_t>(min(kt + 1, last)) * 256);
  };
  // codes: lane (row l32 of the wave's 32 columns, half hh) loads 16 bytes of its
  // column's step; forward: and the column's absmax
  const int wrow = 32 * wave + l32;
  const uint32_t cvoff = static_cast<uint32_t>(wrow) * L2 + 16 * hh;
  const uint32_t svoff = static_cast<uint32_t>(wrow) * LB * 4;
  uint4 creg[2];   // [step parity]
  float sreg[2];
  auto load_codes = [&](int kt, int slot) {
    const uint32_t k = static_cast<uint32_t>(min(kt, last));
    creg[slot] = buf_load16(rs_c, cvoff, k * 32);
    if constexpr (!DX) sreg[slot] = __uint_as_float(buf_load4(rs_s, svoff, k * 4));
  };

  // ---- dequantization of one code dword (8 consecutive reduction elements of one
  // column) into a B fragment: each code byte (two consecutive elements, the lower
  // one in the low nibble) addresses its pair of levels in the table, 8 bytes at
  // 8 b (one 64-bit LDS read per two elements); each level is multiplied by its
  // absmax (fl32(q * a)) and the pair packed to nearest-even bf16.
  const unsigned char* lutb = reinterpret_cast<const unsigned char*>(lut);
  auto levels = [&](uint32_t w, float* v) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t ad = (b == 0 ? (w << 3) : (w >> (8 * b - 3))) & 0x7F8u;
      const float2 p = *reinterpret_cast<const float2*>(lutb + ad);
      v[2 * b] = p.x;
      v[2 * b + 1] = p.y;
    }
  };
  auto code_dword = [&](int slot, int q) -> uint32_t {
    return q == 0 ? creg[slot].x : q == 1 ? creg[slot].y : q == 2 ? creg[slot].z : creg[slot].w;
  };
  // B fragments of the current step, one per k-slice; once k-slice ks's MFMAs have
  // read fragment ks it is overwritten with the next step's
  uint4 bfr[4];
  // astage: (dX) the stage holding the absmax of the step being dequantized; apo:
  // byte offset of this lane's values in it
  auto dequant_dword = [&](int slot, int q, const uint16_t* astage, int apo) {
    float v[8], a[8];
    levels(code_dword(slot, q), v);
    if constexpr (DX) {
      // this lane's 8 reduction rows 32 hh + 8 q .. +7 of the wave's 64 (broadcast reads)
      const float* ap = reinterpret_cast<const float*>(reinterpret_cast<const char*>(astage) + apo) + 8 * q;
      const float4 a0 = *reinterpret_cast<const float4*>(ap), a1 = *reinterpret_cast<const float4*>(ap + 4);
      a[0] = a0.x; a[1] = a0.y; a[2] = a0.z; a[3] = a0.w;
      a[4] = a1.x; a[5] = a1.y; a[6] = a1.z; a[7] = a1.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = sreg[slot];
    }
    bfr[q] = uint4{pack_bf16x2(__fmul_rn(v[0], a[0]), __fmul_rn(v[1], a[1])),
                   pack_bf16x2(__fmul_rn(v[2], a[2]), __fmul_rn(v[3], a[3])),
                   pack_bf16x2(__fmul_rn(v[4], a[4]), __fmul_rn(v[5], a[5])),
                   pack_bf16x2(__fmul_rn(v[6], a[6]), __fmul_rn(v[7], a[7]))};
  };

  // ---- fragment offsets (bytes) into a stage. 32 x 32 x 16 A operand of row block
  // i, k-slice ks: row 32 i + l32, logical chunk 4 hh + ks, i.e. (the chunk bits
  // and the row bits do not overlap) cho0 ^ (ks << 4) + 4096 i.
  const int fkey = (l32 >> 1) & 7;
  const int cho0 = 2 * (l32 * 64 + (((4 * hh) ^ fkey) << 3));
  f32x16_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  // ---- rank 16 (LU): wave w owns rows 32 w .. 32 w + 31 of U (G), two 16 x 16 x 32
  // MFMAs per 32-deep half of a step. A operand: tile row 32 w + 16 rb + (lane & 15),
  // logical chunk 4 kh + (lane >> 4) of the token stage; B operand: rank column
  // lane & 15 at the same 8 reduction rows of the slice (forward: two transposing
  // reads of A's k-major rows; dX: one read of B's row).
  f32x4_t uacc[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int e = 0; e < 4; ++e) uacc[rb][e] = 0.f;
  // byte offsets of half kh = 0; half 1: uxo0 ^ 64 (chunk + 4), and for dX uao0 ^ 64,
  // for the forward uao0 + 1024 (32 rows of A further)
  const int uxo0 = 2 * ((32 * wave + (lane & 15)) * 64 + (((lane >> 4) ^ ((lane & 15) >> 1)) << 3));
  const int uao0 = DX ? 2 * (kTileElems + (lane & 15) * 64 + (((lane >> 4) ^ (lane & 7)) << 3))
                      : 2 * (kTileElems + (8 * (lane >> 4) + ((lane & 15) >> 2)) * 16 + 4 * (lane & 3));
  const int apo0 = 2 * kAOff + 4 * (64 * wave + 32 * hh);  // dX absmax

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

  // ---- prologue: per virtual step v < 3: stage(v), and codes(v) for v < 2 -- the
  // issue order of the steady state, so the end-of-step vmcnt bound holds from the
  // first step: every wave issues kLd loads per step, and between stage(kt + 1)
  // and the end of step kt at least kVm = 2 kLd loads of later steps are issued.
  // dX: the absmax of step v + 1 rides stage v, so step 0's goes first, alone, into
  // the stage before stage 0 (stage 3).
  constexpr int kSt = kXL + (LU ? 1 : 0) + (DX ? 1 : 0);  // loads of one stage
  constexpr int kLd = kSt + (DX ? 1 : 2), kVm = 2 * kLd;
  if constexpr (DX) buf_load4_lds(rs_s, xs3 + kAOff + 128 * wave_u, avoff, 0);
  load_stage(0, xs0);
  load_codes(0, 0);
  load_stage(1, xs1);
  load_codes(1, 1);
  load_stage(2, xs2);
  __syncthreads();  // level table visible
  if constexpr (DX) wait_vmem_upto<3 * kSt + 2>();  // step 0's absmax (this wave's own) has landed
#pragma unroll
  for (int q = 0; q < 4; ++q) dequant_dword(0, q, xs3, apo0);
  wait_vmem_upto<kVm>();  // stage 0 has landed
  __builtin_amdgcn_s_barrier();

  // One K-step: stage CUR of the ring; the step's loads go three steps ahead
  // (stage CUR + 3), its codes two ahead (register set CUR & 1), and the codes of
  // step kt + 1 (the other set) are dequantized slice by slice into the fragments
  // the step's MFMAs have just read.
  auto kstep = [&](int kt, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr int bs = cur & 1, nb = bs ^ 1;
    const char* xc = reinterpret_cast<const char*>(xst(cur_c));
    load_stage(kt + 3, xst(std::integral_constant<int, cur + 3>{}));
    load_codes(kt + 2, bs);
    // the loads stay at the top of the step (left alone, the scheduler sinks them
    // to its end, where their latency is exposed at the next step's dequantization)
    __builtin_amdgcn_sched_barrier(0);
    // The lane offsets, made opaque to the compiler once per step: it then forms
    // the step's LDS addresses from them here (a stage lies beyond the 64 KB reach
    // of an instruction's immediate offset, so each stage needs its own address
    // registers) instead of holding all stages' addresses live across the loop.
    int cho = cho0, uxo = uxo0, uao = uao0, apo = apo0;
    asm volatile("" : "+v"(cho), "+v"(uxo), "+v"(uao), "+v"(apo));
    // Per k-slice: the MFMAs of the slice, the fragment reads of the next slice and
    // the dequantization of this slice's fragment for step kt + 1 (after the MFMAs
    // that read it), interleaved one MFMA, two LDS reads, three VALU operations at
    // a time (measured: the scheduler's own order exposes the LDS latency; this
    // pattern hides it and the barrier's wait). Fragment i of k-slice ks + 1 is
    // read as soon as the MFMA of slice ks has consumed fragment i (one set live).
    uint4 xa[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) xa[i] = *reinterpret_cast<const uint4*>(xc + cho + i * 4096);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 ux, ua;
      if constexpr (LU) {  // rank-16 operands of (row block ks >> 1, half ks & 1)
        const int rb = ks >> 1, kh = ks & 1;
        ux = *reinterpret_cast<const uint4*>(xc + (uxo ^ (kh << 6)) + rb * 2048);
        if constexpr (DX) {
          ua = *reinterpret_cast<const uint4*>(xc + (uao ^ (kh << 6)));
        } else {
          const uint16_t* p = reinterpret_cast<const uint16_t*>(xc + uao + kh * 1024);
          const uint2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 64);
          ua = uint4{lo.x, lo.y, hi.x, hi.y};
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[i] = mfma32(xa[i], bfr[ks], acc[i]);
        if (ks < 3) xa[i] = *reinterpret_cast<const uint4*>(xc + (cho ^ ((ks + 1) << 4)) + i * 4096);
      }
      if constexpr (LU) uacc[ks >> 1] = mfma16(ux, ua, uacc[ks >> 1]);
      dequant_dword(nb, ks, reinterpret_cast<const uint16_t*>(xc), apo);  // dX: this stage carries step kt + 1's absmax
#pragma unroll
      for (int m = 0; m < 8 + (LU ? 1 : 0); ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three VALU
      }
    }
    wait_vmem_upto<kVm>();  // stage kt + 1 has landed
    __builtin_amdgcn_s_barrier();
    // keep the next step's work out of this one (bounds the live registers)
    __builtin_amdgcn_sched_barrier(0);
  };
  // the reduction length % 256 == 0: the loop body is four whole steps, one basic block
  for (int k0 = 0; k0 < LB; k0 += 4) {
    kstep(k0, I0{});
    kstep(k0 + 1, I1{});
    kstep(k0 + 2, I2{});
    kstep(k0 + 3, I3{});
  }
  wait_vmem();       // the run-ahead loads have landed before LDS is reused
  __syncthreads();

  // ---- epilogue: acc += bf16(s U) B (forward) or bf16(s G) A^T (dX) ----------------
  // Rank-wide tiles [256][RE] in stages 0 and 1: rows padded to RE + 8 (16-byte
  // fragment reads free of bank conflicts) when that fits a stage, else (RE = 64)
  // unpadded with the stage's chunk swizzle.
  constexpr int ES = RE + 8;
  constexpr bool kPad = kBT * ES <= kTileElems;
  auto ep = [](int row, int col) {  // element offset of (row, col)
    if constexpr (kPad) return row * ES + col;
    else return swz64(row, col >> 3) + (col & 7);
  };
  uint16_t* us = xs0;  // bf16(s U) / bf16(s G)
  uint16_t* bt = xs1;  // up-projection operand, [output column][rank]
  if constexpr (LU) {  // the wave's rows; bf16(U) / bf16(s G) once per token tile
    uint16_t* side = t.side;
    const float ss = DX ? s : 1.0f;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 32 * wave + 16 * rb + 4 * (lane >> 4) + e, col = lane & 15;
        const float v = uacc[rb][e];
        us[ep(row, col)] = to_bf16(s * v);
        if (side != nullptr && m0 + row < T) side[static_cast<size_t>(m0 + row) * 16 + col] = to_bf16(ss * v);
      }
    if (t.out == nullptr) return;  // uniform: G only
  } else {  // bf16(s U) of this tile's rows, written by the U pass
    const uint16_t* ug = t.usg;
    for (int e = tid; e < kBT * (RE / 8); e += kThreads) {
      const int row = e / (RE / 8), c8 = 8 * (e - row * (RE / 8));
      uint4 v = {0u, 0u, 0u, 0u};
      if (c8 < r && m0 + row < T)
        v = *reinterpret_cast<const uint4*>(ug + static_cast<size_t>(m0 + row) * t.us_stride + c8);
      *reinterpret_cast<uint4*>(us + ep(row, c8)) = v;
    }
  }
  if constexpr (DX) {  // A rows of the tile's columns: 16 contiguous values each
    for (int c = tid; c < kBT; c += kThreads) {
      uint4 v0 = {0u, 0u, 0u, 0u}, v1 = v0;
      if (c0 + c < t.ncols) {
        const uint4* ap = reinterpret_cast<const uint4*>(t.eo + static_cast<size_t>(c0 + c) * 16);
        v0 = ap[0];
        v1 = ap[1];
      }
      *reinterpret_cast<uint4*>(bt + ep(c, 0)) = v0;
      *reinterpret_cast<uint4*>(bt + ep(c, 8)) = v1;
    }
  } else {  // B^T: column c of B's r rows
    const uint16_t* B = t.eo;
    const int N = t.ncols;
    for (int c = tid; c < kBT; c += kThreads) {
      const int n = c0 + c;
#pragma unroll
      for (int j = 0; j < RE; ++j) bt[ep(c, j)] = (j < r && n < N) ? B[static_cast<size_t>(j) * N + n] : uint16_t(0);
    }
  }
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < RE / 16; ++ks) {
    const uint4 b = *reinterpret_cast<const uint4*>(bt + ep(wrow, ks * 16 + hh * 8));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 a = *reinterpret_cast<const uint4*>(us + ep(32 * i + l32, ks * 16 + hh * 8));
      acc[i] = mfma32(a, b, acc[i]);
    }
  }
  // output through LDS: rows 64 b .. 64 b + 63 of the tile in stage b, row-major
  // [64][256] bf16 with the 16-byte chunk index XORed by 4 (row >> 2 & 1) (the two
  // row groups an accumulator's lanes write at once then hit different banks); then
  // each thread stores whole 16-byte chunks, 32 threads per 512-byte row.
  __syncthreads();  // every wave is done with the rank-wide tiles
  auto put = [&](auto bc) {
    constexpr int b = decltype(bc)::value;
    uint16_t* st = xst(bc);
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int col = wrow;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rl = 32 * ii + mfma32_row(e, lane);
        st[rl * 256 + ((((col >> 3) ^ (((rl >> 2) & 1) << 2))) << 3) + (col & 7)] = to_bf16(acc[2 * b + ii][e]);
      }
    }
  };
  put(I0{});
  put(I1{});
  put(I2{});
  put(I3{});
  __syncthreads();
  uint16_t* out = t.out;
  const int NC = t.ncols;
  auto copy_out = [&](auto bc) {
    constexpr int b = decltype(bc)::value;
    const uint16_t* st = xst(bc);
#pragma unroll
    for (int q = 0; q < 64 * 32 / kThreads; ++q) {
      const int idx = q * kThreads + tid, rl = idx >> 5, ch = idx & 31;
      const uint4 v = *reinterpret_cast<const uint4*>(st + rl * 256 + ((ch ^ (((rl >> 2) & 1) << 2)) << 3));
      const int row = m0 + 64 * b + rl, col = c0 + 8 * ch;
      if (row < T && col < NC) *reinterpret_cast<uint4*>(out + static_cast<size_t>(row) * NC + col) = v;
    }
  };
  copy_out(I0{});
  copy_out(I1{});
  copy_out(I2{});
  copy_out(I3{});
}

// Forward: the tiles of every projection of the table (their column tiles side
// by side), XCD-aware order.
template <int RE, bool LU>
__global__ __launch_bounds__(kThreads, 1) void lora_fwd_rw_kernel(int T, int K, int r, float s,
                                                                  const uint16_t* __restrict__ x,
                                                                  const ProjTable tab) {
  const int mt = (T + kBT - 1) / kBT, nt_all = tab.tile_end[tab.n - 1];
  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, mt * nt_all), mt, nt_all, kGroupM, tm, tn);
  int gp = 0;  // this tile's projection (wave-uniform)
  while (gp + 1 < tab.n && tn >= tab.tile_end[gp]) ++gp;
  if (gp > 0) tn -= tab.tile_end[gp - 1];
  RwTile t;
  t.T = T;
  t.L = K;
  t.ncols = tab.N[gp];
  t.m0 = tm * kBT;
  t.c0 = tn * kBT;
  t.r = r;
  t.s = s;
  t.xsrc = x;
  t.wc = tab.codes[gp];
  t.wa = tab.absmax[gp];
  t.lr = tab.A[gp];
  t.usg = tab.usg[gp];
  t.us_stride = tab.us_stride;
  t.eo = tab.B[gp];
  t.out = tab.y[gp];
  t.side = tn == 0 ? tab.u[gp] : nullptr;
  rw_tile<false, RE, LU>(t);
}

// dX at rank 16 on the transposed packed weight.
__global__ __launch_bounds__(kThreads, 1) void lora_dx_rw_kernel(int T, int K, int N, float s,
                                                                 const uint16_t* __restrict__ dy,
                                                                 const uint8_t* __restrict__ codes_t,
                                                                 const float* __restrict__ absmax_t,
                                                                 const uint16_t* __restrict__ A,
                                                                 const uint16_t* __restrict__ B,
                                                                 uint16_t* __restrict__ dx,
                                                                 uint16_t* __restrict__ g_out) {
  const int mt = (T + kBT - 1) / kBT, kt = K / kBT;
  int tm = blockIdx.x, tk = 0;  // dx == null: G only, one column tile per token tile
  if (dx != nullptr) tile_coords(xcd_remap(blockIdx.x, mt * kt), mt, kt, kGroupM, tm, tk);
  RwTile t;
  t.T = T;
  t.L = N;
  t.ncols = K;
  t.m0 = tm * kBT;
  t.c0 = tk * kBT;
  t.r = 16;
  t.s = s;
  t.xsrc = dy;
  t.wc = codes_t;
  t.wa = absmax_t;
  t.lr = B;
  t.usg = nullptr;
  t.us_stride = 0;
  t.eo = A;
  t.out = dx;
  t.side = tk == 0 ? g_out : nullptr;
  rw_tile<true, 16, true>(t);
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

// dX on register-dequantized tiles: from 4096 tokens at rank 16, d_in and d_out
// multiples of 256 (whole tiles of output columns, whole groups of four steps).
bool dx_rw_supported(int64_t T, int64_t K, int64_t N, int r) {
  return T >= 4096 && r == 16 && K % 256 == 0 && N % 256 == 0;
}
size_t dx_rw_bytes(int64_t K, int64_t N) {
  return ((static_cast<size_t>(N) * K / 2 + 255) & ~static_cast<size_t>(255)) +
         ((static_cast<size_t>(K / 64) * N * 4 + 255) & ~static_cast<size_t>(255));
}

hipError_t launch_dx_rw(int T, int K, int N, float s, const uint16_t* dy, const uint8_t* codes,
                        const float* absmax, const uint16_t* A, const uint16_t* B, uint16_t* dx,
                        uint16_t* g_out, void* workspace, hipStream_t stream) {
  uint8_t* codes_t = static_cast<uint8_t*>(workspace);
  float* absmax_t = reinterpret_cast<float*>(codes_t + ((static_cast<size_t>(N) * K / 2 + 255) & ~static_cast<size_t>(255)));
  hipError_t e = launch_nf4_transpose(codes, absmax, N, K, codes_t, absmax_t, stream);
  if (e != hipSuccess) return e;
  const unsigned tiles = static_cast<unsigned>(((T + kBT - 1) / kBT) * (dx != nullptr ? K / kBT : 1));
  lora_dx_rw_kernel<<<tiles, kThreads, 0, stream>>>(T, K, N, s, dy, codes_t, absmax_t, A, B, dx, g_out);
  return hipGetLastError();
}

}  // namespace lnf4
