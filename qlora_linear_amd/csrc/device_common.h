// Device-side helpers shared by the gfx950 kernels: bf16 packing, the bf16 MFMA
// wrapper and its fragment layout, the NF4 level table, and the XCD-aware
// workgroup remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lnf4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// NF4 levels as float32 bit patterns, code 0..15. The QLoRA NormalFloat
// construction: quantiles of N(0,1) at 8 evenly spaced probabilities from
// delta = 1 - (1/30 + 1/32)/2 towards 1/2 (positive side) and 7 (negative side),
// plus an exact zero, divided by the quantile at delta, rounded to float32.
__host__ __device__ constexpr uint32_t kNf4LevelBits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu, 0xbe91a24bu, 0xbe3d353du,
    0xbdba7869u, 0x00000000u, 0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u,
    0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u};

__device__ __forceinline__ float nf4_level(int c) { return __uint_as_float(kNf4LevelBits[c]); }

// The same level for a per-lane code, formed in registers by a select over the 16
// constants: the kernels fill their LDS level tables with it at the start, where a
// read of the table from memory (and the wait for it) would come ahead of their
// first operand loads.
__device__ __forceinline__ float nf4_level_reg(int c) {
  uint32_t b = kNf4LevelBits[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    b = c == i ? kNf4LevelBits[i] : b;
    asm volatile("" : "+v"(b));  // keeps the selects (no table in memory)
  }
  return __uint_as_float(b);
}

// Two float32 -> packed nearest-even bf16 (v_cvt_pk_bf16_f32); `lo` lands in the
// low half, i.e. at the lower address.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ uint16_t to_bf16(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// v_mfma_f32_16x16x32_bf16: D[16x16] = A[16x32] * B[32x16] + C, fp32 accumulate.
// Operand fragments (one 16-byte register quad per lane):
//   A: lane l holds row (l & 15), reduction elements 8*(l >> 4) .. +7
//   B: lane l holds column (l & 15), reduction elements 8*(l >> 4) .. +7
//   C/D: lane l holds column (l & 15), rows 4*(l >> 4) .. +3
// Any permutation of the reduction index applied to both A and B leaves the
// product unchanged; kernels rely only on the row/column mapping.
__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16: D[32x32] = A[32x16] * B[16x32] + C, fp32 accumulate.
//   A: lane l holds row (l & 31), reduction elements 8*(l >> 5) .. +7
//   B: lane l holds column (l & 31), reduction elements 8*(l >> 5) .. +7
//   C/D element e of lane l: column (l & 31), row 8*(e >> 2) + 4*(l >> 5) + (e & 3)
__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ int mfma32_row(int e, int lane) {
  return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}

// Element offset of (row, 16-byte chunk) in a [rows][64] bf16 LDS tile whose
// chunks are XOR-swizzled by (row / 2) % 8. Fragment reads (16 consecutive rows
// at one chunk) and whole-row writes are then free of bank conflicts.
__device__ __forceinline__ int swz64(int row, int chunk) {
  return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3);
}

// ds_read_b64_tr_b16 (transposing LDS read). Within each group of 16 lanes, lane
// m supplies the address of 4 consecutive b16 values; lane j receives value
// (j & 3) of the chunks supplied by lanes 4 i + (j >> 2), i = 0..3. Pointing lane
// m at row n0 + (m >> 2), columns c0 + 4 (m & 3) .. +3 of a row-major [n][c] tile
// hands lane j the column c0 + j, rows n0 .. n0 + 3: a transposed fragment.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// ds_read_b64_tr_b4 (4-bit transposing LDS read). Within each group of 16 lanes,
// lane m supplies the address of 16 consecutive 4-bit values (8 bytes, the first
// value in the low nibble); lane j receives value (j & 15) of the chunks supplied
// by the group's lanes 0 .. 15, the one from lane i in nibble i: a 16 x 16 nibble
// transpose (the layout was read off an in-bounds probe on gfx950).
typedef int i32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 lds_read_tr4(const void* p) {
  const i32x2_t v = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
      (__attribute__((address_space(3))) i32x2_t*)(const_cast<void*>(p)));
  return __builtin_bit_cast(uint2, v);
}

// Eight consecutive bf16 values from global memory, of which only the first n
// (>= 1) exist; the rest read as zero. For rows whose length is not a multiple of
// 8 (no 16-byte alignment, and a full piece would run into the next row).
__device__ __forceinline__ uint4 load8_masked(const uint16_t* p, int n) {
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t lo = 2 * q < n ? p[2 * q] : 0u, hi = 2 * q + 1 < n ? p[2 * q + 1] : 0u;
    w[q] = lo | (hi << 16);
  }
  return uint4{w[0], w[1], w[2], w[3]};
}

// ---- buffer resources (raw buffers: byte offsets, out-of-range loads return 0) ----
// A load whose lane offset (voffset) lies at or past the descriptor's byte count
// returns zeros. The kernels put every row and column index in the lane offset and
// keep the scalar offset (if any) for a K-step that is clamped to the last step,
// or advance the descriptor's base to the step and pass 0; either way no load
// depends on whether the scalar offset enters the range check, and none reaches
// past its operand.
// kOutOfRange: a lane offset past every descriptor's byte count (the library keeps
// each operand a descriptor covers below 0x7FFFFF00 bytes, so it also stays out of
// range, without wrapping, with any scalar offset below that), for loads that must
// read zeros.
constexpr uint32_t kOutOfRange = 0x7FFFFFF0u;
// Word 3 of a raw buffer descriptor on gfx9-family parts (32-bit data format).
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           kBufferFlags);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(voff),
                                                                         static_cast<int>(soff), 0));
}

__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<int>(voff),
                                                                           static_cast<int>(soff), 0));
}

// 16 bytes per lane from global straight into LDS: lane i writes lds_base + 16 i
// (lds_base must be uniform across the wave; it is passed through M0).
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t rs, void* lds_base, uint32_t voff,
                                               uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds_base),
                                           16, static_cast<int>(voff), static_cast<int>(soff), 0, 0);
}

// 4 bytes per lane from global straight into LDS: lane i writes lds_base + 4 i.
__device__ __forceinline__ void buf_load4_lds(__amdgpu_buffer_rsrc_t rs, void* lds_base, uint32_t voff,
                                              uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds_base),
                                           4, static_cast<int>(voff), static_cast<int>(soff), 0, 0);
}

// Wait until every vector-memory load this wave issued has landed (vmcnt = 0).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N (< 16) vector-memory loads are outstanding. Loads retire
// in issue order, so this waits for everything but the N most recent loads.
template <int N>
__device__ __forceinline__ void wait_vmem_upto() {
  // gfx9 s_waitcnt: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// ---- AdamW of one element, as a fixed sequence of float32 operations, each rounded
// to nearest-even (no fused multiply-add), so every path that updates a LoRA
// factor gives the same bits:
//   m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) (g g)
//   p = p (1 - lr wd) - (lr / (1 - b1^t)) (m / (sqrt(v) (1 / sqrt(1 - b2^t)) + eps))
// AdamWArgs (launch.h) carries the constants, rounded once from float64.
// (Contraction is switched off in the body; `/` and __builtin_sqrtf are correctly
// rounded in HIP device code, whereas __fsqrt_rn is the native approximation.)
template <class Args>
__device__ __forceinline__ void adamw_elem(const Args& h, float g, float& p, float& m, float& v) {
#pragma clang fp contract(off)
  m = h.beta1 * m + h.one_m_beta1 * g;
  v = h.beta2 * v + h.one_m_beta2 * (g * g);
  const float d = __builtin_sqrtf(v) * h.inv_sqrt_bc2 + h.eps;
  p = p * h.decay - h.step_size * (m / d);
}

// Workgroup ids are dispatched round-robin over the 8 XCDs of MI355X (each with
// its own L2). Map them so that each XCD receives one contiguous range of
// logical tile ids; neighbouring logical tiles (which share input rows) then
// share an L2. A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int pid, int n) {
  constexpr int kXcd = 8;
  const int per = n / kXcd, rem = n % kXcd;
  const int xcd = pid % kXcd, local = pid / kXcd;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Grouped (m, n) ordering of a logical tile id: `group_m` row-tiles are swept
// together so that their column tiles reuse the same weight strip.
__device__ __forceinline__ void tile_coords(int lid, int mt, int nt, int group_m, int& m, int& n) {
  const int per_group = group_m * nt;
  const int g = lid / per_group;
  const int first_m = g * group_m;
  const int gsize = min(mt - first_m, group_m);
  const int in = lid - g * per_group;
  m = first_m + in % gsize;
  n = in / gsize;
}

}  // namespace lnf4
