// Merged base weight for export: W' = D + s (A B)^T, [d_out, d_in] (gfx950).
//
// After training the adapters are folded into the base weight and saved at 16
// bits ("Unsloth in three lines of code", section 4; "Reading the Unsloth
// changelog", the command-line part of section 2: saving turns the 4-bit model
// into a 16-bit one). Each element is
//     fl32( fl32(q[code] * absmax) + s * sum_j A[k][j] B[j][n] ),
// the low-rank sum accumulated in float32 by MFMA, then rounded once to the
// output type (bf16 nearest-even, or float32).
//
// Tiles of 64 x 256 (64 rows n of d_out, 256 columns k of d_in); a 256-thread
// workgroup takes a run of consecutive tiles of one 256-column block, so that the
// reads of one tile overlap the stores of the one before (the op is bound by HBM:
// 0.5625 bytes of packed weight in, 2 or 4 bytes out per element):
//   1. A rows k0 .. k0 + 255 and B columns n0 .. n0 + 63 of every tile of the
//      workgroup go to LDS once, rank padded with zeros to a multiple of 32, at
//      most 128 rank columns per pass (the only LDS use; its size bounds the run
//      so that two workgroups share a CU); the tiles then run without a barrier,
//      each loading the next one's codes and absmax into registers while it
//      forms and stores its own elements (a store counts in the same in-order
//      counter as a load on gfx9, so staging per tile would wait for the stores);
//   2. v_mfma_f32_16x16x32_bf16 forms (A B)^T with A as the row operand (its rows
//      are contiguous in the reduction j). The MFMA row m of block b reads A row
//      32 (b >> 1) + 8 (m >> 2) + 4 (b & 1) + (m & 3) of the wave's 64 columns, so
//      that a lane (m = l16, g) holds columns 8 g .. 8 g + 7 (blocks 0, 1) and
//      32 + 8 g .. 32 + 8 g + 7 (blocks 2, 3) of one row n;
//   3. each lane dequantizes exactly those 16 elements (2 x 4 bytes of codes, one
//      absmax) and adds s times its accumulators; the wave's 16 rows x 64 columns
//      pass through its own LDS rows, so that each store instruction writes whole
//      row segments of the wave's 64 columns (128 bytes in bf16, 256 in float32)
//      rather than 16 half lines.
#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kMN = 64;    // d_out rows per workgroup
constexpr int kMK = 256;   // d_in columns per workgroup (64 per wave)

// MP: more than one rank pass (r > RP; one tile per workgroup); otherwise the pass
// loop is compiled out and only one n-block's accumulators are live at a time.
// Workgroup (bx, by) takes the tiles of k-block bx and n-blocks by * tiles_per ..
// by * tiles_per + tiles_per - 1, tiles_per <= PT.
template <int RP, int PT, bool OUT_BF16, bool MP>
__global__ __launch_bounds__(kThreads) void lora_merge_kernel(int K, int N, int r, float s, int tiles_per,
                                                              const uint8_t* __restrict__ codes,
                                                              const float* __restrict__ absmax,
                                                              const uint16_t* __restrict__ A,
                                                              const uint16_t* __restrict__ B,
                                                              void* __restrict__ out) {
  constexpr int RS = RP + 8;  // bf16 row stride of the staged factors
  __shared__ __align__(1024) float lut[16];
  __shared__ __align__(16) uint16_t at[kMK * RS];
  __shared__ __align__(16) uint16_t bt[PT * kMN * RS];
  // per wave: 16 rows of 64 output values, rows padded by 16 bytes
  constexpr int kOutB = OUT_BF16 ? 2 : 4, kWRow = 64 * kOutB + 16;
  __shared__ __align__(16) unsigned char wout[4 * 16 * kWRow];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int k0 = blockIdx.x * kMK;
  const int nt_all = (N + kMN - 1) / kMN, t_begin = blockIdx.y * tiles_per;
  const int t_end = min(t_begin + tiles_per, nt_all);
  const int kw = k0 + 64 * wave;  // this wave's 64 columns (one NF4 block per row)
  if (tid < 16) lut[tid] = nf4_level_reg(tid);

  // step 3's codes and absmax of tile t, loaded a tile ahead so their latency
  // overlaps the tile before: n-block nb, lane (l16, g): row n0 + 16 nb + l16,
  // columns kw + 8 g .. +7 and kw + 32 + 8 g .. +7. Buffer loads over the
  // workgroup's rows: rows past d_out (and the run-ahead past its last tile) read
  // zeros without a branch.
  const int K2 = K / 2, KB = K / 64;
  const int row0 = t_begin * kMN, rows = min(N - row0, (t_end - t_begin) * kMN);
  const auto rs_c = make_rsrc(codes + static_cast<size_t>(row0) * K2, static_cast<uint32_t>(rows) * K2);
  const auto rs_s = make_rsrc(absmax + static_cast<size_t>(row0) * KB, static_cast<uint32_t>(rows) * KB * 4);
  uint2 cw[4], cwn[4];
  float av[4], avn[4];
  auto load_codes = [&](int t, uint2* c, float* a) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const uint32_t rr = static_cast<uint32_t>(t * kMN + 16 * nb + l16 - row0);
      const uint32_t co = rr * K2 + kw / 2 + 4 * g;
      c[nb] = uint2{buf_load4(rs_c, co, 0), buf_load4(rs_c, co + 16, 0)};
      a[nb] = __uint_as_float(buf_load4(rs_s, (rr * KB + kw / 64) * 4, 0));
    }
  };

  // ---- 1. stage A and B, RP rank columns per pass (one pass up to r = 128). A rows
  // k0 .. k0 + 255 and B columns n0 .. n0 + 63 of the pass's rank columns go to LDS
  // as 16-byte pieces, element by element where a row of A (r % 8 != 0) or of B
  // (d_out % 8 != 0) is not 16-byte aligned; rank columns past r are zero. A is
  // staged once per workgroup (one pass), B of every tile of the run likewise.
  // The pieces are loaded into registers first, then the codes of the first tile
  // are issued, and only then are the pieces written to LDS: the writes wait for
  // the pieces, not for the codes.
  // ---- 2. per n-block: (A B)^T for 16 rows x 64 columns, accumulated over the passes.
  // A row of MFMA row l16 in block b: 64 wave + 32 (b >> 1) + 8 (l16 >> 2) + 4 (b & 1) + (l16 & 3)
  const int arow = 64 * wave + 8 * (l16 >> 2) + (l16 & 3);
  f32x4_t acc[4][4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[nb][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bool avec = r % 8 == 0, bvec = N % 8 == 0;
  constexpr int kAP = kMK * (RP / 8) / kThreads;  // A pieces per thread
  constexpr int kBP = RP * (kMN / 8) / kThreads;  // B pieces per thread and tile
  static_assert(kAP * kThreads == kMK * (RP / 8) && kBP * kThreads == RP * (kMN / 8), "pieces");
  uint4 apc[kAP], bpc[PT][kBP];
  // Aligned rows (r % 8 == 0, d_out % 8 == 0: the usual case) load as buffer pieces,
  // pieces past r, d_in or d_out through an offset past the range (zeros), so the
  // loads issue back to back; other shapes element by element.
  const auto rs_a = make_rsrc(A, static_cast<uint32_t>(K) * r * 2);
  const auto rs_b = make_rsrc(B, static_cast<uint32_t>(r) * N * 2);
  auto load_a = [&](int j0) {
    if (avec) {
#pragma unroll
      for (int i = 0; i < kAP; ++i) {
        const int c = tid + i * kThreads, kk = c / (RP / 8), j = j0 + 8 * (c - kk * (RP / 8));
        const bool in = j < r && k0 + kk < K;
        apc[i] = buf_load16(rs_a, in ? static_cast<uint32_t>((k0 + kk) * r + j) * 2 : kOutOfRange, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kAP; ++i) {
        const int c = tid + i * kThreads, kk = c / (RP / 8), j = j0 + 8 * (c - kk * (RP / 8));
        const bool in = j < r && k0 + kk < K;
        apc[i] = in ? load8_masked(A + static_cast<size_t>(k0 + kk) * r + j, r - j) : uint4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_a = [&](int j0) {
#pragma unroll
    for (int i = 0; i < kAP; ++i) {
      const int c = tid + i * kThreads, kk = c / (RP / 8), j = j0 + 8 * (c - kk * (RP / 8));
      *reinterpret_cast<uint4*>(at + kk * RS + (j - j0)) = apc[i];
    }
  };
  auto load_b = [&](int j0, int n0, uint4* bp) {
    if (bvec) {
#pragma unroll
      for (int i = 0; i < kBP; ++i) {
        const int c = tid + i * kThreads, jj = c / (kMN / 8), nn = 8 * (c - jj * (kMN / 8)), j = j0 + jj;
        const bool in = j < r && n0 + nn < N;
        bp[i] = buf_load16(rs_b, in ? static_cast<uint32_t>(j * N + n0 + nn) * 2 : kOutOfRange, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kBP; ++i) {
        const int c = tid + i * kThreads, jj = c / (kMN / 8), nn = 8 * (c - jj * (kMN / 8)), j = j0 + jj;
        const bool in = j < r && n0 + nn < N;
        bp[i] = in ? load8_masked(B + static_cast<size_t>(j) * N + n0 + nn, N - n0 - nn) : uint4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_b = [&](const uint4* bp, uint16_t* bt) {
#pragma unroll
    for (int i = 0; i < kBP; ++i) {
      const int c = tid + i * kThreads, jj = c / (kMN / 8), nn = 8 * (c - jj * (kMN / 8));
      const uint32_t w[4] = {bp[i].x, bp[i].y, bp[i].z, bp[i].w};
#pragma unroll
      for (int t = 0; t < 8; ++t) bt[(nn + t) * RS + jj] = static_cast<uint16_t>(w[t >> 1] >> (16 * (t & 1)));
    }
  };
  auto product = [&](int nb, f32x4_t* a4, const uint16_t* bt) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int jq = 0; jq < RP / 32; ++jq) {
        const uint4 a = *reinterpret_cast<const uint4*>(at + (arow + 32 * (b >> 1) + 4 * (b & 1)) * RS + 32 * jq + 8 * g);
        const uint4 bb = *reinterpret_cast<const uint4*>(bt + (16 * nb + l16) * RS + 32 * jq + 8 * g);
        a4[b] = mfma16(a, bb, a4[b]);
      }
  };
  // every pass but the last accumulates all four n-blocks; the last pass forms each
  // n-block's product right before its elements (one pass for r <= 128; with more,
  // one tile per workgroup)
  int j0 = 0;
  for (; MP && j0 + RP < r; j0 += RP) {
    load_a(j0);
    load_b(j0, row0, bpc[0]);
    store_a(j0);
    store_b(bpc[0], bt);
    __syncthreads();
    if (kw < K)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) product(nb, acc[nb], bt);
    __syncthreads();
  }
  load_a(j0);
#pragma unroll
  for (int i = 0; i < PT; ++i)
    if (t_begin + i < t_end) load_b(j0, (t_begin + i) * kMN, bpc[i]);
  load_codes(t_begin, cw, av);
  store_a(j0);
#pragma unroll
  for (int i = 0; i < PT; ++i)
    if (t_begin + i < t_end) store_b(bpc[i], bt + i * kMN * RS);
  __syncthreads();
  if (kw >= K) return;
  const unsigned char* lutb = reinterpret_cast<const unsigned char*>(lut);
  for (int t = t_begin; t < t_end; ++t) {
    const int n0 = t * kMN;
    const uint16_t* btt = bt + (t - t_begin) * kMN * RS;
    if (t > t_begin) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        cw[nb] = cwn[nb];
        av[nb] = avn[nb];
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[nb][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    load_codes(t + 1, cwn, avn);

  // ---- 3. the elements: lane (l16, g) holds column 32 (b >> 1) + 8 g + 4 (b & 1) + e
  // of row n in acc[nb][b][e]; v[i] is column 8 g + i (i < 8) or 32 + 8 g + i - 8,
  // i.e. acc[nb][i >> 2][i & 3]
  unsigned char* const wo = wout + wave * 16 * kWRow;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    product(nb, acc[nb], btt);
    const float sc = av[nb];
    const uint32_t w2[2] = {cw[nb].x, cw[nb].y};
    float v[16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // 8 codes per dword, the even element in the low nibble
      uint32_t ev = (w2[h] << 2) & 0x3C3C3C3Cu, od = (w2[h] >> 2) & 0x3C3C3C3Cu;
      asm volatile("" : "+v"(ev), "+v"(od));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i0 = 8 * h + 2 * j, i1 = i0 + 1;
        v[i0] = __fmul_rn(*reinterpret_cast<const float*>(lutb + __builtin_amdgcn_ubfe(ev, 8 * j, 8)), sc) +
                s * acc[nb][i0 >> 2][i0 & 3];
        v[i1] = __fmul_rn(*reinterpret_cast<const float*>(lutb + __builtin_amdgcn_ubfe(od, 8 * j, 8)), sc) +
                s * acc[nb][i1 >> 2][i1 & 3];
      }
    }
    // row l16 of the wave's LDS rows: columns 8 g .. 8 g + 7 and 32 + 8 g .. +7
    unsigned char* wr = wo + l16 * kWRow;
    if constexpr (OUT_BF16) {
      *reinterpret_cast<uint4*>(wr + 16 * g) = uint4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                    pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
      *reinterpret_cast<uint4*>(wr + 64 + 16 * g) = uint4{pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]),
                                                         pack_bf16x2(v[12], v[13]), pack_bf16x2(v[14], v[15])};
    } else {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4*>(wr + 128 * (q4 >> 1) + 32 * g + 16 * (q4 & 1)) =
            float4{v[4 * q4], v[4 * q4 + 1], v[4 * q4 + 2], v[4 * q4 + 3]};
    }
    // the wave's LDS writes land before its lanes read each other's values
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // each store instruction: 64 * 16 / (64 kOutB) rows, whole 64-column segments
    constexpr int kLanesRow = 64 * kOutB / 16, kRowsIns = 64 / kLanesRow;
#pragma unroll
    for (int h = 0; h < 16 / kRowsIns; ++h) {
      const int rr = kRowsIns * h + lane / kLanesRow, ch = lane % kLanesRow;
      const uint4 val = *reinterpret_cast<const uint4*>(wo + rr * kWRow + 16 * ch);
      const int n = n0 + 16 * nb + rr;
      if (n < N)
        *reinterpret_cast<uint4*>(static_cast<unsigned char*>(out) +
                                  (static_cast<size_t>(n) * K + kw) * kOutB + 16 * ch) = val;
    }
    // every lane has read the rows before the next n-block overwrites them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  }
}

// Tiles per workgroup: a run of at most PT tiles of its k-block (PT bounds the LDS
// of the staged B). Small weights take the PT = 2 instance (about 40 KB of LDS at
// r <= 32: four workgroups per CU) with one or two tiles per workgroup and up to
// 1024 workgroups; large ones PT = 8 (two workgroups per CU) with 512 workgroups
// and longer runs. One tile each when r needs several rank passes.
template <int RP, int PT, bool MP>
hipError_t launch_merge_pt(int K, int N, int r, float s, int per, const uint8_t* codes, const float* absmax,
                           const uint16_t* A, const uint16_t* B, bool out_bf16, void* out, hipStream_t stream) {
  const int kb = (K + kMK - 1) / kMK, nt = (N + kMN - 1) / kMN;
  const dim3 grid(kb, (nt + per - 1) / per);
  if (out_bf16)
    lora_merge_kernel<RP, PT, true, MP><<<grid, kThreads, 0, stream>>>(K, N, r, s, per, codes, absmax, A, B, out);
  else
    lora_merge_kernel<RP, PT, false, MP><<<grid, kThreads, 0, stream>>>(K, N, r, s, per, codes, absmax, A, B, out);
  return hipGetLastError();
}

template <int RP, bool MP = false>
hipError_t launch_merge_t(int K, int N, int r, float s, const uint8_t* codes, const float* absmax,
                          const uint16_t* A, const uint16_t* B, bool out_bf16, void* out,
                          hipStream_t stream) {
  const int tiles = ((K + kMK - 1) / kMK) * ((N + kMN - 1) / kMN);
  if constexpr (MP) {
    return launch_merge_pt<RP, 1, MP>(K, N, r, s, 1, codes, absmax, A, B, out_bf16, out, stream);
  } else {
    if constexpr (RP <= 32)
      if (tiles >= 512 * 8)
        return launch_merge_pt<RP, 8, MP>(K, N, r, s, 8, codes, absmax, A, B, out_bf16, out, stream);
    const int per = tiles >= 2048 ? 2 : 1;
    return launch_merge_pt<RP, 2, MP>(K, N, r, s, per, codes, absmax, A, B, out_bf16, out, stream);
  }
}

}  // namespace

hipError_t launch_lora_merge(int K, int N, int r, float s, const uint8_t* codes, const float* absmax,
                             const uint16_t* A, const uint16_t* B, bool out_bf16, void* out,
                             hipStream_t stream) {
  switch ((r + 31) / 32) {
    case 1: return launch_merge_t<32>(K, N, r, s, codes, absmax, A, B, out_bf16, out, stream);
    case 2: return launch_merge_t<64>(K, N, r, s, codes, absmax, A, B, out_bf16, out, stream);
    case 3: return launch_merge_t<96>(K, N, r, s, codes, absmax, A, B, out_bf16, out, stream);
    case 4: return launch_merge_t<128>(K, N, r, s, codes, absmax, A, B, out_bf16, out, stream);
    default: return launch_merge_t<128, true>(K, N, r, s, codes, absmax, A, B, out_bf16, out, stream);
  }
}

}  // namespace lnf4
