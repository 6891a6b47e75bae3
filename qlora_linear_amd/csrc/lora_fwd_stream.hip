// Fused NF4-LoRA linear, forward, for a few tokens (T <= 32): a weight-streaming
// kernel (gfx950).
//
// With few tokens the linear is bound by reading the packed weight (0.5625 bytes
// per element: one nibble, plus a 4-byte absmax per 64 elements), not by
// arithmetic. The chain is the one the kernel-fusion section of "Unsloth
// acceleration principles: CUDA kernel fusion and memory optimization" describes
// (base linear, LoRA down-projection, LoRA up-projection, add), split along d_out
// only:
//   * one workgroup per 16 weight rows, over all of d_in; its W waves (3 to 8, as
//     many as the per-wave LDS stages allow) take the 128-element reduction
//     chunks w, w + W, w + 2 W, ... independently, with no barrier in the loop;
//   * each lane loads 16 bytes of codes (32 consecutive reduction elements of one
//     row) and dequantizes them straight into four v_mfma_f32_16x16x32_bf16
//     B fragments: the weight never passes through LDS;
//   * every workgroup reads all of x and A (a few token rows and the small LoRA
//     factor, L2-resident), so they are copied per wave and chunk into LDS with
//     contiguous direct-to-LDS loads: a lane-per-row fragment load from global
//     memory would touch four times the cache lines. x chunks are XOR-swizzled
//     for conflict-free 16-byte fragment reads; A chunks are read back transposed
//     (ds_read_b64_tr_b16), since MFMA operands need consecutive reduction
//     elements per lane and A is [d_in, r] row-major;
//   * U = x A accumulates from the same x fragments in every workgroup, which
//     keeps the launch free of workspace and of any synchronisation between
//     workgroups;
//   * the waves' partial sums meet in LDS and are summed by all threads; wave 0
//     adds bf16(s U) B with one more MFMA pass and stores y.
// Loads run ahead of use: codes by four chunks, the x and A chunks by one.
#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int kSRows = 16;   // weight rows (y columns) per workgroup
constexpr int kChunk = 128;  // reduction elements per wave step
constexpr uint32_t kXOut = 0x7FFFFFF0u;  // a per-lane offset past every buffer range: reads zeros

// TB: 16-token blocks (T <= 16 TB); RJ: 16-wide rank blocks (r <= 16 RJ).
template <int TB, int RJ>
struct StreamCfg {
  static constexpr int kRE = ((RJ * 16 + 31) / 32) * 32;   // rank padded to the epilogue MFMA depth
  static constexpr int kXCopy = 16 * TB * kChunk * 2;       // bytes of x copied per wave and chunk
  static constexpr int kACopy = kChunk * RJ * 16 * 2;       // bytes of A copied per wave and chunk
  static constexpr int kRegion = kXCopy + kACopy + 64;      // one wave's stage (x, then A)
  // waves per workgroup: as many as two stages per wave allow in ~150 KB of LDS
  static constexpr int kSWaves = 150000 / (2 * kRegion) > 8 ? 8 : 150000 / (2 * kRegion);
  static constexpr int kSThreads = kSWaves * 64;
  static constexpr int kStage = kSWaves * kRegion;
  static constexpr int kRedBytes = kSWaves * TB * (1 + RJ) * 4 * 64 * 4;
  static constexpr int kMain = 2 * kStage > kRedBytes ? 2 * kStage : kRedBytes;
  static constexpr int kES = kRE + 8;                       // epilogue row stride, bf16
  static constexpr int kBytes = kMain + (16 * TB + 16) * kES * 2;
  static_assert(kSWaves >= 2, "LDS stages");
};

template <int TB, int RJ>
__global__ __launch_bounds__((StreamCfg<TB, RJ>::kSThreads)) void lora_fwd_stream_kernel(
    int T, int K, int N, int r, float s, const uint16_t* __restrict__ x,
    const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ y,
    uint16_t* __restrict__ u_save) {
  using C = StreamCfg<TB, RJ>;
  constexpr int kSWaves = C::kSWaves, kSThreads = C::kSThreads;
  // level pairs of every code byte, (q[b & 15], q[b >> 4]) at 8 b: first in LDS, so
  // a table address needs no base
  __shared__ __align__(1024) float lut[512];
  __shared__ __align__(16) unsigned char smem[C::kBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * kSRows;
  const int K2 = K / 2, KB = K / 64;
  const int nch = (K + kChunk - 1) / kChunk;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int nw = nch > wave_u ? (nch - wave_u + kSWaves - 1) / kSWaves : 0;  // chunks of this wave

  for (int e = tid; e < 256; e += kSThreads) {
    lut[2 * e] = nf4_level_reg(e & 15);
    lut[2 * e + 1] = nf4_level_reg(e >> 4);
  }

  // Buffer resources: rows past N (codes, absmax), token rows past T (x) and rows
  // past d_in (A) read as zeros.
  const int rows_w = min(N - n0, kSRows);
  const auto rs_c = make_rsrc(codes + static_cast<size_t>(n0) * K2, static_cast<uint32_t>(rows_w) * K2);
  const auto rs_s = make_rsrc(absmax + static_cast<size_t>(n0) * KB, static_cast<uint32_t>(rows_w) * KB * 4);
  const auto rs_x = make_rsrc(x, static_cast<uint32_t>(T) * K * 2);
  const auto rs_a = make_rsrc(A, static_cast<uint32_t>(K) * r * 2);

  // Lane (l16, g) owns reduction elements 32 g .. 32 g + 31 of every chunk: codes
  // of weight row n0 + l16, and x of token rows 16 tb + l16. MFMA step q of a
  // chunk uses elements 32 g + 8 q .. +7, in both operands.
  const uint32_t cvoff = static_cast<uint32_t>(l16) * K2 + 16 * g;
  const uint32_t svoff = (static_cast<uint32_t>(l16) * KB + (g >> 1)) * 4;
  // x chunk in LDS: [16 TB rows][16 pieces of 8 elements], piece p of row t stored
  // at physical piece p ^ (t & 15). Copy instruction i fills rows 4 i .. 4 i + 3;
  // lane L lands on row 4 i + (L >> 4), physical piece L & 15, and loads the
  // logical piece stored there.
  uint32_t xvoff[4 * TB];
#pragma unroll
  for (int i = 0; i < 4 * TB; ++i) {
    const int t = 4 * i + (lane >> 4);
    const int p = (lane & 15) ^ (t & 15);
    xvoff[i] = static_cast<uint32_t>(t) * K * 2 + 16 * p;
  }
  // a lane's logical x piece for step q is 4 g + q, physical (4 g + q) ^ l16
  const int x_lane = l16 * kChunk * 2;

  unsigned char* const st0 = smem + wave_u * C::kRegion;
  unsigned char* const st1 = smem + C::kStage + wave_u * C::kRegion;
  // transposed A fragment: rows 32 g + 8 q + 4 h + (l16 >> 2) of the chunk, rank
  // columns 16 jb + 4 (l16 & 3) .. +3; lane l16 receives rank column 16 jb + l16
  const int a_lane = ((32 * g + (l16 >> 2)) * r + 4 * (l16 & 3)) * 2;
  const int a_rows4 = 8 * r;  // bytes of four A rows

  uint4 creg[4];
  float sreg[4];
  auto chunk_of = [&](int i) { return wave_u + kSWaves * i; };
  // Every chunk offset goes into the per-lane offset, which the buffer range check
  // covers: loads past the end of an operand (the run-ahead past the last chunk)
  // read zeros or bytes of the operand itself, never memory beyond it.
  auto load_codes = [&](int i, int slot) {
    const uint32_t c = static_cast<uint32_t>(chunk_of(i));
    creg[slot] = buf_load16(rs_c, cvoff + c * (kChunk / 2), 0);
    sreg[slot] = __uint_as_float(buf_load4(rs_s, svoff + c * (kChunk / 64) * 4, 0));
  };
  // x and A of one chunk into a stage: 4 TB + 4 RJ direct-to-LDS loads. Pieces of
  // x past d_in (the second half of a half-filled last chunk) read as zeros.
  auto load_stage = [&](int i, unsigned char* st) {
    const int c0 = chunk_of(i) * kChunk;
    const uint32_t xbase = static_cast<uint32_t>(c0) * 2;
#pragma unroll
    for (int q = 0; q < 4 * TB; ++q) {
      const int p = (lane & 15) ^ ((4 * q + (lane >> 4)) & 15);
      const uint32_t off = c0 + 8 * p < K ? xvoff[q] + xbase : kXOut;
      buf_load16_lds(rs_x, st + q * 1024, off, 0);
    }
    const uint32_t abase = static_cast<uint32_t>(c0) * r * 2 + lane * 16;
#pragma unroll
    for (int q = 0; q < C::kACopy / 1024; ++q)
      buf_load16_lds(rs_a, st + C::kXCopy + q * 1024, abase + q * 1024, 0);
  };

  const unsigned char* lutb = reinterpret_cast<const unsigned char*>(lut);
  auto dequant = [&](uint32_t w, float a) {
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

  f32x4_t acc[TB], uacc[TB][RJ];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jb = 0; jb < RJ; ++jb) uacc[tb][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // B^T of this block for the epilogue, loaded now so its latency hides under the loop
  constexpr int kBPer = (16 * C::kRE + kSThreads - 1) / kSThreads;
  uint16_t bval[kBPer];
#pragma unroll
  for (int i = 0; i < kBPer; ++i) {
    const int e = tid + i * kSThreads, n = e / C::kRE, j = e - n * C::kRE;
    bval[i] = (e < 16 * C::kRE && j < r && n0 + n < N) ? B[static_cast<size_t>(j) * N + n0 + n] : uint16_t(0);
  }

  __syncthreads();  // level table visible
  // prologue (issue order matters for the counted waits below): the stage of
  // chunk 0, then codes of chunks 0..3
  load_stage(0, st0);
#pragma unroll
  for (int d = 0; d < 4; ++d) load_codes(d, d);

  // One chunk. slot = i % 4 (codes ring), i % 2 selects the stage; the loop is
  // unrolled by four so both are compile-time.
  auto step = [&](int i, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    constexpr int xs = slot & 1;
    unsigned char* const cur = xs ? st1 : st0;
    const unsigned char* const a_cur = cur + C::kXCopy;
    load_stage(i + 1, xs ? st0 : st1);
    // the stage of chunk i has landed once at most the codes of chunk i + 3 and
    // the stage loads above are outstanding
    wait_vmem_upto<2 + C::kACopy / 1024 + 4 * TB>();
    const bool valid = chunk_of(i) * kChunk + 32 * g < K;  // false only in a half-filled last chunk
    uint4 wf[4];
    const uint32_t cw[4] = {creg[slot].x, creg[slot].y, creg[slot].z, creg[slot].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      wf[q] = dequant(cw[q], sreg[slot]);
      if (!valid) wf[q] = uint4{0u, 0u, 0u, 0u};
    }
    load_codes(i + 4, slot);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint4 af[RJ];
#pragma unroll
      for (int jb = 0; jb < RJ; ++jb) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(a_cur + a_lane + 2 * q * a_rows4 + 32 * jb);
        const uint2 lo = lds_read_tr16(p);
        const uint2 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(
            reinterpret_cast<const unsigned char*>(p) + a_rows4));
        af[jb] = uint4{lo.x, lo.y, hi.x, hi.y};
      }
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const uint4 xv = *reinterpret_cast<const uint4*>(cur + tb * 16 * kChunk * 2 + x_lane +
                                                         (((4 * g + q) ^ l16) << 4));
        acc[tb] = mfma16(xv, wf[q], acc[tb]);
#pragma unroll
        for (int jb = 0; jb < RJ; ++jb) uacc[tb][jb] = mfma16(xv, af[jb], uacc[tb][jb]);
      }
    }
  };
  for (int i = 0; i < nw; i += 4) {
    step(i, std::integral_constant<int, 0>{});
    if (i + 1 < nw) step(i + 1, std::integral_constant<int, 1>{});
    if (i + 2 < nw) step(i + 2, std::integral_constant<int, 2>{});
    if (i + 3 < nw) step(i + 3, std::integral_constant<int, 3>{});
  }
  // prefetches past the last chunk (direct-to-LDS ones included) must land before
  // the stages are reused for the reduction
  wait_vmem();
  __syncthreads();

  // ---- cross-wave reduction and epilogue ------------------------------------------
  float* red = reinterpret_cast<float*>(smem);  // [wave][TB (1 + RJ) 4][64]
  uint16_t* us = reinterpret_cast<uint16_t*>(smem + C::kMain);  // [16 TB][kES] bf16(s U)
  uint16_t* bt = us + 16 * TB * C::kES;                         // [16][kES] B^T of this block
  constexpr int kPer = TB * (1 + RJ) * 4;
  {
    float* dst = red + wave * kPer * 64 + lane;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dst[((tb * (1 + RJ)) * 4 + e) * 64] = acc[tb][e];
#pragma unroll
        for (int jb = 0; jb < RJ; ++jb) dst[((tb * (1 + RJ) + 1 + jb) * 4 + e) * 64] = uacc[tb][jb][e];
      }
  }
#pragma unroll
  for (int i = 0; i < kBPer; ++i) {
    const int e = tid + i * kSThreads, n = e / C::kRE, j = e - n * C::kRE;
    if (e < 16 * C::kRE) bt[n * C::kES + j] = bval[i];
  }
  __syncthreads();
  // every thread sums some of the kPer * 64 partials over the waves into wave 0's slot
  for (int e = tid; e < kPer * 64; e += kSThreads) {
    float v = red[e];
#pragma unroll
    for (int w = 1; w < kSWaves; ++w) v += red[w * kPer * 64 + e];
    red[e] = v;
  }
  __syncthreads();
  if (wave == 0) {
    const float* src = red + lane;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[tb][e] = src[((tb * (1 + RJ)) * 4 + e) * 64];
#pragma unroll
        for (int jb = 0; jb < RJ; ++jb) uacc[tb][jb][e] = src[((tb * (1 + RJ) + 1 + jb) * 4 + e) * 64];
      }
    // C layout: lane (l16, g) holds rows 4 g + e, column l16 of each 16 x 16 block
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * tb + 4 * g + e;
#pragma unroll
        for (int jb = 0; jb < RJ; ++jb) {
          const int j = 16 * jb + l16;
          const float uv = uacc[tb][jb][e];
          us[t * C::kES + j] = j < r ? to_bf16(s * uv) : uint16_t(0);
          if (u_save != nullptr && blockIdx.x == 0 && j < r && t < T)
            u_save[static_cast<size_t>(t) * r + j] = to_bf16(uv);
        }
        if constexpr (16 * RJ < C::kRE) us[t * C::kES + 16 * RJ + l16] = 0;
      }
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
      for (int jq = 0; jq < C::kRE / 32; ++jq) {
        const uint4 a = *reinterpret_cast<const uint4*>(us + (16 * tb + l16) * C::kES + 32 * jq + 8 * g);
        const uint4 b = *reinterpret_cast<const uint4*>(bt + l16 * C::kES + 32 * jq + 8 * g);
        acc[tb] = mfma16(a, b, acc[tb]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * tb + 4 * g + e, n = n0 + l16;
        if (t < T && n < N) y[static_cast<size_t>(t) * N + n] = to_bf16(acc[tb][e]);
      }
    }
  }
}

template <int TB, int RJ>
hipError_t launch_stream_t(int T, int K, int N, int r, float s, const uint16_t* x, const uint8_t* codes,
                           const float* absmax, const uint16_t* A, const uint16_t* B, uint16_t* y,
                           uint16_t* u_save, hipStream_t stream) {
  const int blocks = (N + kSRows - 1) / kSRows;
  lora_fwd_stream_kernel<TB, RJ><<<blocks, StreamCfg<TB, RJ>::kSThreads, 0, stream>>>(T, K, N, r, s, x, codes, absmax, A, B,
                                                                    y, u_save);
  return hipGetLastError();
}

}  // namespace

bool lora_fwd_stream_supported(int64_t T, int r) { return T >= 1 && T <= 32 && r % 8 == 0 && r <= 64; }

hipError_t launch_lora_fwd_stream(int T, int K, int N, int r, float s, const uint16_t* x,
                                  const uint8_t* codes, const float* absmax, const uint16_t* A,
                                  const uint16_t* B, uint16_t* y, uint16_t* u_save, hipStream_t stream) {
  const int rj = (r + 15) / 16;
  if (T <= 16) {
    switch (rj) {
      case 1: return launch_stream_t<1, 1>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
      case 2: return launch_stream_t<1, 2>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
      case 3: return launch_stream_t<1, 3>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
      default: return launch_stream_t<1, 4>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    }
  }
  switch (rj) {
    case 1: return launch_stream_t<2, 1>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    case 2: return launch_stream_t<2, 2>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    case 3: return launch_stream_t<2, 3>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
    default: return launch_stream_t<2, 4>(T, K, N, r, s, x, codes, absmax, A, B, y, u_save, stream);
  }
}

}  // namespace lnf4
