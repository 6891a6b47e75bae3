// Fused NF4-LoRA linear, backward input gradient for a few tokens (T <= 32):
//     G  = s dY B^T,   dX = dY deq(Wt) + G A^T
// (the hand-written backward of "Unlocking AI potential: Unsloth's algorithms and
// implementation", core-algorithms section), split for weight streaming (gfx950).
//
// With few tokens the product is bound by reading the packed weight, so the
// work is split over the weight itself: workgroup (kb, sp) owns d_in columns
// 256 kb .. 256 kb + 255 and the d_out slice sp. Per 64-row step it
//   * dequantizes the 64 x 256 NF4 tile (half an NF4 block per thread) into one
//     of three LDS tiles in natural row-major order (loads run two steps ahead), and
//   * reads it back transposed with ds_read_b64_tr_b16 as v_mfma_f32_16x16x32_bf16
//     B fragments (the reduction runs along the weight's rows here) against dY
//     fragments loaded straight from global memory (a few token rows);
// wave 0 of the first column block also accumulates G over the slice from the
// same dY fragments and rows of B (contiguous along d_out). The slices' fp32
// partial sums go to the workspace; a second kernel adds them in a fixed order
// (bitwise reproducible), rounds G to bf16 like the tiled path, adds G A^T and
// stores dX and G.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int kThreads = 256;   // reduce kernel
constexpr int kXThreads = 512;  // streaming kernel: 8 waves, 32 d_in columns each
constexpr int kKB = 256;       // d_in columns per workgroup
constexpr int kNS = 64;        // d_out rows per step
constexpr int kDS = kKB + 16;  // LDS row stride of the dequantized tile, bf16 (+32 B)
constexpr uint32_t kOut = 0x7FFFFFF0u;  // a per-lane offset past every buffer range: reads zeros

template <int TB, int RJ>
__global__ __launch_bounds__(kXThreads) void lora_dx_stream_kernel(
    int T, int K, int N, int r, int rows_per_split, const uint16_t* __restrict__ dy,
    const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
    const uint16_t* __restrict__ B, float* __restrict__ part_x, float* __restrict__ part_g) {
  __shared__ __align__(1024) float lut[16];  // first in LDS: level addresses need no base
  __shared__ __align__(16) uint16_t ds0[kNS * kDS];
  __shared__ __align__(16) uint16_t ds1[kNS * kDS];
  __shared__ __align__(16) uint16_t ds2[kNS * kDS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int kb = blockIdx.x, sp = blockIdx.y;
  const int k0 = kb * kKB, nbeg = sp * rows_per_split;
  const int nend = min(N, nbeg + rows_per_split);
  const int steps = (nend - nbeg + kNS - 1) / kNS;
  const int K2 = K / 2, KB = K / 64;
  const bool with_g = kb == 0 && wave == 0;  // wave-uniform

  if (tid < 16) lut[tid] = nf4_level(tid);

  // Buffer resources over whole operands: rows past d_out (codes, absmax), token
  // rows past T (dY) and rank rows past r (B) read as zeros. Columns past d_in
  // or d_out stay inside a row, so those are masked explicitly.
  const auto rs_c = make_rsrc(codes, static_cast<uint32_t>(static_cast<size_t>(N) * K2));
  const auto rs_s = make_rsrc(absmax, static_cast<uint32_t>(static_cast<size_t>(N) * KB * 4));
  const auto rs_y = make_rsrc(dy, static_cast<uint32_t>(T) * N * 2);
  const auto rs_b = make_rsrc(B, static_cast<uint32_t>(r) * N * 2);

  // codes: thread (nl, cb) owns row nbeg + 64 st + nl, columns k0 + 32 cb .. +31
  // (16 bytes, half an NF4 block)
  const int nl = tid >> 3, cb = tid & 7;
  const bool kval = k0 + 32 * cb < K;
  const uint32_t cvoff = static_cast<uint32_t>(nbeg + nl) * K2 + (k0 + 32 * cb) / 2;
  const uint32_t svoff = (static_cast<uint32_t>(nbeg + nl) * KB + (k0 + 32 * cb) / 64) * 4;
  // dY fragment of step st, half q: lane (l16, g) holds dY[16 tb + l16][n .. n + 7],
  // n = nbeg + 64 st + 32 q + 8 g; B fragment likewise for rank row 16 jb + l16
  uint32_t yvoff[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) yvoff[tb] = static_cast<uint32_t>(16 * tb + l16) * N * 2;
  // every wave issues the B loads (uniform load counts, no branch around them);
  // waves that do not accumulate G point them past the range, reading zeros
  uint32_t bvoff[RJ];
#pragma unroll
  for (int jb = 0; jb < RJ; ++jb) bvoff[jb] = with_g ? static_cast<uint32_t>(16 * jb + l16) * N * 2 : kOut;

  uint4 creg[3];
  float sreg[3];
  uint4 yf[3][TB][2], bf[3][RJ][2];
  auto load = [&](int st, int slot) {
    const uint32_t row = static_cast<uint32_t>(st) * kNS;
    creg[slot] = buf_load16(rs_c, cvoff + row * K2, 0);
    sreg[slot] = __uint_as_float(buf_load4(rs_s, svoff + row * KB * 4, 0));
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int n = nbeg + st * kNS + 32 * q + 8 * g;
      const bool nval = n < N;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const uint4 v = buf_load16(rs_y, yvoff[tb] + n * 2, 0);
        yf[slot][tb][q] = nval ? v : uint4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int jb = 0; jb < RJ; ++jb) {
        const uint4 v = buf_load16(rs_b, with_g ? bvoff[jb] + n * 2 : kOut, 0);
        bf[slot][jb][q] = nval ? v : uint4{0u, 0u, 0u, 0u};
      }
    }
  };

  const unsigned char* lutb = reinterpret_cast<const unsigned char*>(lut);
  auto dequant_store = [&](uint32_t w, float a, uint16_t* dst) {
    uint32_t ev = (w << 2) & 0x3C3C3C3Cu, od = (w >> 2) & 0x3C3C3C3Cu;
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
    *reinterpret_cast<uint4*>(dst) = o;
  };
  const int dw_off = nl * kDS + 32 * cb;  // + 8 i
  // transposed B fragment of the weight tile: rows 32 q + 8 g + 4 h + (l16 >> 2),
  // columns 32 wave + 16 c + 4 (l16 & 3) .. +3; lane l16 receives column 16 c + l16
  const int d_off = (8 * g + (l16 >> 2)) * kDS + 32 * wave + 4 * (l16 & 3);

  f32x4_t acc[TB][2], gacc[TB][RJ];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[tb][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jb = 0; jb < RJ; ++jb) gacc[tb][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  load(0, 0);
  load(1, 1);  // past the last step these loads read unused bytes or zeros
  __syncthreads();  // level table visible

  // One 64-row step; slot = st % 3 for registers and LDS tile (the loop is
  // unrolled by three). Per step a wave issues 2 + 2 TB + 2 RJ loads.
  constexpr int kPerStep = 2 + 2 * TB + 2 * RJ;
  static_assert(kPerStep < 64, "vmcnt");
  auto step = [&](int st, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    uint16_t* dcur = slot == 0 ? ds0 : (slot == 1 ? ds1 : ds2);
    // this step's loads have landed once at most the next step's are outstanding
    wait_vmem_upto<kPerStep>();
    {
      const uint32_t cw[4] = {creg[slot].x, creg[slot].y, creg[slot].z, creg[slot].w};
      // a block past d_in gets scale 0: its (in-range, unrelated) codes dequantize to zeros
      const float a = kval ? sreg[slot] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) dequant_store(cw[i], a, dcur + dw_off + 8 * i);
    }
    load(st + 2, (slot + 2) % 3);
    __syncthreads();  // tile visible; its previous readers (step st - 3) are long done
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint16_t* p = dcur + d_off + 32 * q * kDS + 16 * c;
        const uint2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 4 * kDS);
        const uint4 wfr = uint4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[tb][c] = mfma16(yf[slot][tb][q], wfr, acc[tb][c]);
      }
      if (with_g) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int jb = 0; jb < RJ; ++jb) gacc[tb][jb] = mfma16(yf[slot][tb][q], bf[slot][jb][q], gacc[tb][jb]);
      }
    }
  };
  for (int st = 0; st < steps; st += 3) {
    step(st, std::integral_constant<int, 0>{});
    if (st + 1 < steps) step(st + 1, std::integral_constant<int, 1>{});
    if (st + 2 < steps) step(st + 2, std::integral_constant<int, 2>{});
  }
  wait_vmem();  // no load outlives the workgroup's registers' last use

  // C layout: lane (l16, g) holds rows 4 g + e, column l16 of each 16 x 16 block
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * tb + 4 * g + e;
      if (t >= T) continue;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int k = k0 + 32 * wave + 16 * c + l16;
        if (k < K) part_x[(static_cast<size_t>(sp) * T + t) * K + k] = acc[tb][c][e];
      }
      if (with_g) {
#pragma unroll
        for (int jb = 0; jb < RJ; ++jb) {
          const int j = 16 * jb + l16;
          if (j < r) part_g[(static_cast<size_t>(sp) * T + t) * r + j] = gacc[tb][jb][e];
        }
      }
    }
}

// dX = sum of the slices' partials + bf16(G) A^T, G = bf16(s * sum of G partials).
// Each thread owns 4 consecutive outputs of a token row (K % 64 == 0); its partial
// sums are loaded before the G phase so both latencies overlap. Every workgroup
// forms G (T r values) in LDS; the first one also stores it.
__global__ __launch_bounds__(kThreads) void lora_dx_stream_reduce(
    int T, int K, int r, int S, float s, const float* __restrict__ part_x,
    const float* __restrict__ part_g, const uint16_t* __restrict__ A, uint16_t* __restrict__ dx,
    uint16_t* __restrict__ g_out) {
  __shared__ float gs[32 * 64];
  const int tid = threadIdx.x;
  const int64_t i4 = (static_cast<int64_t>(blockIdx.x) * kThreads + tid) * 4;
  const int64_t TK = static_cast<int64_t>(T) * K;
  const bool act = dx != nullptr && i4 < TK;
  float4 v = {0.f, 0.f, 0.f, 0.f};
  // partials in batches of 8 independent loads (a plain loop waits on each load)
  if (act) {
    for (int p0 = 0; p0 < S; p0 += 8) {
      float4 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        w[u] = p0 + u < S ? *reinterpret_cast<const float4*>(part_x + (p0 + u) * TK + i4)
                          : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v.x += w[u].x; v.y += w[u].y; v.z += w[u].z; v.w += w[u].w;
      }
    }
  }
  for (int e = tid; e < T * r; e += kThreads) {
    float gv = 0.f;
    for (int p0 = 0; p0 < S; p0 += 8) {
      float w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = p0 + u < S ? part_g[static_cast<size_t>(p0 + u) * T * r + e] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) gv += w[u];
    }
    const uint16_t gb = to_bf16(s * gv);
    gs[e] = bf16_to_f32(gb);
    if (blockIdx.x == 0) g_out[e] = gb;
  }
  __syncthreads();
  if (!act) return;
  const int t = static_cast<int>(i4 / K), k = static_cast<int>(i4 - static_cast<int64_t>(t) * K);
  float o[4] = {v.x, v.y, v.z, v.w};
  const float* gt = gs + t * r;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint16_t* ar = A + static_cast<size_t>(k + c) * r;
    for (int j = 0; j < r; j += 8) {  // r % 8 == 0: 16-byte pieces of A's rows
      const uint4 a8 = *reinterpret_cast<const uint4*>(ar + j);
      const uint32_t aw[4] = {a8.x, a8.y, a8.z, a8.w};
#pragma unroll
      for (int h = 0; h < 8; ++h)
        o[c] += gt[j + h] * bf16_to_f32(static_cast<uint16_t>(aw[h >> 1] >> (16 * (h & 1))));
    }
  }
  uint2 packed;
  packed.x = pack_bf16x2(o[0], o[1]);
  packed.y = pack_bf16x2(o[2], o[3]);
  *reinterpret_cast<uint2*>(dx + i4) = packed;
}

template <int TB, int RJ>
hipError_t launch_t(int T, int K, int N, int r, float s, int S, int rows_per_split, const uint16_t* dy,
                    const uint8_t* codes, const float* absmax, const uint16_t* A, const uint16_t* B,
                    uint16_t* dx, uint16_t* g_out, float* part_x, float* part_g, hipStream_t stream) {
  const dim3 grid((K + kKB - 1) / kKB, S);
  lora_dx_stream_kernel<TB, RJ><<<grid, kXThreads, 0, stream>>>(T, K, N, r, rows_per_split, dy, codes,
                                                                absmax, B, part_x, part_g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t quads = static_cast<int64_t>(T) * K / 4;
  lora_dx_stream_reduce<<<static_cast<int>((quads + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
      T, K, r, S, s, part_x, part_g, A, dx, g_out);
  return hipGetLastError();
}

}  // namespace

bool lora_dx_stream_supported(int64_t T, int r) { return T >= 1 && T <= 32 && r % 8 == 0 && r <= 64; }

void dx_stream_split(int64_t K, int64_t N, int* splits, int* rows_per_split) {
  const int64_t kblocks = (K + kKB - 1) / kKB;
  int64_t want = (256 + kblocks - 1) / kblocks;
  const int64_t max_splits = (N + kNS - 1) / kNS;
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  int64_t per = (N + want - 1) / want;
  per = ((per + kNS - 1) / kNS) * kNS;
  *rows_per_split = static_cast<int>(per);
  *splits = static_cast<int>((N + per - 1) / per);
}

hipError_t launch_lora_dx_stream(int T, int K, int N, int r, float s, const uint16_t* dy,
                                 const uint8_t* codes, const float* absmax, const uint16_t* A,
                                 const uint16_t* B, uint16_t* dx, uint16_t* g_out, float* part_x,
                                 float* part_g, hipStream_t stream) {
  int S = 1, per = kNS;
  dx_stream_split(K, N, &S, &per);
  const int rj = (r + 15) / 16;
#define LNF4_DXS(TB_, RJ_)                                                                          \
  return launch_t<TB_, RJ_>(T, K, N, r, s, S, per, dy, codes, absmax, A, B, dx, g_out, part_x, part_g, \
                            stream)
  if (T <= 16) {
    switch (rj) {
      case 1: LNF4_DXS(1, 1);
      case 2: LNF4_DXS(1, 2);
      case 3: LNF4_DXS(1, 3);
      default: LNF4_DXS(1, 4);
    }
  }
  switch (rj) {
    case 1: LNF4_DXS(2, 1);
    case 2: LNF4_DXS(2, 2);
    case 3: LNF4_DXS(2, 3);
    default: LNF4_DXS(2, 4);
  }
#undef LNF4_DXS
}

}  // namespace lnf4
