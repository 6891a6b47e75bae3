// U = x A for the LoRA down-projection of one or several projections that read
// the same x (gfx950), ahead of the register-dequantizing forward, whose epilogue
// adds bf16(s U) B:
//     us[t][g r + j] = bf16(s U_g[t][j]),  u_save_g[t][j] = bf16(U_g[t][j])
// with U_g = x A_g and the projections' ranks side by side (R = n r <= 256 columns:
// one pass over x serves q/k/v up to rank 64 each).
//
// The pass is bound by reading x once (2 T d_in bytes; d_in % 256 == 0). One
// workgroup per 32 token rows streams them, with the matching slices of A^T (R x
// d_in, transposed once per call by the first kernel below), through a ring of LDS
// stages of 256 columns; the four waves split every stage's columns and their
// partial sums meet in LDS at the end, added in a fixed order (deterministic).
#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 32;       // token rows per workgroup

// at[g r + j][k] = A_g[k][j] for every projection of the table.
__global__ __launch_bounds__(256) void transpose_a_table_kernel(UpassTable tab, int K, int r, uint16_t* __restrict__ at) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t R = static_cast<int64_t>(tab.n) * r;
  if (i >= R * K) return;
  const int row = static_cast<int>(i / K), k = static_cast<int>(i - static_cast<int64_t>(row) * K);
  const int g = row / r, j = row - g * r;
  at[i] = tab.A[g][static_cast<size_t>(k) * r + j];
}

// AR: rows of the staged A^T slice (the rank sum padded to 16, 32, 64, 128, 192 or
// 256); NS: ring stages; SC: columns per stage (256, or 128 for AR > 64 so that two
// stages fit the LDS). A stage is x [32 rows][SC] and A^T [AR][SC], rows whose
// 16-byte chunks are XOR-swizzled by row & 15 (32 rows reading one logical chunk
// then hit every bank once per 16 rows). Each 1 KB direct-to-LDS load covers 1024 /
// (2 SC) rows of 2 SC contiguous bytes. Wave w multiplies the 32-column groups w and
// w + 4 of every 256 columns; one barrier per stage.
template <int AR, int NS, int SC>
__global__ __launch_bounds__(kThreads) void lora_upass_kernel(int T, int K, int r, float s, const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ at, UpassTable tab) {
  constexpr int kX = kRows * SC, kStage = (kRows + AR) * SC;  // elements
  constexpr int NU = (AR + 31) / 32;                           // 32-column rank blocks
  constexpr int kRPL = 1024 / (2 * SC);                        // rows per 1 KB load
  constexpr int kCPR = SC / 8;                                 // 16-byte chunks per row
  constexpr int kKS = SC / 64;                                 // 16-wide k-slices per wave and stage
  __shared__ __align__(16) uint16_t ring[NS * kStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int m0 = blockIdx.x * kRows;
  const int rows = min(T - m0, kRows);
  const int R = tab.n * r, nst = K / SC;  // K % SC == 0
  const auto rs_x = make_rsrc(x + static_cast<size_t>(m0) * K, static_cast<uint32_t>(rows) * K * 2);
  const auto rs_a = make_rsrc(at, static_cast<uint32_t>(R) * K * 2);  // rows past R read zeros
  // load q of a wave covers kRPL tile rows from kRPL (4 w + q) (x, then A^T): lane i
  // -> physical chunk i % kCPR of row kRPL (4 w + q) + i / kCPR, holding the
  // logical chunk (i % kCPR) ^ (row & 15)
  auto voff = [&](int row) {
    return static_cast<uint32_t>(row) * K * 2 + (((lane % kCPR) ^ (row & 15)) << 4);
  };
  constexpr int kXL = kRows / kRPL / 4, kAL = AR / kRPL / 4;  // loads per wave per stage
  static_assert(kXL >= 1 && kAL >= 1 && kX % 512 == 0, "stage layout");
  uint32_t xvo[kXL], avo[kAL];
#pragma unroll
  for (int q = 0; q < kXL; ++q) xvo[q] = voff(kRPL * (kXL * wave + q) + lane / kCPR);
  // A^T: wave w loads slice rows AR / 4 w .. AR / 4 (w + 1) - 1
  constexpr int kAW = AR / 4;
#pragma unroll
  for (int q = 0; q < kAL; ++q) avo[q] = voff(kAW * wave + kRPL * q + lane / kCPR);
  // workgroup m starts at 256-column block m % (K / 256) and wraps around: the
  // workgroups in flight then read different columns of x and A^T (all starting at
  // column 0, their 8 KB-strided rows met in the same memory channels: 30 % slower
  // at 8192 x 4096, r = 64). The per-wave column order still depends only on K.
  const int rot = (static_cast<int>(blockIdx.x) % (K / 256)) * (256 / SC);
  auto load_stage = [&](int i, int slot) {
    int g = min(i, nst - 1) + rot;  // clamped: past the end, reload the last
    if (g >= nst) g -= nst;
    const uint32_t soff = static_cast<uint32_t>(g) * SC * 2;
    uint16_t* dst = ring + slot * kStage;
#pragma unroll
    for (int q = 0; q < kXL; ++q) buf_load16_lds(rs_x, dst + kRPL * (kXL * wave_u + q) * SC, xvo[q], soff);
#pragma unroll
    for (int q = 0; q < kAL; ++q) buf_load16_lds(rs_a, dst + kX + (kAW * wave_u + kRPL * q) * SC, avo[q], soff);
  };
  int choff[kKS], boff[kKS];  // x rows l32; A^T rows l32 (rows past AR read row l32 % AR, zeroed)
  // k-slice ks of a stage: 32-column group w + 4 (ks / 2) of each 256 columns, so
  // that every stage width gives each wave the same columns in the same order (one
  // pass over several projections then sums each U exactly as a pass of its own)
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    const int chunk = 16 * (ks / 2) + 4 * wave + 2 * (ks % 2) + hh;
    choff[ks] = l32 * SC + ((chunk ^ (l32 & 15)) << 3);
    const int ar = AR < 32 ? (l32 & (AR - 1)) : l32;
    boff[ks] = ar * SC + ((chunk ^ (ar & 15)) << 3);
  }

  f32x16_t acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[u][e] = 0.f;

#pragma unroll
  for (int p = 0; p < NS - 1; ++p) load_stage(p, p);
  for (int i = 0; i < nst; ++i) {
    wait_vmem_upto<(kXL + kAL) * (NS - 2)>();  // stage i has landed (the NS - 2 after it may not)
    __builtin_amdgcn_s_barrier();               // ... for every wave; and stage i - 1 is free
    load_stage(i + NS - 1, (i + NS - 1) % NS);
    const uint16_t* st = ring + (i % NS) * kStage;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const uint4 xa = *reinterpret_cast<const uint4*>(st + choff[ks]);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        uint4 b = *reinterpret_cast<const uint4*>(st + kX + 32 * u * SC + boff[ks]);
        if (AR < 32 && l32 >= AR) b = uint4{0u, 0u, 0u, 0u};  // rank rows past the staged slice
        acc[u] = mfma32(xa, b, acc[u]);
      }
    }
  }
  wait_vmem();  // the run-ahead loads have landed before the ring is reused
  __syncthreads();

  // fixed-order sum of the four waves' partials, 32 rank columns at a time; wave 0
  // rounds and stores
  float* red = reinterpret_cast<float*>(ring);  // [3][16][64]
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (wave_u > 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) red[((wave_u - 1) * 16 + e) * 64 + lane] = acc[u][e];
    }
    __syncthreads();
    if (wave_u == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float v = acc[u][e] + red[(0 * 16 + e) * 64 + lane] + red[(1 * 16 + e) * 64 + lane] +
                        red[(2 * 16 + e) * 64 + lane];
        const int row = m0 + mfma32_row(e, lane), col = 32 * u + l32;
        if (row < T && col < R) {
          tab.us[static_cast<size_t>(row) * (tab.us_stride > 0 ? tab.us_stride : R) + col] = to_bf16(s * v);
          const int g = col / r, j = col - g * r;
          if (tab.u[g] != nullptr) tab.u[g][static_cast<size_t>(row) * r + j] = to_bf16(v);
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace

size_t upass_table_bytes(int64_t T, int64_t K, int n, int r) {
  const auto al = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
  const size_t R = static_cast<size_t>(n) * r;
  return al(R * K * 2) + al(static_cast<size_t>(T) * R * 2);
}

hipError_t launch_upass(int T, int K, int r, float s, const uint16_t* x, UpassTable& tab, void* workspace,
                        hipStream_t stream) {
  const int R = tab.n * r;
  uint16_t* at = static_cast<uint16_t*>(workspace);
  tab.us = at + ((static_cast<size_t>(R) * K * 2 + 255) & ~static_cast<size_t>(255)) / 2;
  const int64_t n = static_cast<int64_t>(R) * K;
  transpose_a_table_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(tab, K, r, at);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned grid = static_cast<unsigned>((T + kRows - 1) / kRows);
  if (R <= 16)
    lora_upass_kernel<16, 4, 256><<<grid, kThreads, 0, stream>>>(T, K, r, s, x, at, tab);
  else if (R <= 32)
    lora_upass_kernel<32, 4, 256><<<grid, kThreads, 0, stream>>>(T, K, r, s, x, at, tab);
  else if (R <= 64)
    lora_upass_kernel<64, 3, 256><<<grid, kThreads, 0, stream>>>(T, K, r, s, x, at, tab);
  else if (R <= 128)
    lora_upass_kernel<128, 2, 128><<<grid, kThreads, 0, stream>>>(T, K, r, s, x, at, tab);
  else if (R <= 192)
    lora_upass_kernel<192, 2, 128><<<grid, kThreads, 0, stream>>>(T, K, r, s, x, at, tab);
  else if (R <= 256)
    lora_upass_kernel<256, 2, 128><<<grid, kThreads, 0, stream>>>(T, K, r, s, x, at, tab);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gpass(int T, int N, int r, float s, const uint16_t* dy, const uint16_t* B, uint16_t* g,
                        int g_stride, hipStream_t stream) {
  if (N % 256 != 0 || r > 64) return hipErrorInvalidValue;
  UpassTable tab{};
  tab.n = 1;
  tab.us = g;
  tab.us_stride = g_stride;
  const unsigned grid = static_cast<unsigned>((T + kRows - 1) / kRows);
  if (r <= 16)
    lora_upass_kernel<16, 4, 256><<<grid, kThreads, 0, stream>>>(T, N, r, s, dy, B, tab);
  else if (r <= 32)
    lora_upass_kernel<32, 4, 256><<<grid, kThreads, 0, stream>>>(T, N, r, s, dy, B, tab);
  else
    lora_upass_kernel<64, 3, 256><<<grid, kThreads, 0, stream>>>(T, N, r, s, dy, B, tab);
  return hipGetLastError();
}

}  // namespace lnf4
