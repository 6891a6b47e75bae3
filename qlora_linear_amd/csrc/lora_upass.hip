// U = x A for the LoRA down-projection of one or several projections that read
// the same x (gfx950), ahead of the register-dequantizing forward, whose epilogue
// adds bf16(s U) B:
//     us[t][g r + j] = bf16(s U_g[t][j]),  u_save_g[t][j] = bf16(U_g[t][j])
// with U_g = x A_g and the projections' ranks side by side (R = n r <= 64 columns;
// for q/k/v at rank 16 one pass over x serves all three).
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

// AR: rows of the staged A^T slice (the rank sum padded to 16, 32 or 64); NS: ring
// stages. A stage is 256 columns: x [32 rows][256] and A^T [AR][256], rows of 512
// bytes whose 16-byte chunks are XOR-swizzled by row & 15 (32 rows reading one
// logical chunk then hit every bank once per 16 rows). Each 1 KB direct-to-LDS load
// covers two rows x 512 contiguous bytes (runs of 128 bytes read HBM at about 60 %
// of the rate of 512-byte runs). Wave w multiplies columns 64 w .. 64 w + 63 of
// every stage; one barrier per stage.
template <int AR, int NS>
__global__ __launch_bounds__(kThreads) void lora_upass_kernel(int T, int K, int r, float s, const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ at, UpassTable tab) {
  constexpr int kX = kRows * 256, kStage = (kRows + AR) * 256;  // elements
  constexpr int NU = (AR + 31) / 32;                             // 32-column rank blocks
  __shared__ __align__(16) uint16_t ring[NS * kStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int m0 = blockIdx.x * kRows;
  const int rows = min(T - m0, kRows);
  const int R = tab.n * r, nst = K / 256;  // K % 256 == 0
  const auto rs_x = make_rsrc(x + static_cast<size_t>(m0) * K, static_cast<uint32_t>(rows) * K * 2);
  const auto rs_a = make_rsrc(at, static_cast<uint32_t>(R) * K * 2);  // rows past R read zeros
  // load q of a wave covers tile rows 2 (4 w + q) and + 1 (x, then A^T): lane i ->
  // physical chunk i & 31 of row 2 (4 w + q) + (i >> 5), holding the logical chunk
  // (i & 31) ^ (row & 15)
  auto voff = [&](int q) {
    const int row = 2 * (4 * wave + q) + (lane >> 5);
    return static_cast<uint32_t>(row) * K * 2 + (((lane & 31) ^ (row & 15)) << 4);
  };
  constexpr int kXL = kRows / 8, kAL = AR / 8;  // loads per wave per stage (two rows each)
  uint32_t xvo[kXL], avo[kAL];
#pragma unroll
  for (int q = 0; q < kXL; ++q) xvo[q] = voff(q);
  // A^T: wave w loads slice rows AR / 4 w .. AR / 4 (w + 1) - 1
  constexpr int kAW = AR / 4;
#pragma unroll
  for (int q = 0; q < kAL; ++q) {
    const int row = kAW * wave + 2 * q + (lane >> 5);
    avo[q] = static_cast<uint32_t>(row) * K * 2 + (((lane & 31) ^ (row & 15)) << 4);
  }
  auto load_stage = [&](int i, int slot) {
    const uint32_t soff = static_cast<uint32_t>(min(i, nst - 1)) * 512;  // clamped: past the end, reload the last
    uint16_t* dst = ring + slot * kStage;
#pragma unroll
    for (int q = 0; q < kXL; ++q) buf_load16_lds(rs_x, dst + (2 * (4 * wave_u + q)) * 256, xvo[q], soff);
#pragma unroll
    for (int q = 0; q < kAL; ++q) buf_load16_lds(rs_a, dst + kX + (kAW * wave_u + 2 * q) * 256, avo[q], soff);
  };
  int choff[4], boff[4];  // x rows l32; A^T rows l32 (rows past AR read row l32 % AR, zeroed)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    choff[ks] = l32 * 256 + (((8 * wave + 2 * ks + hh) ^ (l32 & 15)) << 3);
    const int ar = AR < 32 ? (l32 & (AR - 1)) : l32;
    boff[ks] = ar * 256 + (((8 * wave + 2 * ks + hh) ^ (ar & 15)) << 3);
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
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 xa = *reinterpret_cast<const uint4*>(st + choff[ks]);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        uint4 b = *reinterpret_cast<const uint4*>(st + kX + 32 * u * 256 + boff[ks]);
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
          tab.us[static_cast<size_t>(row) * R + col] = to_bf16(s * v);
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
    lora_upass_kernel<16, 4><<<grid, kThreads, 0, stream>>>(T, K, r, s, x, at, tab);
  else if (R <= 32)
    lora_upass_kernel<32, 4><<<grid, kThreads, 0, stream>>>(T, K, r, s, x, at, tab);
  else if (R <= 64)
    lora_upass_kernel<64, 3><<<grid, kThreads, 0, stream>>>(T, K, r, s, x, at, tab);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lnf4
