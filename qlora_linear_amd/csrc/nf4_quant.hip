// NF4 blockwise quantization and dequantization kernels (gfx950).
//
// The pages keep the frozen base weight in 4-bit NF4 form ("Unsloth
// acceleration principles: CUDA kernel fusion and memory optimization",
// kernel-fusion section, load_in_4bit=True; "Reading the Unsloth changelog",
// section 1.1). Both kernels are HBM-bound elementwise passes: quantization runs
// once per weight; dequantization to bf16 runs once per forward or backward call
// at large token counts, where the tile kernels then read bf16 weight tiles.
#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

// Decision thresholds between neighbouring levels, exact in float64.
__device__ __forceinline__ double nf4_midpoint(int i) {
  return 0.5 * (static_cast<double>(nf4_level(i)) + static_cast<double>(nf4_level(i + 1)));
}

// Code of w in a block of absmax a > 0: the number of thresholds w reaches,
// i.e. the nearest level to w / a with ties going up. m_i * a is exact in
// float64 (at most 27 + 24 significant bits), so each comparison is exact.
__device__ __forceinline__ uint32_t nf4_code(float w, float a) {
  if (a == 0.0f) return 7u;
  const double wd = w, ad = a;
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) c += (wd >= nf4_midpoint(i) * ad) ? 1u : 0u;
  return c;
}

__device__ __forceinline__ float load_elem(const float* w, int64_t i) { return w[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* w, int64_t i) { return bf16_to_f32(w[i]); }

// One thread per output byte (two elements). A 64-element block is 32
// consecutive threads — half a wavefront — so the absmax is a 32-lane
// butterfly max. The byte count is a multiple of 32, so every half-wave is
// either fully in range or fully out of it.
template <typename In>
__global__ __launch_bounds__(256) void nf4_quantize_kernel(const In* __restrict__ w, int64_t nbytes,
                                                           uint8_t* __restrict__ codes,
                                                           float* __restrict__ absmax) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= nbytes) return;
  const float w0 = load_elem(w, 2 * i), w1 = load_elem(w, 2 * i + 1);
  float m = fmaxf(fabsf(w0), fabsf(w1));
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 32));
  const uint32_t c0 = nf4_code(w0, m), c1 = nf4_code(w1, m);
  codes[i] = static_cast<uint8_t>(c0 | (c1 << 4));
  if ((i & 31) == 0) absmax[i >> 5] = m;
}

// One thread per dword of codes (8 elements of one block). Output: the product
// level * absmax, one float32 rounding; bf16 output rounds that float32 again.
// Dequantization: code word (8 elements, one 64-element block per 8 words) w
// of a workgroup's 4 x 256 words is handled by thread w % 256, so each load and
// store instruction covers consecutive words across the wave and every thread
// has four independent loads in flight. Levels come from a 16-entry LDS table.
constexpr int kDqWords = 4;
template <bool BF16>
__global__ __launch_bounds__(256) void nf4_dequantize_kernel(const uint32_t* __restrict__ codes,
                                                             const float* __restrict__ absmax,
                                                             int64_t ndw, void* __restrict__ out) {
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = nf4_level_reg(threadIdx.x);
  __syncthreads();
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 256 * kDqWords; base < ndw;
       base += static_cast<int64_t>(gridDim.x) * 256 * kDqWords) {
    uint32_t c[kDqWords];
    float a[kDqWords];
#pragma unroll
    for (int q = 0; q < kDqWords; ++q) {
      const int64_t i = base + q * 256 + threadIdx.x;
      c[q] = i < ndw ? codes[i] : 0u;
      a[q] = i < ndw ? absmax[i >> 3] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < kDqWords; ++q) {
      const int64_t i = base + q * 256 + threadIdx.x;
      if (i >= ndw) continue;
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = lut[(c[q] >> (4 * j)) & 15u] * a[q];
      if constexpr (BF16) {
        reinterpret_cast<uint4*>(out)[i] = uint4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                 pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
      } else {
        float4* o = reinterpret_cast<float4*>(out) + 2 * i;
        o[0] = make_float4(v[0], v[1], v[2], v[3]);
        o[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
}

}  // namespace

hipError_t launch_nf4_quantize(const void* w, bool w_is_bf16, int64_t rows, int64_t cols,
                               uint8_t* codes, float* absmax, hipStream_t stream) {
  const int64_t nbytes = rows * cols / 2;
  const dim3 grid(static_cast<unsigned>((nbytes + 255) / 256));
  if (w_is_bf16)
    nf4_quantize_kernel<uint16_t><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(w), nbytes,
                                                            codes, absmax);
  else
    nf4_quantize_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(w), nbytes, codes,
                                                         absmax);
  return hipGetLastError();
}

hipError_t launch_nf4_dequantize(const uint8_t* codes, const float* absmax, int64_t rows,
                                 int64_t cols, bool out_bf16, void* out, hipStream_t stream) {
  const int64_t ndw = rows * cols / 8;
  int64_t blocks = (ndw + 256 * kDqWords - 1) / (256 * kDqWords);
  if (blocks > 65536) blocks = 65536;  // the kernel strides over the rest
  const dim3 grid(static_cast<unsigned>(blocks));
  if (out_bf16)
    nf4_dequantize_kernel<true><<<grid, 256, 0, stream>>>(reinterpret_cast<const uint32_t*>(codes), absmax,
                                                          ndw, out);
  else
    nf4_dequantize_kernel<false><<<grid, 256, 0, stream>>>(reinterpret_cast<const uint32_t*>(codes), absmax,
                                                           ndw, out);
  return hipGetLastError();
}

namespace {
// codes [N][K/2] -> codes^T [K][N/2] and absmax [N][K/64] -> absmax^T [K/64][N]. A
// 256-thread workgroup takes 128 weight rows x 128 columns: thread (g, c) reads
// the code dwords of rows 8 g .. 8 g + 7 at dword column c (8 columns each, 64
// bytes of a row per 16 threads), transposes the 8 x 8 nibbles in registers and
// stages them in LDS, from where each thread stores 32 bytes of one codes^T row.
__global__ __launch_bounds__(256) void nf4_transpose_kernel(const uint32_t* __restrict__ codes,
                                                            const float* __restrict__ absmax, int N, int K,
                                                            uint32_t* __restrict__ codes_t,
                                                            float* __restrict__ absmax_t) {
  __shared__ uint32_t tile[128 * 17];  // [column][row group of 8], padded
  const int tid = threadIdx.x, g = tid >> 4, c = tid & 15;
  const int n0 = blockIdx.y * 128, k0 = blockIdx.x * 128;
  const int kw = K / 8, nw = N / 8;  // dwords per row of codes, of codes^T
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = codes[static_cast<size_t>(n0 + 8 * g + i) * kw + k0 / 8 + c];
  // w[i] nibble j = code(n0 + 8 g + i, k0 + 8 c + j)  ->  o[j] nibble i
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t o = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) o |= ((w[i] >> (4 * j)) & 15u) << (4 * i);
    tile[(8 * c + j) * 17 + g] = o;
  }
  {  // absmax: 128 rows x 2 blocks
    const int n = tid & 127, kb = tid >> 7;
    absmax_t[static_cast<size_t>(k0 / 64 + kb) * N + n0 + n] = absmax[static_cast<size_t>(n0 + n) * (K / 64) + k0 / 64 + kb];
  }
  __syncthreads();
  const int row = tid >> 1, half = tid & 1;  // codes^T row k0 + row, dwords 8 half .. +7 of the block
  uint32_t v[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = tile[row * 17 + 8 * half + q];
  uint4* dst = reinterpret_cast<uint4*>(codes_t + static_cast<size_t>(k0 + row) * nw + n0 / 8 + 8 * half);
  dst[0] = uint4{v[0], v[1], v[2], v[3]};
  dst[1] = uint4{v[4], v[5], v[6], v[7]};
}

__global__ void zero_u16_kernel(uint16_t* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0;
}
}  // namespace

hipError_t launch_nf4_transpose(const uint8_t* codes, const float* absmax, int64_t N, int64_t K,
                                uint8_t* codes_t, float* absmax_t, hipStream_t stream) {
  if (N % 128 != 0 || K % 128 != 0) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(K / 128), static_cast<unsigned>(N / 128));
  nf4_transpose_kernel<<<grid, 256, 0, stream>>>(reinterpret_cast<const uint32_t*>(codes), absmax,
                                                 static_cast<int>(N), static_cast<int>(K),
                                                 reinterpret_cast<uint32_t*>(codes_t), absmax_t);
  return hipGetLastError();
}

hipError_t launch_zero_u16(uint16_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  zero_u16_kernel<<<static_cast<unsigned>(blocks < 4096 ? blocks : 4096), 256, 0, stream>>>(p, n);
  return hipGetLastError();
}

}  // namespace lnf4
