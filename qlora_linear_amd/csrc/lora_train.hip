// Training-step companions of the fused NF4-LoRA linear (gfx950):
//
//  * adamw_kernel — the optimizer update of a LoRA factor. The pages time the
//    optimizer step as its own phase and run it as a GPU kernel with 16-bit
//    state ("Unsloth performance measured: is it really 2x faster?", section 2.2
//    time table and section 3). Decoupled weight decay (AdamW); float32 master
//    weights, bf16 copy for the GEMM kernels, bf16 moments. One pass reads and
//    writes every array once: bound by HBM.
//
//  * absmax double quantization — the float32 block scales of the NF4 weight
//    stored once more as 8-bit E4M3 codes with one float32 scale and offset per
//    256 block scales (QLoRA-style double quantization; the pages only fix that
//    the base weight stays resident in 4-bit form, "Reading the Unsloth
//    changelog", section 1.1). Per 256-block with minimum lo and maximum hi:
//        offset = f32(lo/2 + hi/2), d = max(f32(hi - offset), f32(offset - lo)),
//        scale = f32(d / 448), code = e4m3(f32(f32(a - offset) / scale))
//    and back a' = f32(f32(value(code) * scale) + offset). Every step is one
//    float32 operation with round-to-nearest-even and no contraction into a
//    fused multiply-add, so codes and scales are reproducible exactly.
#include <cmath>

#include "device_common.h"
#include "launch.h"

namespace lnf4 {
namespace {

// ---- AdamW ---------------------------------------------------------------------------

struct AdamWArgs {
  float beta1, one_m_beta1, beta2, one_m_beta2, eps;
  float decay;          // 1 - lr * weight_decay
  float step_size;      // lr / (1 - beta1^t)
  float inv_sqrt_bc2;   // 1 / sqrt(1 - beta2^t)
};

__device__ __forceinline__ void adamw_elem(const AdamWArgs& h, float g, float& p, float& m, float& v) {
  m = h.beta1 * m + h.one_m_beta1 * g;
  v = h.beta2 * v + h.one_m_beta2 * (g * g);
  const float denom = __fsqrt_rn(v) * h.inv_sqrt_bc2 + h.eps;
  p = p * h.decay - h.step_size * __fdiv_rn(m, denom);
}

constexpr int kAdamThreads = 256;

// Thread i owns elements 8 i .. 8 i + 7: 16-byte loads of the bf16 arrays and two
// float4 of the master copy. The last thread of a ragged length runs elementwise.
__global__ __launch_bounds__(kAdamThreads) void adamw_kernel(int64_t n, float* __restrict__ p,
                                                             uint16_t* __restrict__ p_bf16,
                                                             const uint16_t* __restrict__ g,
                                                             uint16_t* __restrict__ m,
                                                             uint16_t* __restrict__ v,
                                                             const AdamWArgs h) {
  const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * kAdamThreads + threadIdx.x) * 8;
  if (i0 >= n) return;
  if (i0 + 8 <= n) {
    const uint4 gq = *reinterpret_cast<const uint4*>(g + i0);
    const uint4 mq = *reinterpret_cast<const uint4*>(m + i0);
    const uint4 vq = *reinterpret_cast<const uint4*>(v + i0);
    float4 pa = *reinterpret_cast<const float4*>(p + i0);
    float4 pb = *reinterpret_cast<const float4*>(p + i0 + 4);
    const uint32_t gw[4] = {gq.x, gq.y, gq.z, gq.w}, mw[4] = {mq.x, mq.y, mq.z, mq.w},
                   vw[4] = {vq.x, vq.y, vq.z, vq.w};
    float pv[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
    uint32_t mo[4], vo[4], po[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float mm[2], vv[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const float gg = __uint_as_float((h2 ? gw[q] & 0xFFFF0000u : gw[q] << 16));
        mm[h2] = __uint_as_float((h2 ? mw[q] & 0xFFFF0000u : mw[q] << 16));
        vv[h2] = __uint_as_float((h2 ? vw[q] & 0xFFFF0000u : vw[q] << 16));
        adamw_elem(h, gg, pv[2 * q + h2], mm[h2], vv[h2]);
      }
      mo[q] = pack_bf16x2(mm[0], mm[1]);
      vo[q] = pack_bf16x2(vv[0], vv[1]);
      po[q] = pack_bf16x2(pv[2 * q], pv[2 * q + 1]);
    }
    *reinterpret_cast<uint4*>(m + i0) = uint4{mo[0], mo[1], mo[2], mo[3]};
    *reinterpret_cast<uint4*>(v + i0) = uint4{vo[0], vo[1], vo[2], vo[3]};
    *reinterpret_cast<uint4*>(p_bf16 + i0) = uint4{po[0], po[1], po[2], po[3]};
    *reinterpret_cast<float4*>(p + i0) = float4{pv[0], pv[1], pv[2], pv[3]};
    *reinterpret_cast<float4*>(p + i0 + 4) = float4{pv[4], pv[5], pv[6], pv[7]};
  } else {
    for (int64_t i = i0; i < n; ++i) {
      float pp = p[i], mm = bf16_to_f32(m[i]), vv = bf16_to_f32(v[i]);
      adamw_elem(h, bf16_to_f32(g[i]), pp, mm, vv);
      p[i] = pp;
      m[i] = to_bf16(mm);
      v[i] = to_bf16(vv);
      p_bf16[i] = to_bf16(pp);
    }
  }
}

// ---- E4M3 and absmax double quantization ---------------------------------------------

constexpr int kDqBlock = 256;

// Nearest E4M3FN code of a finite float32, ties to the even code, saturating at
// 448; the code's sign is the input's sign bit.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9 (code 8 is 2^-6 itself)
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  } else {  // keep 3 mantissa bits, round half to even, rebias the exponent 127 -> 7
    const uint32_t b = __float_as_uint(a);
    code = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
  }
  return sign | code;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, mant = c & 7u;
  float v;
  if ((c & 0x7Fu) == 0x7Fu) v = __uint_as_float(0x7FC00000u);
  else if (e == 0) v = static_cast<float>(mant) * 0.001953125f;  // 2^-9
  else v = __uint_as_float(((e + 120u) << 23) | (mant << 20));
  return (c & 0x80u) ? -v : v;
}

// One 256-thread workgroup per block of 256 scales.
__global__ __launch_bounds__(kDqBlock) void absmax_dq_kernel(int64_t n, const float* __restrict__ a,
                                                             uint8_t* __restrict__ q,
                                                             float* __restrict__ scale,
                                                             float* __restrict__ offset) {
  __shared__ float red[2][kDqBlock / 64];
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * kDqBlock;
  const int64_t i = b0 + threadIdx.x;
  const bool ok = i < n;
  const float x = ok ? a[i] : a[b0];  // past a ragged end: a neutral value for min / max
  float lo = x, hi = x;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o));
    hi = fmaxf(hi, __shfl_xor(hi, o));
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wave] = lo;
    red[1][wave] = hi;
  }
  __syncthreads();
  lo = fminf(fminf(red[0][0], red[0][1]), fminf(red[0][2], red[0][3]));
  hi = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  const float off = __fadd_rn(__fmul_rn(lo, 0.5f), __fmul_rn(hi, 0.5f));
  const float d = fmaxf(__fsub_rn(hi, off), __fsub_rn(off, lo));
  const float sc = __fdiv_rn(d, 448.0f);
  if (threadIdx.x == 0) {
    scale[blockIdx.x] = sc;
    offset[blockIdx.x] = off;
  }
  if (ok) q[i] = static_cast<uint8_t>(sc > 0.0f ? e4m3_encode(__fdiv_rn(__fsub_rn(x, off), sc)) : 0u);
}

__global__ __launch_bounds__(256) void absmax_undq_kernel(int64_t n, const uint8_t* __restrict__ q,
                                                          const float* __restrict__ scale,
                                                          const float* __restrict__ offset,
                                                          float* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t b = i / kDqBlock;
  float prod = e4m3_value(q[i]) * scale[b];
  asm volatile("" : "+v"(prod));  // two roundings: keep the multiply and add from fusing
  out[i] = prod + offset[b];
}

}  // namespace

hipError_t launch_adamw(int64_t n, float* p, uint16_t* p_bf16, const uint16_t* g, uint16_t* m,
                        uint16_t* v, int step, float lr, float beta1, float beta2, float eps,
                        float weight_decay, hipStream_t stream) {
  AdamWArgs h;
  h.beta1 = beta1;
  h.one_m_beta1 = static_cast<float>(1.0 - static_cast<double>(beta1));
  h.beta2 = beta2;
  h.one_m_beta2 = static_cast<float>(1.0 - static_cast<double>(beta2));
  h.eps = eps;
  h.decay = static_cast<float>(1.0 - static_cast<double>(lr) * weight_decay);
  const double bc1 = 1.0 - std::pow(static_cast<double>(beta1), step);
  const double bc2 = 1.0 - std::pow(static_cast<double>(beta2), step);
  h.step_size = static_cast<float>(lr / bc1);
  h.inv_sqrt_bc2 = static_cast<float>(1.0 / std::sqrt(bc2));
  const int64_t threads = (n + 7) / 8;
  const int64_t blocks = (threads + kAdamThreads - 1) / kAdamThreads;
  adamw_kernel<<<static_cast<unsigned>(blocks), kAdamThreads, 0, stream>>>(n, p, p_bf16, g, m, v, h);
  return hipGetLastError();
}

hipError_t launch_absmax_dq(int64_t n, const float* absmax, uint8_t* q, float* scale, float* offset,
                            hipStream_t stream) {
  const int64_t blocks = (n + kDqBlock - 1) / kDqBlock;
  absmax_dq_kernel<<<static_cast<unsigned>(blocks), kDqBlock, 0, stream>>>(n, absmax, q, scale, offset);
  return hipGetLastError();
}

hipError_t launch_absmax_undq(int64_t n, const uint8_t* q, const float* scale, const float* offset,
                              float* out, hipStream_t stream) {
  const int64_t blocks = (n + 255) / 256;
  absmax_undq_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(n, q, scale, offset, out);
  return hipGetLastError();
}

}  // namespace lnf4
