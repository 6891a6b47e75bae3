// Training-step companions of the fused NF4-LoRA linear (gfx950):
//
//  * adamw_kernel / adamw8_kernel — the optimizer update of a LoRA factor. The
//    pages time the optimizer step as its own phase, a GPU kernel with low-bit
//    state ("Unsloth performance measured: is it really 2x faster?", section 2.2
//    time table; "Reading the Unsloth changelog", section 1: 8-bit AdamW at a
//    quarter of the state memory). Decoupled weight decay (AdamW); float32
//    master weights, bf16 copy for the GEMM kernels; moments in float32, or
//    8-bit: per 256-element block one float32 scale and one E4M3 code per
//    element. One pass reads and writes every array once: bound by HBM. (The
//    backward can also apply the float32-moment update itself, in its rank-r
//    reduction: lora_skinny.hip.)
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

constexpr int kAdamThreads = 256;

// float32 moments. Thread i owns elements 4 i .. 4 i + 3: float4 loads of the
// master copy and both moments, 8-byte loads of the bf16 gradient. The last
// thread of a ragged length runs elementwise.
__global__ __launch_bounds__(kAdamThreads) void adamw_kernel(int64_t n, float* __restrict__ p,
                                                             uint16_t* __restrict__ p_bf16,
                                                             const uint16_t* __restrict__ g,
                                                             float* __restrict__ m, float* __restrict__ v,
                                                             const AdamWArgs h) {
  const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * kAdamThreads + threadIdx.x) * 4;
  if (i0 >= n) return;
  if (i0 + 4 <= n) {
    const uint2 gq = *reinterpret_cast<const uint2*>(g + i0);
    float4 pq = *reinterpret_cast<const float4*>(p + i0);
    float4 mq = *reinterpret_cast<const float4*>(m + i0);
    float4 vq = *reinterpret_cast<const float4*>(v + i0);
    adamw_elem(h, __uint_as_float(gq.x << 16), pq.x, mq.x, vq.x);
    adamw_elem(h, __uint_as_float(gq.x & 0xFFFF0000u), pq.y, mq.y, vq.y);
    adamw_elem(h, __uint_as_float(gq.y << 16), pq.z, mq.z, vq.z);
    adamw_elem(h, __uint_as_float(gq.y & 0xFFFF0000u), pq.w, mq.w, vq.w);
    *reinterpret_cast<float4*>(p + i0) = pq;
    *reinterpret_cast<float4*>(m + i0) = mq;
    *reinterpret_cast<float4*>(v + i0) = vq;
    *reinterpret_cast<uint2*>(p_bf16 + i0) = uint2{pack_bf16x2(pq.x, pq.y), pack_bf16x2(pq.z, pq.w)};
  } else {
    for (int64_t i = i0; i < n; ++i) {
      float pp = p[i], mm = m[i], vv = v[i];
      adamw_elem(h, bf16_to_f32(g[i]), pp, mm, vv);
      p[i] = pp;
      m[i] = mm;
      v[i] = vv;
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

// ---- AdamW with 8-bit blockwise moments ---------------------------------------------
// One 256-thread workgroup per block of 256 state elements: decode both moments
// (f32(e4m3(code) * scale)), the float32 step, then the block's new maxima (exact,
// two-level max over the waves) give the new scales f32(max / 448) and codes
// e4m3(f32(x / scale)) (code 0 when the scale is 0).
__global__ __launch_bounds__(kDqBlock) void adamw8_kernel(int64_t n, float* __restrict__ p,
                                                          uint16_t* __restrict__ p_bf16,
                                                          const uint16_t* __restrict__ g,
                                                          uint8_t* __restrict__ mq, float* __restrict__ ms,
                                                          uint8_t* __restrict__ vq, float* __restrict__ vs,
                                                          const AdamWArgs h) {
  __shared__ float red[2][kDqBlock / 64];
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kDqBlock + threadIdx.x;
  const bool ok = i < n;
  float pp = 0.f, m = 0.f, v = 0.f;
  if (ok) {
    m = __fmul_rn(e4m3_value(mq[i]), ms[blockIdx.x]);
    v = __fmul_rn(e4m3_value(vq[i]), vs[blockIdx.x]);
    pp = p[i];
    adamw_elem(h, bf16_to_f32(g[i]), pp, m, v);
  }
  float am = fabsf(m), av = v;  // zero past a ragged end
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    am = fmaxf(am, __shfl_xor(am, o));
    av = fmaxf(av, __shfl_xor(av, o));
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wave] = am;
    red[1][wave] = av;
  }
  __syncthreads();  // every thread has read its block's old scales
  am = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  av = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  const float nms = __fdiv_rn(am, 448.0f), nvs = __fdiv_rn(av, 448.0f);
  if (ok) {
    mq[i] = static_cast<uint8_t>(nms > 0.0f ? e4m3_encode(__fdiv_rn(m, nms)) : 0u);
    vq[i] = static_cast<uint8_t>(nvs > 0.0f ? e4m3_encode(__fdiv_rn(v, nvs)) : 0u);
    p[i] = pp;
    p_bf16[i] = to_bf16(pp);
  }
  if (threadIdx.x == 0) {
    ms[blockIdx.x] = nms;
    vs[blockIdx.x] = nvs;
  }
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

AdamWArgs adamw_args(int step, float lr, float beta1, float beta2, float eps, float weight_decay) {
  AdamWArgs h;
  h.beta1 = beta1;
  h.one_m_beta1 = static_cast<float>(1.0 - static_cast<double>(beta1));
  h.beta2 = beta2;
  h.one_m_beta2 = static_cast<float>(1.0 - static_cast<double>(beta2));
  h.eps = eps;
  h.decay = static_cast<float>(1.0 - static_cast<double>(lr) * static_cast<double>(weight_decay));
  const double bc1 = 1.0 - std::pow(static_cast<double>(beta1), static_cast<double>(step));
  const double bc2 = 1.0 - std::pow(static_cast<double>(beta2), static_cast<double>(step));
  h.step_size = static_cast<float>(static_cast<double>(lr) / bc1);
  h.inv_sqrt_bc2 = static_cast<float>(1.0 / std::sqrt(bc2));
  return h;
}

hipError_t launch_adamw(int64_t n, float* p, uint16_t* p_bf16, const uint16_t* g, float* m, float* v,
                        const AdamWArgs& h, hipStream_t stream) {
  const int64_t threads = (n + 3) / 4;
  const int64_t blocks = (threads + kAdamThreads - 1) / kAdamThreads;
  adamw_kernel<<<static_cast<unsigned>(blocks), kAdamThreads, 0, stream>>>(n, p, p_bf16, g, m, v, h);
  return hipGetLastError();
}

hipError_t launch_adamw8(int64_t n, float* p, uint16_t* p_bf16, const uint16_t* g, uint8_t* m_codes,
                         float* m_scales, uint8_t* v_codes, float* v_scales, const AdamWArgs& h,
                         hipStream_t stream) {
  const int64_t blocks = (n + kDqBlock - 1) / kDqBlock;
  adamw8_kernel<<<static_cast<unsigned>(blocks), kDqBlock, 0, stream>>>(n, p, p_bf16, g, m_codes, m_scales,
                                                                       v_codes, v_scales, h);
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
