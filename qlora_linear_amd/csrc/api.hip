// C ABI of the fused NF4-LoRA linear (declared in include/lora_nf4.h).
//
// Every entry point validates its arguments on the host before touching HIP, so
// argument errors are reported without a GPU and nothing is enqueued on error.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "launch.h"
#include "lora_nf4.h"

namespace lnf4 {
namespace {
std::atomic<bool> g_weight_staging{false};
}  // namespace
bool weight_staging() { return g_weight_staging.load(std::memory_order_relaxed); }
}  // namespace lnf4

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  const void* p;
  size_t bytes;
};

bool overlap(const Span& a, const Span& b) {
  if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Every output span must be disjoint from every input span and from the other outputs.
bool any_alias(const Span* outs, int n_out, const Span* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

// Shared shape rules of the forward and backward (T = 0 is an empty batch).
int check_linear_shape(int64_t T, int64_t K, int64_t N, int32_t r, float alpha) {
  if (T < 0 || K < 1 || N < 1) return LN_EINVAL;
  if (!std::isfinite(alpha)) return LN_EINVAL;
  if (r < 1 || r > LN_MAX_RANK) return LN_ERANK;
  if (K % 64 != 0) return LN_ESHAPE;
  if (T > kMaxDim || K > kMaxDim || N > kMaxDim) return LN_ESHAPE;
  return LN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? LN_OK : LN_EHIP; }

}  // namespace

extern "C" {

const char* lora_nf4_status_string(int status) {
  switch (status) {
    case LN_OK: return "ok";
    case LN_EINVAL: return "invalid argument (null pointer, negative T or other size < 1, non-finite alpha or unknown dtype)";
    case LN_ESHAPE: return "unsupported shape (d_in/cols must be a multiple of 64, sizes below 2^31)";
    case LN_EALIGN: return "data pointer not 16-byte aligned (workspace: 256-byte)";
    case LN_ERANK: return "LoRA rank r outside [1, LN_MAX_RANK]";
    case LN_EWORKSPACE: return "workspace missing or smaller than the entry point's *_workspace_bytes()";
    case LN_EALIAS: return "an output overlaps an input or another output";
    case LN_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int nf4_quantize(const void* w, int w_dtype, int64_t rows, int64_t cols, uint8_t* codes,
                 float* absmax, void* stream) {
  if (w == nullptr || codes == nullptr || absmax == nullptr) return LN_EINVAL;
  if (w_dtype != LN_F32 && w_dtype != LN_BF16) return LN_EINVAL;
  if (rows < 1 || cols < 1) return LN_EINVAL;
  if (cols % 64 != 0 || rows > kMaxDim || cols > kMaxDim || rows * cols > (int64_t(1) << 38))
    return LN_ESHAPE;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(absmax)) return LN_EALIGN;
  const size_t n = static_cast<size_t>(rows * cols);
  const Span outs[2] = {{codes, n / 2}, {absmax, n / 64 * 4}};
  const Span ins[1] = {{w, n * (w_dtype == LN_BF16 ? 2 : 4)}};
  if (any_alias(outs, 2, ins, 1)) return LN_EALIAS;
  return hip_status(lnf4::launch_nf4_quantize(w, w_dtype == LN_BF16, rows, cols, codes, absmax,
                                              static_cast<hipStream_t>(stream)));
}

int nf4_dequantize(const uint8_t* codes, const float* absmax, int64_t rows, int64_t cols,
                   int out_dtype, void* out, void* stream) {
  if (codes == nullptr || absmax == nullptr || out == nullptr) return LN_EINVAL;
  if (out_dtype != LN_F32 && out_dtype != LN_BF16) return LN_EINVAL;
  if (rows < 1 || cols < 1) return LN_EINVAL;
  if (cols % 64 != 0 || rows > kMaxDim || cols > kMaxDim || rows * cols > (int64_t(1) << 38))
    return LN_ESHAPE;
  if (!aligned16(codes) || !aligned16(absmax) || !aligned16(out)) return LN_EALIGN;
  const size_t n = static_cast<size_t>(rows * cols);
  const Span outs[1] = {{out, n * (out_dtype == LN_BF16 ? 2 : 4)}};
  const Span ins[2] = {{codes, n / 2}, {absmax, n / 64 * 4}};
  if (any_alias(outs, 1, ins, 2)) return LN_EALIAS;
  return hip_status(lnf4::launch_nf4_dequantize(codes, absmax, rows, cols, out_dtype == LN_BF16, out,
                                                static_cast<hipStream_t>(stream)));
}

size_t lora_nf4_fwd_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int32_t r) {
  if (T == 0 || check_linear_shape(T, d_in, d_out, r, 1.0f) != LN_OK) return 0;
  return lnf4::fwd_workspace_bytes(T, d_in, d_out, r);
}

int lora_nf4_fwd(int64_t T, int64_t d_in, int64_t d_out, int32_t r, float lora_alpha,
                 const uint16_t* x, const uint8_t* w_codes, const float* w_absmax,
                 const uint16_t* A, const uint16_t* B, uint16_t* y, uint16_t* u_save,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (w_codes == nullptr || w_absmax == nullptr || A == nullptr || B == nullptr) return LN_EINVAL;
  if (T != 0 && (x == nullptr || y == nullptr)) return LN_EINVAL;
  int st = check_linear_shape(T, d_in, d_out, r, lora_alpha);
  if (st != LN_OK) return st;
  if (T == 0) return LN_OK;  // empty batch: nothing to compute
  if (!aligned16(x) || !aligned16(w_codes) || !aligned16(w_absmax) || !aligned16(A) ||
      !aligned16(B) || !aligned16(y) || (u_save != nullptr && !aligned16(u_save)))
    return LN_EALIGN;
  const size_t need = lnf4::fwd_workspace_bytes(T, d_in, d_out, r);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LN_EWORKSPACE;
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LN_EALIGN;
  const size_t t = T, k = d_in, n = d_out, rr = r;
  const Span outs[3] = {{y, t * n * 2}, {u_save, t * rr * 2}, {need > 0 ? workspace : nullptr, need}};
  const Span ins[5] = {{x, t * k * 2}, {w_codes, n * k / 2}, {w_absmax, n * k / 64 * 4},
                       {A, k * rr * 2}, {B, rr * n * 2}};
  if (any_alias(outs, 3, ins, 5)) return LN_EALIAS;
  const float s = lora_alpha / static_cast<float>(r);
  return hip_status(lnf4::launch_lora_fwd(static_cast<int>(T), static_cast<int>(d_in),
                                          static_cast<int>(d_out), r, s, x, w_codes, w_absmax, A, B,
                                          y, u_save, workspace, static_cast<hipStream_t>(stream)));
}

size_t lora_nf4_fwd_multi_workspace_bytes(int64_t T, int64_t d_in, int32_t n_proj, const int64_t* d_out,
                                          int32_t r) {
  if (T == 0 || n_proj < 1 || n_proj > LN_MAX_PROJ || d_out == nullptr) return 0;
  int N[LN_MAX_PROJ];
  for (int g = 0; g < n_proj; ++g) {
    if (check_linear_shape(T, d_in, d_out[g], r, 1.0f) != LN_OK) return 0;
    N[g] = static_cast<int>(d_out[g]);
  }
  return lnf4::fwd_multi_workspace_bytes(T, d_in, n_proj, N, r);
}

int lora_nf4_fwd_multi(int64_t T, int64_t d_in, int32_t n_proj, const int64_t* d_out, int32_t r,
                       float lora_alpha, const uint16_t* x, const uint8_t* const* w_codes,
                       const float* const* w_absmax, const uint16_t* const* A,
                       const uint16_t* const* B, uint16_t* const* y, uint16_t* const* u_save,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (n_proj < 1 || n_proj > LN_MAX_PROJ) return LN_EINVAL;
  if ((T != 0 && x == nullptr) || d_out == nullptr || w_codes == nullptr || w_absmax == nullptr ||
      A == nullptr || B == nullptr || y == nullptr)
    return LN_EINVAL;
  if (!aligned16(x)) return LN_EALIGN;
  const size_t t = T, k = d_in, rr = r;
  Span outs[2 * LN_MAX_PROJ + 1];
  Span ins[1 + 4 * LN_MAX_PROJ];
  int n_out = 0, n_in = 0;
  int N[LN_MAX_PROJ];
  ins[n_in++] = {x, t * k * 2};
  for (int g = 0; g < n_proj; ++g) {
    if (w_codes[g] == nullptr || w_absmax[g] == nullptr || A[g] == nullptr || B[g] == nullptr ||
        (T != 0 && y[g] == nullptr))
      return LN_EINVAL;
    const int st = check_linear_shape(T, d_in, d_out[g], r, lora_alpha);
    if (st != LN_OK) return st;
    uint16_t* u = u_save == nullptr ? nullptr : u_save[g];
    if (!aligned16(w_codes[g]) || !aligned16(w_absmax[g]) || !aligned16(A[g]) || !aligned16(B[g]) ||
        !aligned16(y[g]) || (u != nullptr && !aligned16(u)))
      return LN_EALIGN;
    const size_t n = d_out[g];
    N[g] = static_cast<int>(d_out[g]);
    outs[n_out++] = {y[g], t * n * 2};
    outs[n_out++] = {u, t * rr * 2};
    ins[n_in++] = {w_codes[g], n * k / 2};
    ins[n_in++] = {w_absmax[g], n * k / 64 * 4};
    ins[n_in++] = {A[g], k * rr * 2};
    ins[n_in++] = {B[g], rr * n * 2};
  }
  const size_t need = T == 0 ? 0 : lnf4::fwd_multi_workspace_bytes(T, d_in, n_proj, N, r);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LN_EWORKSPACE;
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LN_EALIGN;
  if (need > 0) outs[n_out++] = {workspace, need};
  if (any_alias(outs, n_out, ins, n_in)) return LN_EALIAS;
  if (T == 0) return LN_OK;  // empty batch
  const float s = lora_alpha / static_cast<float>(r);
  return hip_status(lnf4::launch_lora_fwd_multi(static_cast<int>(T), static_cast<int>(d_in), n_proj, N,
                                                r, s, x, w_codes, w_absmax, A, B, y, u_save, workspace,
                                                static_cast<hipStream_t>(stream)));
}

int lora_nf4_merge(int64_t d_in, int64_t d_out, int32_t r, float lora_alpha, const uint8_t* w_codes,
                   const float* w_absmax, const uint16_t* A, const uint16_t* B, int out_dtype,
                   void* out, void* stream) {
  if (w_codes == nullptr || w_absmax == nullptr || A == nullptr || B == nullptr || out == nullptr)
    return LN_EINVAL;
  if (out_dtype != LN_F32 && out_dtype != LN_BF16) return LN_EINVAL;
  if (d_in < 1 || d_out < 1 || !std::isfinite(lora_alpha)) return LN_EINVAL;
  if (r < 1 || r > LN_MAX_RANK) return LN_ERANK;
  if (d_in % 64 != 0 || d_in > kMaxDim || d_out > kMaxDim || d_in * d_out > (int64_t(1) << 38))
    return LN_ESHAPE;
  if (!aligned16(w_codes) || !aligned16(w_absmax) || !aligned16(A) || !aligned16(B) || !aligned16(out))
    return LN_EALIGN;
  const size_t k = d_in, n = d_out, rr = r;
  const Span outs[1] = {{out, n * k * (out_dtype == LN_BF16 ? 2 : 4)}};
  const Span ins[4] = {{w_codes, n * k / 2}, {w_absmax, n * k / 64 * 4}, {A, k * rr * 2}, {B, rr * n * 2}};
  if (any_alias(outs, 1, ins, 4)) return LN_EALIAS;
  const float s = lora_alpha / static_cast<float>(r);
  return hip_status(lnf4::launch_lora_merge(static_cast<int>(d_in), static_cast<int>(d_out), r, s, w_codes,
                                            w_absmax, A, B, out_dtype == LN_BF16, out,
                                            static_cast<hipStream_t>(stream)));
}

size_t lora_nf4_bwd_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int32_t r) {
  if (T == 0 || check_linear_shape(T, d_in, d_out, r, 1.0f) != LN_OK) return 0;
  return lnf4::plan_bwd(T, d_in, d_out, r).bytes;
}

}  // extern "C"

namespace {

// Argument checks of lora_nf4_bwd that precede the workspace: LN_OK with *empty set
// when T = 0 (after zeroing dA and dB on the stream), LN_OK otherwise, or the error.
int check_bwd(int64_t T, int64_t d_in, int64_t d_out, int32_t r, float lora_alpha, const uint16_t* x,
              const uint16_t* dy, const uint8_t* w_codes, const float* w_absmax, const uint16_t* A,
              const uint16_t* B, const uint16_t* u_saved, uint16_t* dx, uint16_t* dA, uint16_t* dB,
              void* stream, bool* empty) {
  *empty = false;
  if (w_codes == nullptr || w_absmax == nullptr || A == nullptr || B == nullptr || dA == nullptr ||
      dB == nullptr)
    return LN_EINVAL;
  if (T != 0 && (x == nullptr || dy == nullptr)) return LN_EINVAL;
  int st = check_linear_shape(T, d_in, d_out, r, lora_alpha);
  if (st != LN_OK) return st;
  if (T == 0) {  // empty batch: the gradients of A and B are empty sums
    if (!aligned16(dA) || !aligned16(dB)) return LN_EALIGN;
    const Span outs[2] = {{dA, static_cast<size_t>(d_in) * r * 2}, {dB, static_cast<size_t>(r) * d_out * 2}};
    const Span ins[4] = {{w_codes, static_cast<size_t>(d_out) * d_in / 2},
                         {w_absmax, static_cast<size_t>(d_out) * d_in / 64 * 4},
                         {A, static_cast<size_t>(d_in) * r * 2}, {B, static_cast<size_t>(r) * d_out * 2}};
    if (any_alias(outs, 2, ins, 4)) return LN_EALIAS;
    hipError_t e = lnf4::launch_zero_u16(dA, static_cast<int64_t>(d_in) * r, static_cast<hipStream_t>(stream));
    if (e == hipSuccess)
      e = lnf4::launch_zero_u16(dB, static_cast<int64_t>(r) * d_out, static_cast<hipStream_t>(stream));
    *empty = true;
    return hip_status(e);
  }
  if (!aligned16(x) || !aligned16(dy) || !aligned16(w_codes) || !aligned16(w_absmax) ||
      !aligned16(A) || !aligned16(B) || !aligned16(dA) || !aligned16(dB) ||
      (u_saved != nullptr && !aligned16(u_saved)) || (dx != nullptr && !aligned16(dx)))
    return LN_EALIGN;
  return LN_OK;
}

// Alias checks of the backward's outputs (the workspace among them) against its inputs.
bool bwd_aliases(int64_t T, int64_t d_in, int64_t d_out, int32_t r, const uint16_t* x, const uint16_t* dy,
                 const uint8_t* w_codes, const float* w_absmax, const uint16_t* A, const uint16_t* B,
                 const uint16_t* u_saved, uint16_t* dx, uint16_t* dA, uint16_t* dB, const void* workspace,
                 size_t ws_bytes) {
  const size_t t = T, k = d_in, n = d_out, rr = r;
  const Span outs[4] = {{dx, t * k * 2}, {dA, k * rr * 2}, {dB, rr * n * 2}, {workspace, ws_bytes}};
  const Span ins[7] = {{x, t * k * 2},        {dy, t * n * 2},   {w_codes, n * k / 2},
                       {w_absmax, n * k / 64 * 4}, {A, k * rr * 2}, {B, rr * n * 2},
                       {u_saved, t * rr * 2}};
  return any_alias(outs, 4, ins, 7);
}

// The no-allocation backward's scratch: one backward workspace in device memory the
// library owns. A file-scope device array, so each GPU the library runs on holds
// its own copy (64 MiB) until the process ends. Host code must not pass the array's
// name to a kernel (on the host it only stands in for the symbol): its device
// address is looked up once per device, with that device current, and kept.
constexpr size_t kScratchBytes = LN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int lora_nf4_bwd(int64_t T, int64_t d_in, int64_t d_out, int32_t r, float lora_alpha,
                 const uint16_t* x, const uint16_t* dy, const uint8_t* w_codes,
                 const float* w_absmax, const uint16_t* A, const uint16_t* B,
                 const uint16_t* u_saved, uint16_t* dx, uint16_t* dA, uint16_t* dB,
                 void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  const int st = check_bwd(T, d_in, d_out, r, lora_alpha, x, dy, w_codes, w_absmax, A, B, u_saved, dx, dA, dB,
                           stream, &empty);
  if (st != LN_OK || empty) return st;
  const lnf4::BwdPlan plan = lnf4::plan_bwd(T, d_in, d_out, r);
  if (workspace == nullptr || workspace_bytes < plan.bytes) return LN_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LN_EALIGN;
  if (bwd_aliases(T, d_in, d_out, r, x, dy, w_codes, w_absmax, A, B, u_saved, dx, dA, dB, workspace, plan.bytes))
    return LN_EALIAS;
  const float s = lora_alpha / static_cast<float>(r);
  return hip_status(lnf4::launch_lora_bwd(static_cast<int>(T), static_cast<int>(d_in),
                                          static_cast<int>(d_out), r, s, x, dy, w_codes, w_absmax,
                                          A, B, u_saved, dx, dA, dB, workspace, plan,
                                          static_cast<hipStream_t>(stream)));
}

size_t lora_nf4_grad_ab_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int32_t r) {
  if (T == 0 || check_linear_shape(T, d_in, d_out, r, 1.0f) != LN_OK) return 0;
  return lnf4::plan_grad_ab(T, d_in, d_out, r).bytes;
}

int lora_nf4_grad_ab(int64_t T, int64_t d_in, int64_t d_out, int32_t r, float lora_alpha, const uint16_t* x,
                     const uint16_t* g, const uint16_t* dy, const uint16_t* u, uint16_t* dA, uint16_t* dB,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (dA == nullptr || dB == nullptr) return LN_EINVAL;
  if (T != 0 && (x == nullptr || g == nullptr || dy == nullptr || u == nullptr)) return LN_EINVAL;
  const int st = check_linear_shape(T, d_in, d_out, r, lora_alpha);
  if (st != LN_OK) return st;
  if (!aligned16(dA) || !aligned16(dB)) return LN_EALIGN;
  const size_t t = T, k = d_in, n = d_out, rr = r;
  if (T == 0) {  // empty sums
    const Span outs[2] = {{dA, k * rr * 2}, {dB, rr * n * 2}};
    if (any_alias(outs, 2, nullptr, 0)) return LN_EALIAS;
    hipError_t e = lnf4::launch_zero_u16(dA, static_cast<int64_t>(k * rr), static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = lnf4::launch_zero_u16(dB, static_cast<int64_t>(rr * n), static_cast<hipStream_t>(stream));
    return hip_status(e);
  }
  if (!aligned16(x) || !aligned16(g) || !aligned16(dy) || !aligned16(u)) return LN_EALIGN;
  const lnf4::GradPlan plan = lnf4::plan_grad_ab(T, d_in, d_out, r);
  if (workspace == nullptr || workspace_bytes < plan.bytes) return LN_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LN_EALIGN;
  const Span outs[3] = {{dA, k * rr * 2}, {dB, rr * n * 2}, {workspace, plan.bytes}};
  const Span ins[4] = {{x, t * k * 2}, {g, t * rr * 2}, {dy, t * n * 2}, {u, t * rr * 2}};
  if (any_alias(outs, 3, ins, 4)) return LN_EALIAS;
  const float s = lora_alpha / static_cast<float>(r);
  return hip_status(lnf4::launch_grad_ab(static_cast<int>(T), static_cast<int>(d_in), static_cast<int>(d_out), r,
                                         s, x, g, dy, u, dA, dB, workspace, plan,
                                         static_cast<hipStream_t>(stream)));
}

int lora_nf4_bwd_noalloc(int64_t T, int64_t d_in, int64_t d_out, int32_t r, float lora_alpha,
                         const uint16_t* x, const uint16_t* dy, const uint8_t* w_codes,
                         const float* w_absmax, const uint16_t* A, const uint16_t* B,
                         const uint16_t* u_saved, uint16_t* dx, uint16_t* dA, uint16_t* dB, void* stream) {
  bool empty = false;
  const int st = check_bwd(T, d_in, d_out, r, lora_alpha, x, dy, w_codes, w_absmax, A, B, u_saved, dx, dA, dB,
                           stream, &empty);
  if (st != LN_OK || empty) return st;
  // the same plan as lora_nf4_bwd where its workspace fits the scratch, else the
  // plan without the dequantized weight (the same results, in-loop dequantization)
  lnf4::BwdPlan plan = lnf4::plan_bwd(T, d_in, d_out, r);
  if (plan.bytes > kScratchBytes) plan = lnf4::plan_bwd(T, d_in, d_out, r, false);
  if (plan.bytes > kScratchBytes) return LN_EWORKSPACE;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return LN_EHIP;
  if (bwd_aliases(T, d_in, d_out, r, x, dy, w_codes, w_absmax, A, B, u_saved, dx, dA, dB, ws, plan.bytes))
    return LN_EALIAS;
  const float s = lora_alpha / static_cast<float>(r);
  return hip_status(lnf4::launch_lora_bwd(static_cast<int>(T), static_cast<int>(d_in),
                                          static_cast<int>(d_out), r, s, x, dy, w_codes, w_absmax,
                                          A, B, u_saved, dx, dA, dB, ws, plan, static_cast<hipStream_t>(stream)));
}

size_t lora_nf4_bwd_multi_workspace_bytes(int64_t T, int64_t d_in, int32_t n_proj, const int64_t* d_out,
                                          int32_t r) {
  if (T == 0 || n_proj < 1 || n_proj > LN_MAX_PROJ || d_out == nullptr) return 0;
  int N[LN_MAX_PROJ];
  for (int g = 0; g < n_proj; ++g) {
    if (check_linear_shape(T, d_in, d_out[g], r, 1.0f) != LN_OK) return 0;
    N[g] = static_cast<int>(d_out[g]);
  }
  return lnf4::plan_bwd_multi(T, d_in, n_proj, N, r).bytes;
}

int lora_nf4_bwd_multi(int64_t T, int64_t d_in, int32_t n_proj, const int64_t* d_out, int32_t r,
                       float lora_alpha, const uint16_t* x, const uint16_t* const* dy,
                       const uint8_t* const* w_codes, const float* const* w_absmax,
                       const uint16_t* const* A, const uint16_t* const* B,
                       const uint16_t* const* u_saved, uint16_t* dx, uint16_t* const* dA,
                       uint16_t* const* dB, void* workspace, size_t workspace_bytes, void* stream) {
  if (n_proj < 1 || n_proj > LN_MAX_PROJ) return LN_EINVAL;
  if (d_out == nullptr || dy == nullptr || w_codes == nullptr || w_absmax == nullptr || A == nullptr ||
      B == nullptr || dA == nullptr || dB == nullptr)
    return LN_EINVAL;
  if (T != 0 && x == nullptr) return LN_EINVAL;
  const size_t t = T, k = d_in, rr = r;
  Span outs[2 + 2 * LN_MAX_PROJ];
  Span ins[1 + 6 * LN_MAX_PROJ];
  int n_out = 0, n_in = 0;
  int N[LN_MAX_PROJ];
  ins[n_in++] = {x, t * k * 2};
  outs[n_out++] = {dx, t * k * 2};
  for (int g = 0; g < n_proj; ++g) {
    if (w_codes[g] == nullptr || w_absmax[g] == nullptr || A[g] == nullptr || B[g] == nullptr ||
        dA[g] == nullptr || dB[g] == nullptr || (T != 0 && dy[g] == nullptr))
      return LN_EINVAL;
    const int st = check_linear_shape(T, d_in, d_out[g], r, lora_alpha);
    if (st != LN_OK) return st;
    const uint16_t* u = u_saved == nullptr ? nullptr : u_saved[g];
    if (!aligned16(w_codes[g]) || !aligned16(w_absmax[g]) || !aligned16(A[g]) || !aligned16(B[g]) ||
        !aligned16(dA[g]) || !aligned16(dB[g]) || !aligned16(dy[g]) || (u != nullptr && !aligned16(u)))
      return LN_EALIGN;
    const size_t n = d_out[g];
    N[g] = static_cast<int>(d_out[g]);
    outs[n_out++] = {dA[g], k * rr * 2};
    outs[n_out++] = {dB[g], rr * n * 2};
    ins[n_in++] = {dy[g], t * n * 2};
    ins[n_in++] = {w_codes[g], n * k / 2};
    ins[n_in++] = {w_absmax[g], n * k / 64 * 4};
    ins[n_in++] = {A[g], k * rr * 2};
    ins[n_in++] = {B[g], rr * n * 2};
    ins[n_in++] = {u, t * rr * 2};
  }
  if (!aligned16(x) || (dx != nullptr && !aligned16(dx))) return LN_EALIGN;
  if (T == 0) {  // empty batch: every dA and dB is an empty sum
    if (any_alias(outs, n_out, ins, n_in)) return LN_EALIAS;
    hipError_t e = hipSuccess;
    for (int g = 0; g < n_proj && e == hipSuccess; ++g) {
      e = lnf4::launch_zero_u16(dA[g], static_cast<int64_t>(d_in) * r, static_cast<hipStream_t>(stream));
      if (e == hipSuccess)
        e = lnf4::launch_zero_u16(dB[g], static_cast<int64_t>(r) * d_out[g], static_cast<hipStream_t>(stream));
    }
    return hip_status(e);
  }
  const lnf4::BwdMultiPlan plan = lnf4::plan_bwd_multi(T, d_in, n_proj, N, r);
  if (workspace == nullptr || workspace_bytes < plan.bytes) return LN_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LN_EALIGN;
  outs[n_out++] = {workspace, plan.bytes};
  if (any_alias(outs, n_out, ins, n_in)) return LN_EALIAS;
  const float s = lora_alpha / static_cast<float>(r);
  return hip_status(lnf4::launch_lora_bwd_multi(static_cast<int>(T), static_cast<int>(d_in), n_proj, N, r, s,
                                                x, dy, w_codes, w_absmax, A, B, u_saved, dx, dA, dB,
                                                workspace, plan, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {
bool adamw_hparams_ok(int32_t step, float lr, float beta1, float beta2, float eps, float weight_decay) {
  return step >= 1 && std::isfinite(lr) && std::isfinite(weight_decay) && std::isfinite(eps) && eps > 0.0f &&
         beta1 >= 0.0f && beta1 < 1.0f && beta2 >= 0.0f && beta2 < 1.0f;
}
}  // namespace

extern "C" {

int lora_adamw_step(int64_t n, float* p, uint16_t* p_bf16, const uint16_t* grad, float* m, float* v,
                    int32_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                    void* stream) {
  if (n < 0 || !adamw_hparams_ok(step, lr, beta1, beta2, eps, weight_decay)) return LN_EINVAL;
  if (n == 0) return LN_OK;
  if (p == nullptr || p_bf16 == nullptr || grad == nullptr || m == nullptr || v == nullptr)
    return LN_EINVAL;
  if (n > (int64_t(1) << 40)) return LN_ESHAPE;
  if (!aligned16(p) || !aligned16(p_bf16) || !aligned16(grad) || !aligned16(m) || !aligned16(v))
    return LN_EALIGN;
  const size_t nn = static_cast<size_t>(n);
  const Span outs[4] = {{p, nn * 4}, {p_bf16, nn * 2}, {m, nn * 4}, {v, nn * 4}};
  const Span ins[1] = {{grad, nn * 2}};
  if (any_alias(outs, 4, ins, 1)) return LN_EALIAS;
  return hip_status(lnf4::launch_adamw(n, p, p_bf16, grad, m, v,
                                       lnf4::adamw_args(step, lr, beta1, beta2, eps, weight_decay),
                                       static_cast<hipStream_t>(stream)));
}

int lora_adamw8_step(int64_t n, float* p, uint16_t* p_bf16, const uint16_t* grad, uint8_t* m_codes,
                     float* m_scales, uint8_t* v_codes, float* v_scales, int32_t step, float lr, float beta1,
                     float beta2, float eps, float weight_decay, void* stream) {
  if (n < 0 || !adamw_hparams_ok(step, lr, beta1, beta2, eps, weight_decay)) return LN_EINVAL;
  if (n == 0) return LN_OK;
  if (p == nullptr || p_bf16 == nullptr || grad == nullptr || m_codes == nullptr || m_scales == nullptr ||
      v_codes == nullptr || v_scales == nullptr)
    return LN_EINVAL;
  if (n > (int64_t(1) << 40)) return LN_ESHAPE;
  if (!aligned16(p) || !aligned16(p_bf16) || !aligned16(grad) || !aligned16(m_codes) || !aligned16(m_scales) ||
      !aligned16(v_codes) || !aligned16(v_scales))
    return LN_EALIGN;
  const size_t nn = static_cast<size_t>(n), nb = (nn + 255) / 256;
  const Span outs[6] = {{p, nn * 4}, {p_bf16, nn * 2}, {m_codes, nn}, {m_scales, nb * 4}, {v_codes, nn},
                        {v_scales, nb * 4}};
  const Span ins[1] = {{grad, nn * 2}};
  if (any_alias(outs, 6, ins, 1)) return LN_EALIAS;
  return hip_status(lnf4::launch_adamw8(n, p, p_bf16, grad, m_codes, m_scales, v_codes, v_scales,
                                        lnf4::adamw_args(step, lr, beta1, beta2, eps, weight_decay),
                                        static_cast<hipStream_t>(stream)));
}

int lora_nf4_bwd_adamw(int64_t T, int64_t d_in, int64_t d_out, int32_t r, float lora_alpha,
                       const uint16_t* x, const uint16_t* dy, const uint8_t* w_codes, const float* w_absmax,
                       uint16_t* A, uint16_t* B, const uint16_t* u_saved, uint16_t* dx, float* a_master,
                       float* a_m, float* a_v, float* b_master, float* b_m, float* b_v, int32_t step, float lr,
                       float beta1, float beta2, float eps, float weight_decay, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (x == nullptr || dy == nullptr || w_codes == nullptr || w_absmax == nullptr || A == nullptr ||
      B == nullptr || a_master == nullptr || a_m == nullptr || a_v == nullptr || b_master == nullptr ||
      b_m == nullptr || b_v == nullptr)
    return LN_EINVAL;
  if (T < 1 || !adamw_hparams_ok(step, lr, beta1, beta2, eps, weight_decay)) return LN_EINVAL;
  int st = check_linear_shape(T, d_in, d_out, r, lora_alpha);
  if (st != LN_OK) return st;
  const lnf4::BwdPlan plan = lnf4::plan_bwd(T, d_in, d_out, r);
  if (!lnf4::bwd_adamw_supported(plan)) return r % 8 != 0 || r > 64 ? LN_ERANK : LN_ESHAPE;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(w_codes) || !aligned16(w_absmax) || !aligned16(A) ||
      !aligned16(B) || (u_saved != nullptr && !aligned16(u_saved)) || (dx != nullptr && !aligned16(dx)) ||
      !aligned16(a_master) || !aligned16(a_m) || !aligned16(a_v) || !aligned16(b_master) || !aligned16(b_m) ||
      !aligned16(b_v))
    return LN_EALIGN;
  if (workspace == nullptr || workspace_bytes < plan.bytes) return LN_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LN_EALIGN;
  const size_t t = T, k = d_in, n = d_out, rr = r;
  // A and B are read by the backward and rewritten by the update: each counts as an output
  const Span outs[10] = {{dx, t * k * 2},       {A, k * rr * 2},       {B, rr * n * 2},
                         {a_master, k * rr * 4}, {a_m, k * rr * 4},     {a_v, k * rr * 4},
                         {b_master, rr * n * 4}, {b_m, rr * n * 4},     {b_v, rr * n * 4},
                         {workspace, plan.bytes}};
  const Span ins[5] = {{x, t * k * 2}, {dy, t * n * 2}, {w_codes, n * k / 2}, {w_absmax, n * k / 64 * 4},
                       {u_saved, t * rr * 2}};
  if (any_alias(outs, 10, ins, 5)) return LN_EALIAS;
  lnf4::SkinnyAdamW adam;
  adam.a = lnf4::AdamState{a_master, A, a_m, a_v};
  adam.b = lnf4::AdamState{b_master, B, b_m, b_v};
  adam.h = lnf4::adamw_args(step, lr, beta1, beta2, eps, weight_decay);
  const float s = lora_alpha / static_cast<float>(r);
  return hip_status(lnf4::launch_lora_bwd(static_cast<int>(T), static_cast<int>(d_in), static_cast<int>(d_out),
                                          r, s, x, dy, w_codes, w_absmax, A, B, u_saved, dx, nullptr, nullptr,
                                          workspace, plan, static_cast<hipStream_t>(stream), &adam));
}

int64_t lora_nf4_mfma_probe(int32_t iters, float* sink, void* stream) {
  if (iters < 1 || iters > (1 << 20) || sink == nullptr) return LN_EINVAL;
  if (!aligned16(sink)) return LN_EALIGN;
  const int64_t f = lnf4::launch_mfma_probe(iters, sink, static_cast<hipStream_t>(stream));
  return f < 0 ? static_cast<int64_t>(LN_EINVAL) : f;
}

int lora_nf4_set_weight_staging(int32_t mode) {
  if (mode < -1 || mode > 1) return LN_EINVAL;
  if (mode < 0) return lnf4::weight_staging() ? 1 : 0;
  return lnf4::g_weight_staging.exchange(mode == 1) ? 1 : 0;
}

float lora_nf4_rslora_alpha(float lora_alpha, int32_t r) {
  if (r < 1 || r > LN_MAX_RANK || !std::isfinite(lora_alpha)) return std::nanf("");
  const float rf = static_cast<float>(r);
  const float target = static_cast<float>(static_cast<double>(lora_alpha) / std::sqrt(static_cast<double>(r)));
  // x -> f32(x / r) is monotone: walk from target * r to the first x whose
  // quotient reaches target, then keep whichever neighbour lands nearer.
  float a = target * rf;
  if (!std::isfinite(a)) return std::nanf("");
  for (int it = 0; it < 64 && a / rf > target; ++it) a = std::nextafter(a, -HUGE_VALF);
  for (int it = 0; it < 64 && a / rf < target; ++it) a = std::nextafter(a, HUGE_VALF);
  const float below = std::nextafter(a, -HUGE_VALF);
  return (a / rf - target <= target - below / rf) ? a : below;
}

int nf4_absmax_quantize(const float* absmax, int64_t n, uint8_t* q, float* scale, float* offset,
                        void* stream) {
  if (n < 0) return LN_EINVAL;
  if (n == 0) return LN_OK;
  if (absmax == nullptr || q == nullptr || scale == nullptr || offset == nullptr) return LN_EINVAL;
  if (n > (int64_t(1) << 38)) return LN_ESHAPE;
  if (!aligned16(absmax) || !aligned16(q) || !aligned16(scale) || !aligned16(offset)) return LN_EALIGN;
  const size_t nn = static_cast<size_t>(n), nb = (nn + 255) / 256;
  const Span outs[3] = {{q, nn}, {scale, nb * 4}, {offset, nb * 4}};
  const Span ins[1] = {{absmax, nn * 4}};
  if (any_alias(outs, 3, ins, 1)) return LN_EALIAS;
  return hip_status(lnf4::launch_absmax_dq(n, absmax, q, scale, offset, static_cast<hipStream_t>(stream)));
}

int nf4_absmax_dequantize(const uint8_t* q, const float* scale, const float* offset, int64_t n,
                          float* absmax, void* stream) {
  if (n < 0) return LN_EINVAL;
  if (n == 0) return LN_OK;
  if (absmax == nullptr || q == nullptr || scale == nullptr || offset == nullptr) return LN_EINVAL;
  if (n > (int64_t(1) << 38)) return LN_ESHAPE;
  if (!aligned16(absmax) || !aligned16(q) || !aligned16(scale) || !aligned16(offset)) return LN_EALIGN;
  const size_t nn = static_cast<size_t>(n), nb = (nn + 255) / 256;
  const Span outs[1] = {{absmax, nn * 4}};
  const Span ins[3] = {{q, nn}, {scale, nb * 4}, {offset, nb * 4}};
  if (any_alias(outs, 1, ins, 3)) return LN_EALIAS;
  return hip_status(lnf4::launch_absmax_undq(n, q, scale, offset, absmax, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
