/*
 * lora_nf4.h — C ABI of the fused NF4-LoRA linear for AMD Instinct MI355X (gfx950).
 *
 * The operation is the LoRA linear over a frozen base weight held in 4-bit
 * NormalFloat (NF4) form, as the Unsloth pages describe it:
 *   - "Unsloth acceleration principles: CUDA kernel fusion and memory optimization"
 *     (kernel-fusion section): the base linear, the LoRA down- and up-projections
 *     and the add run as one fused pass; the model is loaded with
 *     load_in_4bit=True and get_peft_model(r, lora_alpha, lora_dropout=0,
 *     bias="none"). Its compact-layout section fixes A in R^{d_in x r} and
 *     B in R^{r x d_out}.
 *   - "Unlocking AI potential: Unsloth's algorithms and implementation"
 *     (core algorithms): a hand-written backward instead of autograd.
 *   - "Reading the Unsloth changelog" (section 1.1): base weights resident in NF4.
 *
 * With T tokens, K = d_in, N = d_out, s = lora_alpha / r and D = deq(Wt), where
 * Wt = W^T is the nn.Linear-oriented [N, K] base weight:
 *     forward : y  = x D^T + s (x A) B
 *     backward: dX = dY D + s (dY B^T) A^T,  dA = x^T (s dY B^T),  dB = s (x A)^T dY
 * There is no dropout, no bias and no base-weight gradient (the base is frozen).
 *
 * NF4 format (the pages name NF4 but do not define it; the QLoRA NormalFloat
 * construction is used): 16 levels q[0..15] (normal quantiles, exact zero at
 * code 7, q[0] = -1, q[15] = 1, stored as float32); blocks of 64 consecutive
 * elements along a row; one float32 absmax per block; code = nearest level to
 * w / absmax, ties to the higher code; an all-zero block has absmax +0 and codes
 * 7; two codes per byte, the even element in the low nibble.
 *
 * Conventions for every entry point:
 *   - Matrices are row-major and dense. bf16 values are passed as uint16_t bit
 *     patterns.
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library
 *     never allocates, frees or synchronizes. Work is enqueued on `stream`
 *     (a hipStream_t; NULL = the default stream) and the call returns at once.
 *   - Arguments are validated on the host before any HIP call; on error nothing
 *     is enqueued and a negative ln_status is returned. Faults inside kernels
 *     cannot be detected without a synchronization and are not reported.
 *   - Data pointers must be 16-byte aligned. Outputs must not overlap inputs.
 *   - Calls are stateless and thread-safe; concurrent calls on different streams
 *     are safe when their outputs do not overlap.
 *   - Floating-point inputs must be finite (not checked: a check needs a sync).
 */
#ifndef LORA_NF4_H
#define LORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LN_OK = 0,
    LN_EINVAL = -1,      /* null pointer, negative T or other size < 1, non-finite
                            alpha, unknown dtype                                    */
    LN_ESHAPE = -2,      /* d_in or cols not a multiple of 64, or a size beyond the
                            2^31 element-index range                                */
    LN_EALIGN = -3,      /* a data pointer is not 16-byte aligned                    */
    LN_ERANK = -4,       /* r < 1 or r > LN_MAX_RANK                                 */
    LN_EWORKSPACE = -5,  /* workspace null or smaller than the entry point's *_workspace_bytes */
    LN_EALIAS = -6,      /* an output overlaps an input or another output            */
    LN_EHIP = -7         /* a HIP launch reported an error                           */
} ln_status;

typedef enum { LN_F32 = 0, LN_BF16 = 1 } ln_dtype;

#define LN_MAX_RANK 256
#define LN_MAX_PROJ 8   /* projections per lora_nf4_fwd_multi / lora_nf4_bwd_multi call */

/*
 * nf4_quantize — blockwise NF4 quantization of w [rows, cols] (float32 or bf16
 * per w_dtype) into codes uint8 [rows, cols/2] and absmax float32
 * [rows, cols/64]. cols % 64 == 0. Codes and absmax are bit-exact with the
 * definition above: the level comparisons are made exactly (float64).
 * The frozen weight is quantized once at load time ("load_in_4bit").
 */
int nf4_quantize(const void* w, int w_dtype, int64_t rows, int64_t cols,
                 uint8_t* codes, float* absmax, void* stream);

/*
 * nf4_dequantize — out [rows, cols] = q[code] * absmax, rounded once to float32
 * (nearest-even); for LN_BF16 output that float32 is rounded to nearest-even
 * bf16. cols % 64 == 0.
 */
int nf4_dequantize(const uint8_t* codes, const float* absmax, int64_t rows, int64_t cols,
                   int out_dtype, void* out, void* stream);

/*
 * lora_nf4_fwd — y = x D^T + s (x A) B, one fused pass.
 *   x        bf16 [T, d_in]
 *   w_codes  uint8 [d_out, d_in/2], w_absmax float32 [d_out, d_in/64] (from nf4_quantize
 *            of the [d_out, d_in] base weight)
 *   A        bf16 [d_in, r],  B bf16 [r, d_out]
 *   y        bf16 [T, d_out]  (output)
 *   u_save   bf16 [T, r] = x A, rounded to bf16 (output; may be NULL). Passing it
 *            to lora_nf4_bwd saves that pass recomputing it.
 *   workspace  device scratch of at least lora_nf4_fwd_workspace_bytes(T, d_in,
 *            d_out, r) bytes, 256-byte aligned, owned by the caller (contents on
 *            entry do not matter, on return unspecified; concurrent calls need
 *            separate workspaces). That size is non-zero where the reduction
 *            over d_in is split across workgroups and fp32 partial sums meet in
 *            the workspace (few tokens: T <= 128 at r % 8 == 0, r <= 64; and
 *            token counts whose output tiles leave most of the GPU idle); from
 *            T = 4096 with d_in % 256 == 0, r % 8 == 0, r <= 64 (256 x 256 tiles
 *            that dequantize into registers), at ranks other than 16, where it
 *            holds A^T and bf16(s x A) of a pass over x ahead of the tiles
 *            (2 r (d_in + T) bytes, each part rounded up to 256; at r = 16 the
 *            tiles form x A themselves); and, with weight staging on
 *            (lora_nf4_set_weight_staging), from T = 1024 (T = 4096 on
 *            256 x 256 tiles), where the weight is dequantized once into it
 *            (bf16 [d_out, d_in]: 2 d_in d_out bytes, the same values the fused
 *            kernels produce). When it is 0 the workspace may be NULL.
 * T >= 0, d_in % 64 == 0, d_out >= 1 (any; a d_out that is not a multiple of 8, and
 * ranks r % 8 != 0 or r > 64, run the generic 128 x 128 kernels: same results,
 * lower speed), 1 <= r <= LN_MAX_RANK. s = lora_alpha / r
 * is formed in float32 on the host. T = 0 is an empty batch: nothing is computed
 * and x, y, u_save and the workspace may be NULL. LN_EWORKSPACE if the workspace
 * is needed and NULL or too small; the workspace must not overlap any operand.
 */
int lora_nf4_fwd(int64_t T, int64_t d_in, int64_t d_out, int32_t r, float lora_alpha,
                 const uint16_t* x, const uint8_t* w_codes, const float* w_absmax,
                 const uint16_t* A, const uint16_t* B, uint16_t* y, uint16_t* u_save,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes lora_nf4_fwd needs (0 if the sizes are invalid, T = 0, or the
   shape takes a path without one). */
size_t lora_nf4_fwd_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int32_t r);

/*
 * lora_nf4_fwd_multi — the forward of n_proj LoRA projections that read the same
 * x, e.g. q/k/v or gate/up (the target modules q_proj, k_proj, v_proj, o_proj of
 * "Unsloth acceleration principles: CUDA kernel fusion and memory optimization",
 * kernel-fusion section; the q/k/v projection products issued as one group on the
 * "Unsloth in three lines of code" page, section 2). For every g < n_proj:
 *     y[g] = x D_g^T + s (x A[g]) B[g],   u_save[g] = bf16(x A[g])
 * exactly as n_proj calls of lora_nf4_fwd would compute them, but in one launch
 * over the column tiles of all projections when they take the tiled path (x is
 * then read once per token tile for all of them; narrow projections such as
 * k/v at d_out = 1024 no longer leave most of the GPU idle).
 *   n_proj               1 .. LN_MAX_PROJ
 *   d_out                HOST array [n_proj]: d_out of each projection (>= 1)
 *   w_codes, w_absmax,
 *   A, B, y              HOST arrays [n_proj] of DEVICE pointers, each laid out as
 *                        for lora_nf4_fwd with that projection's d_out
 *   u_save               NULL, or a HOST array [n_proj] whose entries may be NULL
 *   workspace            as for lora_nf4_fwd, sized by
 *                        lora_nf4_fwd_multi_workspace_bytes: non-zero when the
 *                        projections run one after the other on a path that
 *                        needs one (they reuse it in turn), and for one shared
 *                        launch at large token counts (on register-
 *                        dequantizing tiles at ranks other than 16, A^T and
 *                        bf16(s x A) of all projections: one pass over x when
 *                        n_proj r <= 64, else one per projection; with weight
 *                        staging on, every projection's weight dequantized
 *                        into it, one after another)
 * All projections share T, d_in, r and lora_alpha. The host arrays are read
 * during the call only. Every output (each y[g], each u_save[g], the workspace)
 * must be disjoint from every input and from the other outputs (LN_EALIAS).
 * Errors as for lora_nf4_fwd, plus LN_EINVAL for n_proj out of range or a NULL
 * array.
 */
int lora_nf4_fwd_multi(int64_t T, int64_t d_in, int32_t n_proj, const int64_t* d_out, int32_t r,
                       float lora_alpha, const uint16_t* x, const uint8_t* const* w_codes,
                       const float* const* w_absmax, const uint16_t* const* A,
                       const uint16_t* const* B, uint16_t* const* y, uint16_t* const* u_save,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes lora_nf4_fwd_multi needs (0 if the sizes are invalid, T = 0, or
   no projection needs one). */
size_t lora_nf4_fwd_multi_workspace_bytes(int64_t T, int64_t d_in, int32_t n_proj, const int64_t* d_out,
                                          int32_t r);

/*
 * lora_nf4_bwd — dX, dA, dB of the forward above for upstream gradient dY.
 *   dy       bf16 [T, d_out]
 *   u_saved  bf16 [T, r] from lora_nf4_fwd, or NULL (then recomputed from x and A)
 *   dx       bf16 [T, d_in] (output; may be NULL to skip the input gradient —
 *            the pass over the base weight still runs, since it also forms dY B^T)
 *   dA       bf16 [d_in, r], dB bf16 [r, d_out] (outputs)
 *   workspace  device scratch of at least lora_nf4_bwd_workspace_bytes(T, d_in,
 *            d_out, r) bytes, 256-byte aligned, owned by the caller; its contents
 *            on entry do not matter and on return are unspecified. Two calls that
 *            may run concurrently need separate workspaces. From T = 4096 at
 *            r = 16 with d_in and d_out multiples of 256 (dX on 256 x 256 tiles
 *            that dequantize into registers) it also holds the packed weight
 *            transposed, d_in d_out / 2 + d_in d_out / 16 bytes (codes and
 *            absmax, each part rounded up to 256). With weight staging on
 *            (lora_nf4_set_weight_staging) it instead holds, at large token
 *            counts (from T = 1024, or 4096 where dX runs 256 x 256 tiles), the
 *            bf16 dequantized weight, 2 d_in d_out bytes.
 * Shape rules as for lora_nf4_fwd. With T = 0 (empty batch) dA and dB are set to
 * zero (empty sums), x, dy, u_saved, dx and the workspace may be NULL, and
 * lora_nf4_bwd_workspace_bytes is 0.
 */
int lora_nf4_bwd(int64_t T, int64_t d_in, int64_t d_out, int32_t r, float lora_alpha,
                 const uint16_t* x, const uint16_t* dy,
                 const uint8_t* w_codes, const float* w_absmax,
                 const uint16_t* A, const uint16_t* B, const uint16_t* u_saved,
                 uint16_t* dx, uint16_t* dA, uint16_t* dB,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * lora_nf4_grad_ab — the gradients of the LoRA factors alone, from the
 * intermediates the backward forms ("Unlocking AI potential: Unsloth's algorithms
 * and implementation", core algorithms: the hand-written backward's dA and dB):
 *     dA = x^T G      bf16 [d_in, r]
 *     dB = s U^T dY   bf16 [r, d_out],  s = lora_alpha / r
 * with G = bf16(s dY B^T) and U = bf16(x A) as the caller holds them (the
 * backward's own rank-r step, for callers that keep G and U, and to time that
 * step alone). Float32 sums over the T tokens in split-T partials, reduced in a
 * fixed order (the results do not depend on the run).
 *   x   bf16 [T, d_in]     g  bf16 [T, r]     dy  bf16 [T, d_out]     u  bf16 [T, r]
 *   workspace  at least lora_nf4_grad_ab_workspace_bytes(T, d_in, d_out, r) bytes,
 *            256-byte aligned, caller-owned, contents on entry irrelevant.
 * Shape rules as for lora_nf4_fwd. T = 0: dA and dB are set to zero, the inputs and
 * the workspace may be NULL. dA, dB and the workspace must not overlap the inputs
 * or each other (LN_EALIAS).
 */
size_t lora_nf4_grad_ab_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int32_t r);
int lora_nf4_grad_ab(int64_t T, int64_t d_in, int64_t d_out, int32_t r, float lora_alpha,
                     const uint16_t* x, const uint16_t* g, const uint16_t* dy, const uint16_t* u,
                     uint16_t* dA, uint16_t* dB, void* workspace, size_t workspace_bytes, void* stream);

/*
 * lora_nf4_bwd_multi — the backward of n_proj projections that read the same x
 * (q/k/v or gate/up, as for lora_nf4_fwd_multi): their input gradients add up,
 *     dX = sum_g ( dY[g] D_g + s (dY[g] B[g]^T) A[g]^T )
 *     dA[g] = x^T (s dY[g] B[g]^T),   dB[g] = s (x A[g])^T dY[g]
 * the same sums n_proj calls of lora_nf4_bwd compute, with dX summed. When every
 * d_out is a multiple of 64, r % 8 == 0, n_proj r <= 64 and T > 32, one dX pass
 * runs over the projections' concatenated d_out (no per-projection dX in HBM)
 * and one pass over x yields every dA; otherwise the projections run one after
 * another and dX accumulates (float32 add of bf16 partial results).
 *   n_proj             1 .. LN_MAX_PROJ;  d_out  HOST array [n_proj] (>= 1)
 *   dy, w_codes, w_absmax, A, B, dA, dB
 *                      HOST arrays [n_proj] of DEVICE pointers, laid out as for
 *                      lora_nf4_bwd with that projection's d_out
 *   u_saved            NULL, or a HOST array [n_proj] whose entries may be NULL
 *                      (bf16 x A[g] from lora_nf4_fwd_multi; recomputed if NULL)
 *   dx                 bf16 [T, d_in] (output; may be NULL to skip it)
 *   workspace          at least lora_nf4_bwd_multi_workspace_bytes(...) bytes,
 *                      256-byte aligned, as for lora_nf4_bwd
 * All projections share T, d_in, r and lora_alpha. Every output (dx, each dA[g],
 * dB[g], the workspace) must be disjoint from every input and the other outputs
 * (LN_EALIAS). T = 0 zeroes every dA[g] and dB[g]. Other errors as for
 * lora_nf4_bwd, plus LN_EINVAL for n_proj out of range or a NULL array.
 */
int lora_nf4_bwd_multi(int64_t T, int64_t d_in, int32_t n_proj, const int64_t* d_out, int32_t r,
                       float lora_alpha, const uint16_t* x, const uint16_t* const* dy,
                       const uint8_t* const* w_codes, const float* const* w_absmax,
                       const uint16_t* const* A, const uint16_t* const* B,
                       const uint16_t* const* u_saved, uint16_t* dx, uint16_t* const* dA,
                       uint16_t* const* dB, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes lora_nf4_bwd_multi needs (0 if the sizes are invalid or T = 0). */
size_t lora_nf4_bwd_multi_workspace_bytes(int64_t T, int64_t d_in, int32_t n_proj, const int64_t* d_out,
                                          int32_t r);

/*
 * lora_nf4_merge — the merged base weight for export after training,
 *     W' = D + s (A B)^T,   [d_out, d_in],  s = lora_alpha / r
 * (the adapters folded into the base and saved at 16 bits: "Unsloth in three
 * lines of code", section 4; "Reading the Unsloth changelog", command-line part
 * of section 2). Element (n, k) is the float32 sum of q[code] * absmax (rounded
 * once to float32, as nf4_dequantize) and s * sum_j A[k][j] B[j][n] (float32
 * accumulation), rounded once to out_dtype (LN_BF16: nearest-even). Then
 * x W'^T reproduces lora_nf4_fwd's y up to rounding.
 *   w_codes, w_absmax   as for lora_nf4_fwd ([d_out, d_in] base weight)
 *   A bf16 [d_in, r],  B bf16 [r, d_out]
 *   out  [d_out, d_in] of out_dtype (LN_BF16 or LN_F32), output
 * d_in % 64 == 0, d_out >= 1, 1 <= r <= LN_MAX_RANK; out disjoint from the inputs.
 */
int lora_nf4_merge(int64_t d_in, int64_t d_out, int32_t r, float lora_alpha, const uint8_t* w_codes,
                   const float* w_absmax, const uint16_t* A, const uint16_t* B, int out_dtype,
                   void* out, void* stream);

/* Workspace bytes lora_nf4_bwd needs for these sizes (0 if the sizes are invalid). */
size_t lora_nf4_bwd_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int32_t r);

/*
 * lora_nf4_bwd_noalloc — lora_nf4_bwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same results. Its
 * workspace is a scratch array the library owns, LN_NOALLOC_SCRATCH_BYTES of device
 * memory per GPU, reserved when the library's code is loaded on that GPU and held
 * until the process ends; the call itself allocates nothing. Where lora_nf4_bwd's
 * workspace fits the scratch it runs exactly that plan; otherwise the plan without
 * the dequantized weight copy (bf16 d_in x d_out bytes), which gives the same bits;
 * LN_EWORKSPACE if even that does not fit (the rank-r partial sums and G, U of very
 * large shapes). Every call on one GPU shares that GPU's scratch: calls that overlap
 * in time on one GPU (concurrent streams, several host threads) race and must be
 * serialized by the caller; calls on different GPUs are independent. The scratch
 * keeps the last call's contents; nothing in it needs to start at zero.
 */
#define LN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int lora_nf4_bwd_noalloc(int64_t T, int64_t d_in, int64_t d_out, int32_t r, float lora_alpha,
                         const uint16_t* x, const uint16_t* dy, const uint8_t* w_codes,
                         const float* w_absmax, const uint16_t* A, const uint16_t* B,
                         const uint16_t* u_saved, uint16_t* dx, uint16_t* dA, uint16_t* dB,
                         void* stream);

/*
 * lora_adamw_step — one AdamW update of a LoRA factor (A or B), the optimizer
 * phase of a training step ("Unsloth performance measured: is it really 2x
 * faster?", section 2.2 time table, optimizer.step row). Decoupled weight decay;
 * for every element i < n, as this fixed sequence of float32 operations, each
 * rounded to nearest-even:
 *     g = grad[i];  m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) (g g)
 *     p = p (1 - lr wd) - (lr / (1 - b1^step)) (m / (sqrt(v) (1 / sqrt(1 - b2^step)) + eps))
 * where each parenthesised constant is formed in float64 from the float32
 * arguments and rounded once. p stays float32 and p_bf16 = bf16(p) is the copy
 * lora_nf4_fwd / lora_nf4_bwd read.
 *   p       float32 [n] master copy (in/out)      p_bf16  bf16 [n] (out)
 *   grad    bf16 [n] (e.g. dA or dB of lora_nf4_bwd)
 *   m, v    float32 [n] first and second moments (in/out; zero before step 1)
 *   step    1-based step number (bias correction)
 * n >= 0 (0: nothing to do); eps > 0; 0 <= beta1, beta2 < 1; finite lr and
 * weight_decay. All arrays disjoint (LN_EALIAS), 16-byte aligned (LN_EALIGN).
 */
int lora_adamw_step(int64_t n, float* p, uint16_t* p_bf16, const uint16_t* grad, float* m, float* v,
                    int32_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                    void* stream);

/*
 * lora_adamw8_step — lora_adamw_step with 8-bit moments (the 8-bit AdamW of
 * "Reading the Unsloth changelog", section 1 memory list: optimizer state at a
 * quarter of float32). Each moment is stored blockwise, 256 consecutive elements
 * per block: one E4M3 code per element (OCP FP8 E4M3FN: nearest code, ties to
 * even, saturating at 448) and one float32 scale per block. A step decodes
 * m = f32(e4m3(code) * scale) (likewise v), runs lora_adamw_step's float32
 * update, and re-encodes: scale = f32(max |x| over the block / 448), code =
 * e4m3(f32(x / scale)), code 0 where the scale is 0.
 *   m_codes, v_codes    uint8 [n] (in/out; zero before step 1)
 *   m_scales, v_scales  float32 [ceil(n / 256)] (in/out; zero before step 1)
 *   the other arguments and rules as for lora_adamw_step.
 */
int lora_adamw8_step(int64_t n, float* p, uint16_t* p_bf16, const uint16_t* grad, uint8_t* m_codes,
                     float* m_scales, uint8_t* v_codes, float* v_scales, int32_t step, float lr, float beta1,
                     float beta2, float eps, float weight_decay, void* stream);

/*
 * lora_nf4_bwd_adamw — lora_nf4_bwd followed by lora_adamw_step of A and B, with
 * the update applied by the backward's final reduction of dA and dB: the
 * gradients are the float32 sums themselves (never rounded to bf16, never stored)
 * and A and B are rewritten in place as bf16 of their updated masters. The
 * optimizer phase then costs no launch of its own (the low-bit AdamW kernel of
 * "Unsloth performance measured: is it really 2x faster?", section 2.2 time
 * table). Use lora_nf4_bwd + lora_adamw_step where gradients accumulate over
 * several micro-batches before a step.
 *   A, B               bf16, read by the backward, then overwritten (in/out)
 *   a_master, a_m, a_v float32 [d_in, r]: A's master copy and moments (in/out)
 *   b_master, b_m, b_v float32 [r, d_out]: B's (in/out)
 *   step, lr, beta1, beta2, eps, weight_decay   as for lora_adamw_step
 *   the other arguments as for lora_nf4_bwd (dA, dB are not produced); the
 *   workspace is sized by lora_nf4_bwd_workspace_bytes.
 * T >= 1; r % 8 == 0 and r <= 64, d_out % 8 == 0 (the shapes whose rank-r
 * gradients take the one-launch reduction; LN_ERANK / LN_ESHAPE otherwise).
 * Every output (dx, A, B, the six state arrays, the workspace) disjoint from
 * every input and from the others (LN_EALIAS).
 */
int lora_nf4_bwd_adamw(int64_t T, int64_t d_in, int64_t d_out, int32_t r, float lora_alpha,
                       const uint16_t* x, const uint16_t* dy, const uint8_t* w_codes, const float* w_absmax,
                       uint16_t* A, uint16_t* B, const uint16_t* u_saved, uint16_t* dx, float* a_master,
                       float* a_m, float* a_v, float* b_master, float* b_m, float* b_v, int32_t step, float lr,
                       float beta1, float beta2, float eps, float weight_decay, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * lora_nf4_mfma_probe — measurement aid, no part of the linear: one launch of
 * v_mfma_f32_32x32x16_bf16 issued back to back on register operands (eight
 * independent accumulators per wave, two waves per SIMD, one 512-thread
 * workgroup on each of 256 CUs, no memory traffic), `iters` rounds of eight per
 * wave. Timing it (e.g. with HIP events on `stream`) gives the bf16 matrix-core
 * throughput the GPU sustains, the practical ceiling of the tile kernels next to
 * the published 2.5 PFLOP/s dense bf16 peak.
 *   iters  1 .. 2^20
 *   sink   device float32 [256], 16-byte aligned: one value per workgroup (output;
 *          keeps the work observable, value meaningless)
 * Returns the launch's floating-point operation count (2 x 32 x 32 x 16 per MFMA)
 * on success, a negative LN_* status otherwise (LN_EINVAL for bad arguments or a
 * launch error, LN_EALIGN).
 */
int64_t lora_nf4_mfma_probe(int32_t iters, float* sink, void* stream);

/*
 * lora_nf4_set_weight_staging — how the tile kernels at large token counts read
 * the NF4 weight, for every later call in the process.
 *   mode 0 (the default): every path dequantizes the packed weight inside its
 *          GEMM main loop, into LDS or straight into MFMA fragments (the fused
 *          design of "Unsloth acceleration principles: CUDA kernel fusion and
 *          memory optimization", kernel-fusion section); no bf16 copy of the
 *          weight exists at any time.
 *   mode 1: from 1024 tokens (4096 where the grid runs 256 x 256 tiles) the
 *          forward and dX first dequantize the weight to bf16 into their
 *          workspace (2 d_in d_out bytes per projection, see the
 *          *_workspace_bytes queries) and the tile kernels read that copy. The
 *          results are identical in value to mode 0's within the tolerance of
 *          the linear (the same dequantized bf16 weights; products summed in a
 *          different order). Measured on MI355X at 8192 tokens, 4096 -> 4096,
 *          r = 16: forward 257 us (mode 1) vs 287 us (mode 0), dX 250 vs 278 us.
 *   mode -1: query only.
 * Returns the mode in effect before the call (0 or 1), LN_EINVAL for any other
 * mode. Process-wide and read when a call is enqueued and when workspace sizes
 * are queried: set it before querying sizes and keep it while calls sized that
 * way are issued. Host function, no GPU work.
 */
int lora_nf4_set_weight_staging(int32_t mode);

/*
 * lora_nf4_rslora_alpha — the lora_alpha to pass to the entry points above so
 * that their scale lora_alpha / r (formed in float32) equals the rank-stabilized
 * scale alpha / sqrt(r) rounded to float32 (the --use_rslora option of "Reading
 * the Unsloth changelog", section 2.1). Exact whenever such a float32 exists
 * (always for power-of-two r); otherwise the one whose scale is nearest. Host
 * function, no GPU work. NaN for r outside [1, LN_MAX_RANK] or non-finite alpha.
 */
float lora_nf4_rslora_alpha(float lora_alpha, int32_t r);

/*
 * nf4_absmax_quantize / nf4_absmax_dequantize — double quantization of the
 * float32 block scales of an NF4 weight (the absmax array of nf4_quantize, n =
 * rows * cols / 64 entries in row-major order). The pages keep the base weight
 * resident in 4-bit form ("Reading the Unsloth changelog", section 1.1); the
 * scales are stored once more at 8 bits (QLoRA-style double quantization):
 * blocks of 256 consecutive scales (the last may be shorter); per block with
 * minimum lo and maximum hi, in float32 with nearest-even rounding per step:
 *     offset = lo/2 + hi/2,   d = max(hi - offset, offset - lo),   scale = d / 448
 *     code   = E4M3((a - offset) / scale)   (0 when scale == 0)
 * E4M3 = OCP FP8 E4M3FN, nearest value with ties to the even code, saturating
 * at +-448, sign from the input's sign bit. Dequantization gives
 *     a' = value(code) * scale + offset   (two roundings, no fused multiply-add),
 * which the NF4 entry points take in place of absmax. Storage: 8 bits per 64
 * weights plus 64 bits per 16384 weights, against 32 bits per 64 weights.
 *   absmax  float32 [n];  q  uint8 [n];  scale, offset  float32 [ceil(n / 256)]
 * n >= 0 (0: nothing to do); all pointers 16-byte aligned; outputs disjoint from
 * inputs. Scales must be finite.
 */
int nf4_absmax_quantize(const float* absmax, int64_t n, uint8_t* q, float* scale, float* offset,
                        void* stream);
int nf4_absmax_dequantize(const uint8_t* q, const float* scale, const float* offset, int64_t n,
                          float* absmax, void* stream);

/* A static, human-readable description of a status code. */
const char* lora_nf4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LORA_NF4_H */
