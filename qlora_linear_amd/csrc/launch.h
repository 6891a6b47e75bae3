// Internal launchers, one per kernel family. Arguments are already validated by
// the C-ABI layer (api.cpp); each launcher only enqueues work on `stream` and
// returns the hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lnf4 {

hipError_t launch_nf4_quantize(const void* w, bool w_is_bf16, int64_t rows, int64_t cols,
                               uint8_t* codes, float* absmax, hipStream_t stream);

hipError_t launch_nf4_dequantize(const uint8_t* codes, const float* absmax, int64_t rows,
                                 int64_t cols, bool out_bf16, void* out, hipStream_t stream);

// The packed weight of N rows x K columns transposed: codes_t [K][N/2] (code of
// (n, k) in byte n / 2 of row k, the even n in the low nibble) and absmax_t
// [K/64][N]. N % 128 == 0, K % 128 == 0.
hipError_t launch_nf4_transpose(const uint8_t* codes, const float* absmax, int64_t N, int64_t K,
                                uint8_t* codes_t, float* absmax_t, hipStream_t stream);

// MFMA-only throughput probe over every CU: returns the launch's FLOPs (-1 on a
// launch error); sink receives one float per workgroup (256).
int64_t launch_mfma_probe(int iters, float* sink, hipStream_t stream);

// Zero n 16-bit elements (a fill kernel, so the call can sit in a captured graph).
hipError_t launch_zero_u16(uint16_t* p, int64_t n, hipStream_t stream);

hipError_t launch_lora_fwd_generic(int T, int K, int N, int r, float s, const uint16_t* x,
                                   const uint8_t* codes, const float* absmax, const uint16_t* A,
                                   const uint16_t* B, uint16_t* y, uint16_t* u_save,
                                   hipStream_t stream);

// Forward dispatch: generic kernels (ranks not a multiple of 8 or above 64, operands
// past the buffer range), split-K weight streaming (few tokens; needs a workspace of
// fwd_workspace_bytes), tiled kernels otherwise. `workspace` may be null when
// fwd_workspace_bytes is 0.
size_t fwd_workspace_bytes(int64_t T, int64_t K, int64_t N, int r);
hipError_t launch_lora_fwd(int T, int K, int N, int r, float s, const uint16_t* x,
                           const uint8_t* codes, const float* absmax, const uint16_t* A,
                           const uint16_t* B, uint16_t* y, uint16_t* u_save, void* workspace,
                           hipStream_t stream);

// Several projections of the same x (q/k/v, gate/up) in one forward launch when
// every projection takes the tiled kernels; otherwise one forward per projection,
// one after the other on the stream, sharing the workspace (the largest of theirs).
constexpr int kMaxProj = 8;
size_t fwd_multi_workspace_bytes(int64_t T, int64_t K, int n_proj, const int* N, int r);
hipError_t launch_lora_fwd_multi(int T, int K, int n_proj, const int* N, int r, float s,
                                 const uint16_t* x, const uint8_t* const* codes,
                                 const float* const* absmax, const uint16_t* const* A,
                                 const uint16_t* const* B, uint16_t* const* y,
                                 uint16_t* const* u_save, void* workspace, hipStream_t stream);

// Projections of one tiled forward launch (a single projection is a one-entry
// table); tile_end[g] = column tiles of projections 0..g.
struct ProjTable {
  int n;
  int tile_end[kMaxProj];
  int N[kMaxProj];
  const uint8_t* codes[kMaxProj];
  const float* absmax[kMaxProj];
  const uint16_t* wdq[kMaxProj];  // bf16 [N][K] dequantized weight (DQ kernels only)
  const uint16_t* usg[kMaxProj];  // bf16(s U) [T][r] from the U pass (RU = 0 kernels only)
  int us_stride;                  // row stride of usg (register-dequantizing kernel)
  const uint16_t* A[kMaxProj];
  const uint16_t* B[kMaxProj];
  uint16_t* y[kMaxProj];
  uint16_t* u[kMaxProj];
};

// U = x A of up to LN_MAX_PROJ projections that share x, in one pass over x:
// us [T][n r] bf16(s U) side by side (set by launch_upass inside the workspace),
// u[g] [T][r] bf16(U_g) (nullable). n r <= 256.
struct UpassTable {
  int n;
  const uint16_t* A[kMaxProj];
  uint16_t* u[kMaxProj];
  uint16_t* us;
  int us_stride;  // row stride of us (elements); 0: n r
};
size_t upass_table_bytes(int64_t T, int64_t K, int n, int r);
hipError_t launch_upass(int T, int K, int r, float s, const uint16_t* x, UpassTable& tab, void* workspace,
                        hipStream_t stream);
// G = bf16(s dY B^T) of one projection (r <= 64, d_out % 256 == 0) into columns
// 0 .. r - 1 of g [T][g_stride]: the U pass with dY for x and B (r rows along
// d_out) for A^T.
hipError_t launch_gpass(int T, int N, int r, float s, const uint16_t* dy, const uint16_t* B, uint16_t* g,
                        int g_stride, hipStream_t stream);

// Register-dequantizing forward (256 x 256 tiles, eight waves of 256 x 32): the
// packed NF4 codes of a K-step go straight into MFMA B fragments in registers,
// x runs through a four-stage LDS pipeline; at rank 16 U = x A is formed in the
// K loop, otherwise bf16(s U) is read from tab.usg (the U pass).
bool fwd_rw_supported(int64_t T, int64_t K, int r);
// Weight staging (lora_nf4_set_weight_staging): false (default) = every tile path
// dequantizes in its main loop; true = from 1024 / 4096 tokens the weight is
// dequantized to bf16 once into the workspace and the tile kernels read that.
bool weight_staging();
bool fwd_rw_inloop_u(int r);  // the kernel computes U itself (no U pass, no workspace)
hipError_t launch_fwd_rw(int T, int K, int r, float s, const uint16_t* x, const ProjTable& tab,
                         hipStream_t stream);
// dX on register-dequantized 256 x 256 tiles (rank 16, from 4096 tokens, d_in and
// d_out multiples of 256): the packed weight is transposed into the workspace
// (dx_rw_bytes), then one launch forms dX and bf16(s G) into g_out [T][16]. dx
// null: G only (the same tiles' G, one column tile per token tile).
bool dx_rw_supported(int64_t T, int64_t K, int64_t N, int r);
size_t dx_rw_bytes(int64_t K, int64_t N);
hipError_t launch_dx_rw(int T, int K, int N, float s, const uint16_t* dy, const uint8_t* codes,
                        const float* absmax, const uint16_t* A, const uint16_t* B, uint16_t* dx,
                        uint16_t* g_out, void* workspace, hipStream_t stream);

// Split-K weight-streaming forward for up to 128 tokens (r % 8 == 0, r <= 64):
// workgroups of 64 weight rows x one of `splits` d_in chunks (plus one per split
// and 16-wide rank block for U), fp32 partials [splits][T][N] and [splits][T][r]
// in the workspace, then one reduce that stores y and U.
struct SplitKPlan {
  int ncb;          // 64-row column blocks
  int splits;       // d_in chunks (each non-empty)
  int steps_per;    // 128-element reduction steps per chunk
  size_t part_bytes, bytes;
};
bool lora_fwd_splitk_supported(int64_t T, int r);
// y = bf16(sum_sp part[sp] + bf16(s sum_sp upart[sp]) B), u_save = bf16(sum_sp upart)
// (nullable), for part [S][T][N] and upart [S][T][r] fp32, S <= 16.
hipError_t launch_fwd_splitk_reduce(int T, int N, int r, int S, float s, const float* part,
                                    const float* upart, const uint16_t* B, uint16_t* y, uint16_t* u_save,
                                    hipStream_t stream);
SplitKPlan plan_fwd_splitk(int T, int K, int N, int r);
hipError_t launch_lora_fwd_splitk(int T, int K, int N, int r, float s, const uint16_t* x,
                                  const uint8_t* codes, const float* absmax, const uint16_t* A,
                                  const uint16_t* B, uint16_t* y, uint16_t* u_save, void* workspace,
                                  hipStream_t stream);

// Weight-streaming forward for a few tokens (1 <= T <= 32, r % 8 == 0, r <= 64):
// one workgroup per 16 weight rows, no workspace.
bool lora_fwd_stream_supported(int64_t T, int r);
hipError_t launch_lora_fwd_stream(int T, int K, int N, int r, float s, const uint16_t* x,
                                  const uint8_t* codes, const float* absmax, const uint16_t* A,
                                  const uint16_t* B, uint16_t* y, uint16_t* u_save, hipStream_t stream);

// Merged base weight W' = D + s (A B)^T, [N, K], bf16 or float32 (any r <= 128).
hipError_t launch_lora_merge(int K, int N, int r, float s, const uint8_t* codes, const float* absmax,
                             const uint16_t* A, const uint16_t* B, bool out_bf16, void* out,
                             hipStream_t stream);

// dX kernel for ranks r % 8 == 0, r <= 64 (256 x 256 or 128 x 128 tiles); also
// writes bf16 G = s dY B^T [T, r] to g_out. With part_x / part_g (sized by
// dx_tiled_split: [splits][T][K] and [splits][T][r] fp32) a small tile grid splits
// its reduction over d_out and the split-K dX reduce finishes; null: no split.
bool lora_dx_supported(int r);
struct DxTiledSplit {
  int splits, steps_per;
};
DxTiledSplit dx_tiled_split(int64_t T, int64_t K, int64_t N, int r);
// wdq: bf16 [N][K] deq(W) written beforehand (then codes and absmax are not read),
// or nullptr to dequantize in the loop.
hipError_t launch_lora_dx(int T, int K, int N, int r, float s, const uint16_t* dy,
                          const uint8_t* codes, const float* absmax, const uint16_t* A,
                          const uint16_t* B, const uint16_t* wdq, uint16_t* dx, uint16_t* g_out, float* part_x,
                          float* part_g, hipStream_t stream, bool g_ready = false);
// Whether the tiled dX takes a weight dequantized beforehand (large token counts).
bool dx_dq(int64_t T, int64_t K, int64_t N, int r);

// The dX kernel over a table of projections that share x: the reduction runs over
// their concatenated d_out (step_end[g] = 64-wide steps of projections 0..g) and
// dX = sum_g dY_g D_g + G_g A_g^T; g_out [T][n r] receives every G_g side by side.
// A one-entry table is the single-projection kernel.
struct DxTable {
  int n;
  int step_end[kMaxProj];
  int N[kMaxProj];
  const uint16_t* dy[kMaxProj];
  const uint8_t* codes[kMaxProj];
  const float* absmax[kMaxProj];
  const uint16_t* A[kMaxProj];
  const uint16_t* B[kMaxProj];
  // bf16 [N][K] dequantized weights; when wdq[0] is non-null every entry is set and
  // the kernel reads these instead of the codes
  const uint16_t* wdq[kMaxProj];
};
// Several projections take this kernel when every d_out is a multiple of 64 and
// r % 8 == 0, r <= 64 (rank sums above 64 take several epilogue passes).
bool lora_dx_multi_supported(int n_proj, const int* N, int r);
// g_ready: G (bf16, [T][n r]) is already in g_out (launch_gpass); the tiles then
// read it in their epilogue instead of forming it in the K loop.
hipError_t launch_lora_dx_table(int T, int K, int r, float s, const DxTable& tab, uint16_t* dx,
                                uint16_t* g_out, hipStream_t stream, bool g_ready = false);

// Split-K weight-streaming dX for up to 128 tokens (r % 8 == 0, r <= 64):
// workgroups of 128 d_in columns x one of `splits` d_out slices (plus one per slice
// and 16-wide rank block for G), fp32 partials part_x [splits][T][K] and part_g
// [splits][T][r], then one reduce that stores dX (if non-null) and bf16 G.
struct DxSplitPlan {
  int kcb;              // 128-column blocks of d_in
  int splits;           // d_out slices (each non-empty)
  int rows_per_split;   // multiple of 64
  bool tr;              // the transposing-code kernel (up to 32 tokens, long slices)
  size_t part_x_bytes, part_g_bytes;
};
bool lora_dx_splitk_supported(int64_t T, int r);
DxSplitPlan plan_dx_splitk(int64_t T, int64_t K, int64_t N, int r);
// dX = sum_sp part_x[sp] + bf16(G) A^T, G = s sum_sp part_g[sp]; g_out = bf16(G);
// S <= 16; dx may be null (G only).
hipError_t launch_dx_splitk_reduce(int T, int K, int r, int S, float s, const float* part_x,
                                   const float* part_g, const uint16_t* A, uint16_t* dx, uint16_t* g_out,
                                   hipStream_t stream);
hipError_t launch_lora_dx_splitk(int T, int K, int N, int r, float s, const uint16_t* dy,
                                 const uint8_t* codes, const float* absmax, const uint16_t* A,
                                 const uint16_t* B, uint16_t* dx, uint16_t* g_out, float* part_x,
                                 float* part_g, hipStream_t stream);

// The tiled, few-token and rank-r-gradient kernels address operands through
// buffer resources (at most 2^31 - 1 bytes) and move rows of d_out elements in
// 16-byte pieces: they are used only when every operand they cover fits and
// d_out % 8 == 0. Other shapes take the generic kernels.
inline bool fits_buffer(int64_t T, int64_t K, int64_t N) {
  const int64_t lim = 0x7FFFFF00;  // below kOutOfRange (device_common.h)
  return N % 8 == 0 && T * K * 2 < lim && T * N * 2 < lim && N * K / 2 < lim && N * (K / 64) * 4 < lim &&
         K * 128 * 2 < lim && N * 64 * 2 < lim;
}

// 16-column rank tiles of the generic kernels' instances: every count up to 8
// (r <= 128), then 12 (r <= 192) and 16 (r <= 256).
inline int generic_rank_tiles(int r) { return r <= 128 ? (r + 15) / 16 : (r <= 192 ? 12 : 16); }

// One AdamW step's float32 constants, formed in float64 and rounded once (see
// adamw_elem in device_common.h).
struct AdamWArgs {
  float beta1, one_m_beta1, beta2, one_m_beta2, eps;
  float decay;          // 1 - lr * weight_decay
  float step_size;      // lr / (1 - beta1^t)
  float inv_sqrt_bc2;   // 1 / sqrt(1 - beta2^t)
};
AdamWArgs adamw_args(int step, float lr, float beta1, float beta2, float eps, float weight_decay);
// AdamW of a LoRA factor with float32 moments m, v [n].
hipError_t launch_adamw(int64_t n, float* p, uint16_t* p_bf16, const uint16_t* g, float* m, float* v,
                        const AdamWArgs& h, hipStream_t stream);
// AdamW with 8-bit blockwise moments: E4M3 codes [n] and float32 scales [ceil(n / 256)].
hipError_t launch_adamw8(int64_t n, float* p, uint16_t* p_bf16, const uint16_t* g, uint8_t* m_codes,
                         float* m_scales, uint8_t* v_codes, float* v_scales, const AdamWArgs& h,
                         hipStream_t stream);
// The AdamW state of one LoRA factor updated in place by the fused backward: float32
// master copy, the bf16 factor the kernels read, float32 moments.
struct AdamState {
  float* p;
  uint16_t* w;
  float* m;
  float* v;
};

// Double quantization of n float32 block scales: E4M3 codes, one float32 scale
// and offset per 256 scales; and its inverse.
// The float32-moment AdamW step of A and B, applied by the rank-r reduction in
// place of storing dA and dB (one projection).
struct SkinnyAdamW {
  AdamState a, b;
  AdamWArgs h;
};

// Rank-r gradients dA, dB in one launch plus one reduce (ranks % 8 == 0, <= 64):
// dA = x^T G over K columns with G [T][ra] at row stride vsa (>= ra: a column
// slice of a wider array), dB = s U^T dY over N columns with U [T][rb]; K = 0 or
// N = 0 leaves that job out. dA's ra columns are split into
// projections of da.gw columns each, projection g stored at da.p[g] as [K][gw].
// part_a: [splits][ra][K] fp32, part_b: [splits][rb][N] fp32.
struct DaOut {
  uint16_t* p[kMaxProj];
  int gw;
};
bool lora_skinny_supported(int r);
// the rank-r gradient kernel for a side-by-side G of several projections (dA only)
bool lora_skinny_wide_supported(int r);
int skinny_splits(int64_t T, int64_t K, int64_t N);
// token splits for `blocks` 256-column blocks in one launch
int skinny_splits_blocks(int64_t T, int64_t blocks);

// One job of a rank-r gradient launch: M^T V reduced over the T tokens, M [T][C]
// (x or dY), V [T][vstr] of which the first r columns are used (G or U; r % 8 == 0,
// r <= 192), fp32 partials [splits][r][C] at part. is_a (first job only): dA,
// stored through the DaOut split, unscaled; otherwise out [r][C] = bf16(s sum) (dB).
constexpr int kMaxSkinnyJobs = kMaxProj + 1;
struct SkinnyJob {
  const uint16_t* M;
  const uint16_t* V;
  float* part;
  uint16_t* out;
  int C, r, vstr;
  bool is_a;
};
// Up to kMaxSkinnyJobs jobs in one partial-sum launch (every job's column blocks x
// the same token splits) and one reduce: several projections' dB in one pass.
hipError_t launch_skinny_jobs(int T, int n, const SkinnyJob* jobs, int splits, float s, const DaOut& da,
                              hipStream_t stream, const SkinnyAdamW* adam = nullptr);
hipError_t launch_lora_skinny(int T, int K, int N, int ra, int rb, int vsa, float s, const uint16_t* x,
                              const uint16_t* g, const uint16_t* dy, const uint16_t* u,
                              float* part_a, float* part_b, int splits, const DaOut& da,
                              uint16_t* dB, hipStream_t stream, const SkinnyAdamW* adam = nullptr);

// The rank-r gradients alone (dA = x^T G, dB = s U^T dY from bf16 G [T][r] and U
// [T][r]): partials [splits_a][K][rs] at offset 0 and [splits_b][N][rs] at off_pb.
struct GradPlan {
  bool fast;  // the one-launch rank-r kernel (r % 8 == 0, r <= 64)
  int rs, splits_a, splits_b;
  size_t off_pb, bytes;
};
GradPlan plan_grad_ab(int64_t T, int64_t K, int64_t N, int r);
hipError_t launch_grad_ab(int T, int K, int N, int r, float s, const uint16_t* x, const uint16_t* g,
                          const uint16_t* dy, const uint16_t* u, uint16_t* dA, uint16_t* dB, void* workspace,
                          const GradPlan& p, hipStream_t stream);

// Backward plan: how the workspace is carved. Shared by the launcher and the
// workspace-size query so the two always agree.
struct BwdPlan {
  bool fast;          // 256 x 256 dX kernel and the one-launch rank-r gradients
  bool splitk;        // up to 128 tokens: split-K weight-streaming dX (with the fast rank-r gradients)
  int splits_x;       // d_out slices of the split-K dX
  int rp;             // r rounded up to the MFMA reduction granularity (32)
  int splits_a;       // token splits of the dA reduction
  int splits_b;       // token splits of the dB reduction
  size_t off_g, off_u, off_pa, off_pb;  // byte offsets into the workspace
  size_t off_px, off_pg;                // weight-streaming dX partials
  bool dqx;                             // tiled dX on the dequantized weight (dx_dq)
  bool rwx;                             // dX on register-dequantized tiles (dx_rw_supported)
  size_t off_w;                         // dqx: that weight, bf16 [N][K]; rwx: the transposed packed weight
  bool gpass;                           // G from a G pass (launch_gpass), the tiles at RU = 0
  size_t bytes;       // total workspace bytes
};
// allow_dq = false: never the dequantized-weight dX (its workspace holds 2 d_in d_out
// bytes more); the results are the same bits either way.
BwdPlan plan_bwd(int64_t T, int64_t K, int64_t N, int r, bool allow_dq = true);

hipError_t launch_lora_bwd(int T, int K, int N, int r, float s, const uint16_t* x,
                           const uint16_t* dy, const uint8_t* codes, const float* absmax,
                           const uint16_t* A, const uint16_t* B, const uint16_t* u_saved,
                           uint16_t* dx, uint16_t* dA, uint16_t* dB, void* workspace,
                           const BwdPlan& plan, hipStream_t stream, const SkinnyAdamW* adam = nullptr);
// Whether the backward can apply AdamW in its rank-r reduction (plan.fast).
inline bool bwd_adamw_supported(const BwdPlan& plan) { return plan.fast; }

// Backward of several projections that share x (dX summed over them). Fused: one
// dX launch over all projections (G side by side in [T][n r]); for n r <= 64 one
// rank-r launch for every dA (one pass over x) and every dB, for n r <= 192 one for
// every dA and one for every dB, else one per projection for its dA and dB.
// Otherwise (ragged d_out, up to 128 tokens) one backward per projection, dX
// accumulated from a scratch copy.
struct BwdMultiPlan {
  bool fused;
  int n, R;                   // projections, n r
  int splits_a;               // fused: token splits of the launch with every dA
  int splits_b[kMaxProj];     // fused: [0] of the launch with every dB (n r <= 192), else
                              // [g] of projection g's own launch (g >= 1)
  size_t off_g, off_u, off_pa, off_pb;  // fused
  bool dq;                              // fused: dX on the dequantized weights (dx_dq)
  size_t off_w[kMaxProj];               // those weights, bf16 [N_g][K]
  size_t off_single, off_dxt;           // per-projection fallback
  size_t bytes;
};
BwdMultiPlan plan_bwd_multi(int64_t T, int64_t K, int n, const int* N, int r);
hipError_t launch_lora_bwd_multi(int T, int K, int n, const int* N, int r, float s, const uint16_t* x,
                                 const uint16_t* const* dy, const uint8_t* const* codes,
                                 const float* const* absmax, const uint16_t* const* A,
                                 const uint16_t* const* B, const uint16_t* const* u_saved, uint16_t* dx,
                                 uint16_t* const* dA, uint16_t* const* dB, void* workspace,
                                 const BwdMultiPlan& p, hipStream_t stream);

// AdamW step of one parameter array (float32 master p, bf16 copy, bf16 gradient
// and moments), elementwise over n elements.
hipError_t launch_absmax_dq(int64_t n, const float* absmax, uint8_t* q, float* scale, float* offset,
                            hipStream_t stream);
hipError_t launch_absmax_undq(int64_t n, const uint8_t* q, const float* scale, const float* offset,
                              float* out, hipStream_t stream);

}  // namespace lnf4
