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
                          float* part_g, hipStream_t stream);
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
// n r <= 64 (r % 8 == 0).
bool lora_dx_multi_supported(int n_proj, const int* N, int r);
hipError_t launch_lora_dx_table(int T, int K, int r, float s, const DxTable& tab, uint16_t* dx,
                                uint16_t* g_out, hipStream_t stream);

// Split-K weight-streaming dX for up to 128 tokens (r % 8 == 0, r <= 64):
// workgroups of 128 d_in columns x one of `splits` d_out slices (plus one per slice
// and 16-wide rank block for G), fp32 partials part_x [splits][T][K] and part_g
// [splits][T][r], then one reduce that stores dX (if non-null) and bf16 G.
struct DxSplitPlan {
  int kcb;              // 128-column blocks of d_in
  int splits;           // d_out slices (each non-empty)
  int rows_per_split;   // multiple of 64
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

// Buffer resources address at most 2^31 - 1 bytes; the 256 x 256 kernels are
// used only when every operand they cover fits.
inline bool fits_buffer(int64_t T, int64_t K, int64_t N) {
  const int64_t lim = (int64_t(1) << 31) - 1;
  return T * K * 2 < lim && T * N * 2 < lim && N * K / 2 < lim && N * (K / 64) * 4 < lim &&
         K * 128 * 2 < lim && N * 64 * 2 < lim;
}

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
int skinny_splits(int64_t T, int64_t K, int64_t N);
hipError_t launch_lora_skinny(int T, int K, int N, int ra, int rb, int vsa, float s, const uint16_t* x,
                              const uint16_t* g, const uint16_t* dy, const uint16_t* u,
                              float* part_a, float* part_b, int splits, const DaOut& da,
                              uint16_t* dB, hipStream_t stream);

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
  size_t off_w;                         // that weight, bf16 [N][K]
  size_t bytes;       // total workspace bytes
};
BwdPlan plan_bwd(int64_t T, int64_t K, int64_t N, int r);

hipError_t launch_lora_bwd(int T, int K, int N, int r, float s, const uint16_t* x,
                           const uint16_t* dy, const uint8_t* codes, const float* absmax,
                           const uint16_t* A, const uint16_t* B, const uint16_t* u_saved,
                           uint16_t* dx, uint16_t* dA, uint16_t* dB, void* workspace,
                           const BwdPlan& plan, hipStream_t stream);

// Backward of several projections that share x (dX summed over them). Fused: one
// dX launch over all projections (G side by side in [T][n r]); for n r <= 64 one
// pass over x for every dA with the first projection's dB and one pass per further
// dB, else one pass per projection for its dA and dB. Otherwise (ragged d_out, up
// to 128 tokens) one backward per projection, dX accumulated from a scratch copy.
struct BwdMultiPlan {
  bool fused;
  int n, R;                   // projections, n r
  int splits_a;               // fused: token splits of the first rank-r pass
  int splits_b[kMaxProj];     // fused: token splits of the passes of projections 1 ..
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
hipError_t launch_adamw(int64_t n, float* p, uint16_t* p_bf16, const uint16_t* g, uint16_t* m,
                        uint16_t* v, int step, float lr, float beta1, float beta2, float eps,
                        float weight_decay, hipStream_t stream);

// Double quantization of n float32 block scales: E4M3 codes, one float32 scale
// and offset per 256 scales; and its inverse.
hipError_t launch_absmax_dq(int64_t n, const float* absmax, uint8_t* q, float* scale, float* offset,
                            hipStream_t stream);
hipError_t launch_absmax_undq(int64_t n, const uint8_t* q, const float* scale, const float* offset,
                              float* out, hipStream_t stream);

}  // namespace lnf4
