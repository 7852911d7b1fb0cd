/*
 * vdn.h — C ABI of the MI355X (gfx950) Video DeltaNet hybrid video-to-video
 * attention layer, forward pass.
 *
 * The layer (sources cited by page title and section):
 *  - Softmax branch: latent frames form chunks of `chunk_frames` (five); a query
 *    chunk sees its own chunk and `window_chunks` chunks either side; every
 *    frame also sees the first and last frame, those two anchors see the whole
 *    sequence, and text tokens stay visible as softmax keys.
 *    [PaperDaily "伯克利与Impossible视频生成:14.3秒视频6.70秒去噪" §二;
 *     arXiv listing "Video DeltaNet: A Video-Native Hybrid Attention for
 *     Livestream Video Generation", abstract]
 *  - Linear branch (Video Delta Attention): per frame the state is updated
 *    once, jointly over all the frame's tokens, by
 *    S <- (alpha_f S + B_f)(I + A_f)^-1 with A_f = sum beta k k^T and
 *    B_f = sum beta v k^T.  A forward and a backward state start from half of
 *    the text write, skip the anchors, and each frame reads only the far
 *    frames outside its window; the two reads are summed.
 *    [deepmagic blog "生成比播放還快：Video DeltaNet 用 11 秒產出 14 秒 768p
 *     影片", section 用兩條分支取代一條; PaperDaily §三, §四]
 *  - Merge: the summed read is RMS-normalised, then each branch is scaled by
 *    its own sigmoid gate and the two are added.  [PaperDaily §三]
 *
 * Conventions for every entry point:
 *  - All tensors are dense, row-major, innermost dimension unit-stride, in
 *    device memory owned by the caller.  Token-major "BNHD" layout:
 *      q, k, v, o        [B, T*P, H, d]           (layout->dtype)
 *      text_k, text_v    [B, L, H, d]             (layout->dtype)
 *      beta              [B, T*P + L, H]          float32, video tokens then text
 *      alpha             [B, T, H]                float32, one decay per frame
 *      gate_logits       [B, T*P, H, 2]           float32, [...,0] softmax gate,
 *                                                 [...,1] linear gate
 *  - Device pointers must be 16-byte aligned.  text_k/text_v may be NULL when
 *    L == 0.
 *  - Argument errors are detected on the host before anything is enqueued and
 *    leave every output untouched.  Work is enqueued on `stream`; the call
 *    never synchronises the host.  Kernel faults surface through the stream.
 *  - The library never allocates device memory in these calls; scratch memory
 *    is the caller's `workspace`.
 *  - Calls are re-entrant; concurrent calls must use distinct workspaces.
 */
#ifndef VDN_H
#define VDN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VDN_VERSION 100   /* 1.0.0 */

typedef enum {
  VDN_OK = 0,
  VDN_ERR_NULL_ARG = 1,            /* a required pointer is NULL */
  VDN_ERR_BAD_SHAPE = 2,           /* a size is out of range */
  VDN_ERR_UNSUPPORTED = 3,         /* dtype / head size not implemented */
  VDN_ERR_MISALIGNED = 4,          /* a device pointer is not 16-byte aligned */
  VDN_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace_bytes below the required size */
  VDN_ERR_HIP = 6,                 /* a HIP launch failed; see vdn_last_hip_error */
  VDN_ERR_SCRATCH_TOO_SMALL = 7    /* the layout needs more than the built-in scratch of
                                      vdn_hybrid_attn_fwd_noalloc */
} vdn_status_t;

typedef enum { VDN_F32 = 0, VDN_BF16 = 1 } vdn_dtype_t;

/* Shape and geometry of one call.
 *  batch, heads        B, H >= 1
 *  head_dim_k/_v       d; equal, in {16, 32, 64, 128}
 *  frames              T >= 1 latent frames
 *  tokens_per_frame    P >= 1 (frame t holds video tokens t*P .. t*P+P-1)
 *  chunk_frames        C >= 1 (five in the pages)
 *  window_chunks       w >= 0 (one in the pages: previous and next chunk)
 *  anchor_first/_last  0/1: frame 0 / frame T-1 is a boundary anchor
 *  text_tokens         L >= 0 text tokens, visible softmax keys for every query
 *  dtype               vdn_dtype_t of q, k, v, text_k, text_v, o
 *  softmax_scale       0 -> 1/sqrt(d)
 *  rms_eps             0 -> 1e-6
 * Limits: B*T*P*H*d and (T*P+L)*H*d below 2^31 elements per batch entry set. */
typedef struct {
  int32_t batch, heads, head_dim_k, head_dim_v;
  int32_t frames, tokens_per_frame;
  int32_t chunk_frames, window_chunks;
  int32_t anchor_first, anchor_last;
  int32_t text_tokens;
  int32_t dtype;
  float softmax_scale;
  float rms_eps;
} vdn_layout_t;

/* Library version (VDN_VERSION of the built library). */
int vdn_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* vdn_status_str(vdn_status_t status);

/* hipError_t of the most recent VDN_ERR_HIP on the calling thread (0 if none). */
int vdn_last_hip_error(void);

/* Diagnostics for a failing call (not part of the method).  Name of the stage
 * (kernel launch: "vda_stats", "scan_split", "softmax_merge", ...) whose launch
 * failed most recently on the calling thread, or NULL if none has.  With the
 * environment variable VDN_SYNC_DEBUG=1 set before the first call, every stage
 * synchronises its stream and checks for errors, so a fault during a kernel is
 * reported by the call and stage that launched it (not on a stream under graph
 * capture; slower).  With VDN_ROCTX=1, each stage is bracketed by a roctx range
 * when the ROCm roctx library can be loaded.  The returned string is static. */
const char* vdn_last_failed_stage(void);

/* Host-only check of a layout: returns VDN_OK, VDN_ERR_NULL_ARG,
 * VDN_ERR_BAD_SHAPE or VDN_ERR_UNSUPPORTED.  Touches no device. */
vdn_status_t vdn_validate_layout(const vdn_layout_t* layout);

/* Number of chunks ceil(T / C); slot index of the text-only state in the
 * per-chunk state arrays below.  0 for an invalid layout.  Host only. */
int32_t vdn_num_chunks(const vdn_layout_t* layout);

/* Bytes of workspace vdn_hybrid_attn_fwd needs for `layout` (0 if the layout is
 * invalid).  Host only. */
size_t vdn_hybrid_attn_workspace_size(const vdn_layout_t* layout);

/* The whole layer: O = sigmoid(g0) * O_soft + sigmoid(g1) * RMSNorm(R q), with
 * O_soft the block-sparse softmax branch and R the summed forward/backward
 * VDA states of the query's chunk (the text write alone for anchor frames).
 * o must not alias any input.  workspace: device memory of at least
 * vdn_hybrid_attn_workspace_size(layout) bytes, 256-byte aligned; its contents
 * on entry are ignored.  Softmax scores (bf16 layouts, d >= 32, P and L
 * multiples of 8): formed from q * scale * log2(e) rounded to bf16, which
 * perturbs each score by about 2^-9 of its terms; with the environment
 * variable VDN_EXACT_SCORES=1 (read at every call) they are formed exactly in
 * float32 instead, about 4 % slower.  [all sections cited above] */
vdn_status_t vdn_hybrid_attn_fwd(const void* q, const void* k, const void* v,
                                 const void* text_k, const void* text_v,
                                 const float* beta, const float* alpha,
                                 const float* gate_logits,
                                 const vdn_layout_t* layout, void* o,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Size of the device scratch array vdn_hybrid_attn_fwd_noalloc uses in place
 * of a workspace (64 MiB; each GPU the library runs on holds one copy until
 * the process ends). */
#define VDN_NOALLOC_SCRATCH_BYTES (64u << 20)

/* vdn_hybrid_attn_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and output, with the workspace taken from a
 * static device array of VDN_NOALLOC_SCRATCH_BYTES instead of a caller's
 * buffer.  The call allocates nothing (no hipMalloc, no library allocation);
 * its first call on a device looks the array up there.  Layouts whose
 * workspace (vdn_hybrid_attn_workspace_size) exceeds the array are rejected
 * with VDN_ERR_SCRATCH_TOO_SMALL before anything is enqueued.  Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 * Nothing in the array needs to start at zero (every region is written
 * before it is read). */
vdn_status_t vdn_hybrid_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                         const void* text_k, const void* text_v,
                                         const float* beta, const float* alpha,
                                         const float* gate_logits,
                                         const vdn_layout_t* layout, void* o,
                                         hipStream_t stream);

/* ---- Per-stage entry points: the same kernels the layer runs, one stage at
 * ---- a time (for checking and profiling each stage). ---- */

/* Bytes of workspace vdn_softmax_fwd needs for `layout` (0 when the layout
 * needs none or is invalid).  Host only. */
size_t vdn_softmax_workspace_size(const vdn_layout_t* layout);

/* Softmax branch alone: o_soft [B, T*P, H, d] (layout->dtype) gets, for every
 * video query, one softmax over the keys of its visible frames together with
 * all text keys, times the matching values.  workspace: device memory of at
 * least vdn_softmax_workspace_size(layout) bytes (may be NULL when that is 0),
 * used for a transposed copy of V.  [PaperDaily §二; arXiv abstract] */
vdn_status_t vdn_softmax_fwd(const void* q, const void* k, const void* v,
                             const void* text_k, const void* text_v,
                             const vdn_layout_t* layout, void* o_soft,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Softmax branch and merge in one pass (the layer's last stage):
 *   o = sigmoid(g0) * O_soft + sigmoid(g1) * RMSNorm(R[c] q)
 * with O_soft as in vdn_softmax_fwd (kept in float32, not rounded, before
 * the merge) and R from vdn_vda_factor_scan (slot nc for anchor frames).
 * Covers bf16 layouts with d in {32, 64, 128} and P, L multiples of 8;
 * returns VDN_ERR_UNSUPPORTED otherwise (vdn_softmax_fwd + vdn_merge cover
 * every layout).  workspace: as for vdn_softmax_fwd.  o must not alias any
 * input.  [PaperDaily §二, §三; arXiv abstract] */
vdn_status_t vdn_softmax_merge_fwd(const void* q, const void* k, const void* v,
                                   const void* text_k, const void* text_v,
                                   const float* R, const float* gate_logits,
                                   const vdn_layout_t* layout, void* o,
                                   void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* The two gated branches side by side, the input of the per-branch output
 * projections: x2 [B, T*P, 2, H, d] (layout->dtype) with
 *   x2[b][n][0][h] = sigmoid(g0) * O_soft,  x2[b][n][1][h] = sigmoid(g1) * RMSNorm(R[c] q)
 * (O_soft and R q kept in float32 until this final rounding).  Covers the
 * layouts vdn_softmax_merge_fwd covers, else VDN_ERR_UNSUPPORTED.
 * workspace: as for vdn_softmax_fwd.  x2 must not alias any input.
 * [PaperDaily §三, figure 3 (each branch has its own gate and output
 *  projection); arXiv abstract (separate output projections)] */
vdn_status_t vdn_softmax_branches_fwd(const void* q, const void* k, const void* v,
                                      const void* text_k, const void* text_v,
                                      const float* R, const float* gate_logits,
                                      const vdn_layout_t* layout, void* x2,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* Output projections of the two branches as one product:
 *   y[m][n] = sum_k x[m][k] * w[n][k]     (fp32 accumulation)
 * x: bf16 [M, K] row-major (M tokens; per token the K = 2*H*d values of x2),
 * w: bf16 [N, K] row-major = [W_softmax | W_linear] in (out, in) order, softmax
 * branch columns first, y: bf16 [M, N].  So y = W_s x_s + W_l x_l per token,
 * each branch through its own matrix.  Needs K a positive multiple of 64 and
 * N a multiple of 8 (else VDN_ERR_UNSUPPORTED); y must not alias x or w.
 * [PaperDaily §三, figure 3; arXiv abstract] */
vdn_status_t vdn_out_proj(const void* x, const void* w, int64_t M, int32_t K, int32_t N,
                          void* y, hipStream_t stream);

/* FP8 form of the projections (the pages' block runs its linear layers in
 * FP8; deepmagic blog, section 實測數據).  Format: OCP MXFP8 - E4M3 codes
 * (1 byte each, OCP encoding: bias 7, largest finite 448) with one E8M0
 * scale byte (2^(s-127)) per 32 consecutive values along the contraction.
 * For a block with largest magnitude a: X = floor(log2 a) - 8 (X >= -127;
 * X = 0 for an all-zero block), codes = E4M3(v / 2^X) rounded to nearest
 * even and clamped to +-448, scale byte = X + 127.
 *
 * vdn_mxfp8_quantize: x bf16 [M, K] (K a multiple of 32) -> q [M, K] codes,
 * scales [M, K/32].  x, q 16-byte aligned.  Used for the weights once and by
 * the layer below for its activations. */
vdn_status_t vdn_mxfp8_quantize(const void* x, int64_t M, int32_t K, void* q, void* scales,
                                hipStream_t stream);

/* y[m][n] = sum_k X[m][k] W[n][k] with X, W given as MXFP8 codes + scales
 * ([M, K] + [M, K/32] and [N, K] + [N, K/32]); bf16 y [M, N], fp32
 * accumulation.  K a multiple of 128, N of 8 (else VDN_ERR_UNSUPPORTED);
 * codes 16-byte and scales 4-byte aligned. */
vdn_status_t vdn_out_proj_mxfp8(const void* xq, const void* xs, const void* wq, const void* ws,
                                int64_t M, int32_t K, int32_t N, void* y, hipStream_t stream);

/* vdn_softmax_branches_fwd with the two gated branches written as MXFP8
 * instead of bf16: quantized from the fp32 values inside the same kernel, in
 * the format above (blocks of 32 consecutive d of one head and branch).
 * codes: [B*T*P, 2*H*d] bytes, 16-byte aligned (per token the softmax branch
 * of every head, then the linear branch, as x2); scales: [B*T*P, 2*H*d/32]
 * bytes.  Same inputs, workspace and support (d in {32, 64, 128}, P and L
 * multiples of 8) as vdn_softmax_branches_fwd, else VDN_ERR_UNSUPPORTED.
 * The activation operand of vdn_out_proj_mxfp8.
 * [PaperDaily §三, figure 3; deepmagic blog, section 實測數據] */
vdn_status_t vdn_softmax_branches_mxfp8_fwd(const void* q, const void* k, const void* v,
                                            const void* text_k, const void* text_v,
                                            const float* R, const float* gate_logits,
                                            const vdn_layout_t* layout, void* codes,
                                            void* scales, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace vdn_hybrid_attn_proj_mxfp8_fwd needs (0 if invalid). */
size_t vdn_hybrid_attn_proj_mxfp8_workspace_size(const vdn_layout_t* layout);

/* vdn_hybrid_attn_proj_fwd with FP8 projections: the softmax kernel writes
 * the gated branches as MXFP8 (vdn_softmax_branches_mxfp8_fwd), which are
 * multiplied with pre-quantized w_o (codes w_q [d_model, 2*H*d], scales
 * w_scales [d_model, 2*H*d/32], e.g. from vdn_mxfp8_quantize).  2*H*d must
 * be a multiple of 128; d_model of 8. */
vdn_status_t vdn_hybrid_attn_proj_mxfp8_fwd(const void* q, const void* k, const void* v,
                                            const void* text_k, const void* text_v,
                                            const float* beta, const float* alpha,
                                            const float* gate_logits, const void* w_q,
                                            const void* w_scales, int32_t d_model,
                                            const vdn_layout_t* layout, void* y,
                                            void* workspace, size_t workspace_bytes,
                                            hipStream_t stream);

/* Bytes of workspace vdn_hybrid_attn_proj_fwd needs (0 if the layout is
 * invalid): the vdn_hybrid_attn_fwd workspace plus x2.  Host only. */
size_t vdn_hybrid_attn_proj_workspace_size(const vdn_layout_t* layout);

/* The layer with its separate output projections:
 *   y = [sigmoid(g0) O_soft ; sigmoid(g1) RMSNorm(R q)] . w_o^T
 * per video token, i.e. vdn_hybrid_attn_fwd's stages with the branches kept
 * apart (vdn_softmax_branches_fwd) followed by vdn_out_proj.  w_o: bf16
 * [d_model, 2*H*d] (softmax-branch columns first); y: bf16 [B, T*P, d_model].
 * Covers bf16 layouts with d in {32, 64, 128}, P and L multiples of 8, and
 * d_model a multiple of 8; else VDN_ERR_UNSUPPORTED.  workspace: at least
 * vdn_hybrid_attn_proj_workspace_size(layout) bytes, 256-byte aligned.
 * [PaperDaily §三, figure 3; arXiv abstract] */
vdn_status_t vdn_hybrid_attn_proj_fwd(const void* q, const void* k, const void* v,
                                      const void* text_k, const void* text_v,
                                      const float* beta, const float* alpha,
                                      const float* gate_logits, const void* w_o,
                                      int32_t d_model, const vdn_layout_t* layout, void* y,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* ---- Backward pass ---- */

/* Bytes of workspace vdn_hybrid_attn_bwd needs (0 if the layout is invalid).
 * Host only. */
size_t vdn_hybrid_attn_bwd_workspace_size(const vdn_layout_t* layout);

/* Gradients of the layer (the vector-Jacobian product with dO, the gradient
 * of the loss with respect to O): with the same inputs as
 * vdn_hybrid_attn_fwd and dO [B, T*P, H, d] (layout->dtype), writes
 *   dq, dk, dv        [B, T*P, H, d]   float32
 *   dtext_k, dtext_v  [B, L, H, d]     float32 (may be NULL when L == 0)
 *   dbeta             [B, T*P + L, H]  float32 (zero for tokens of frames no
 *                                      state folds)
 *   dalpha            [B, T, H]        float32 (zero for frames no state folds)
 *   dgate_logits      [B, T*P, H, 2]   float32
 * The forward is recomputed inside (the VDA statistics, factor and scan,
 * keeping every scan state, and the softmax with the merge backward in its
 * epilogue); nothing from a previous forward call is needed.  Covers bf16
 * layouts with d in {32, 64, 128} and P, L multiples of 8; else
 * VDN_ERR_UNSUPPORTED.  workspace: at least
 * vdn_hybrid_attn_bwd_workspace_size(layout) bytes, 256-byte aligned.
 * Outputs must not alias inputs or each other.  The gradient of the softmax
 * branch is the standard attention backward over each query's visible keys;
 * that of the linear branch runs the scan in reverse (PaperDaily §三/§四 and
 * the deepmagic closed form define the forward it differentiates). */
vdn_status_t vdn_hybrid_attn_bwd(const void* q, const void* k, const void* v,
                                 const void* text_k, const void* text_v,
                                 const float* beta, const float* alpha,
                                 const float* gate_logits, const void* dO,
                                 const vdn_layout_t* layout, float* dq, float* dk,
                                 float* dv, float* dtext_k, float* dtext_v, float* dbeta,
                                 float* dalpha, float* dgate_logits, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* ---- Training pair: forward that keeps its residuals, backward from them ---- */

/* Bytes of the saved-residual buffer of vdn_hybrid_attn_fwd_train /
 * vdn_hybrid_attn_bwd_saved (0 if the layout is invalid).  It holds the
 * backward's workspace plus O_soft and RMSNorm(R q) in float32 and one float
 * per token-head: about 8 d bytes per token-head more than
 * vdn_hybrid_attn_bwd_workspace_size.  Host only. */
size_t vdn_hybrid_attn_train_saved_size(const vdn_layout_t* layout);

/* vdn_hybrid_attn_fwd that also leaves in `saved` what the backward needs
 * (the VDA statistics, factor, read slots and every scan state; the softmax
 * branch output, the RMS-normalised linear read and the RMS factor; the
 * softmax's log-sum-exp), so that vdn_hybrid_attn_bwd_saved skips the
 * recomputation.  o is the layer output with the softmax scores formed
 * exactly in float32 (the backward recomputes its weights from q and k as
 * given); vdn_hybrid_attn_fwd forms them from q scaled and rounded to bf16,
 * so the two outputs agree to rounding (about 1e-4 relative on unit keys),
 * not bit for bit.  Covers the layouts vdn_hybrid_attn_bwd covers; else
 * VDN_ERR_UNSUPPORTED.  saved: device memory owned by the caller, at least
 * vdn_hybrid_attn_train_saved_size(layout) bytes, 256-byte aligned; it must
 * stay untouched until the matching vdn_hybrid_attn_bwd_saved call.
 * [PaperDaily §三, figure 3; deepmagic blog, 用兩條分支取代一條] */
vdn_status_t vdn_hybrid_attn_fwd_train(const void* q, const void* k, const void* v,
                                       const void* text_k, const void* text_v,
                                       const float* beta, const float* alpha,
                                       const float* gate_logits, const vdn_layout_t* layout,
                                       void* o, void* saved, size_t saved_bytes,
                                       hipStream_t stream);

/* vdn_hybrid_attn_bwd from the residuals a vdn_hybrid_attn_fwd_train call left
 * in `saved`, with the same inputs (q, k, v, text, beta, alpha, gate logits
 * unchanged since that call) and the same outputs and coverage.  The merge
 * backward runs as an elementwise pass over the saved branch outputs instead
 * of a second softmax forward.  The call consumes `saved` (the statistics
 * are overwritten by their gradients): one backward per training forward.
 * Outputs must not alias inputs, `saved` or each other. */
vdn_status_t vdn_hybrid_attn_bwd_saved(const void* q, const void* k, const void* v,
                                       const void* text_k, const void* text_v,
                                       const float* beta, const float* alpha,
                                       const float* gate_logits, const void* dO,
                                       const vdn_layout_t* layout, float* dq, float* dk,
                                       float* dv, float* dtext_k, float* dtext_v,
                                       float* dbeta, float* dalpha, float* dgate_logits,
                                       void* saved, size_t saved_bytes, hipStream_t stream);

/* Frame statistics: for every frame f < T and for the text block (slot T),
 * A[b,h,slot] = sum_i beta_i k_i k_i^T and B[b,h,slot] = sum_i beta_i v_i k_i^T
 * over the slot's tokens.  A_out, B_out: float32 [B, H, T+1, d, d] (row index
 * first).  The text slot is zero when L == 0.
 * [deepmagic blog, 用兩條分支取代一條; PaperDaily §四] */
vdn_status_t vdn_vda_gram(const void* k, const void* v, const void* text_k,
                          const void* text_v, const float* beta,
                          const vdn_layout_t* layout, float* A_out, float* B_out,
                          hipStream_t stream);

/* Bytes of workspace vdn_vda_factor_scan needs (0 if invalid).  Host only. */
size_t vdn_vda_factor_scan_workspace_size(const vdn_layout_t* layout);

/* Factor and scan: A_io holds the frame Grams from vdn_vda_gram and is
 * overwritten with (I + A)^-1 for the frames the scan uses (a symmetric
 * sweep: in-place Gauss-Jordan on the SPD matrix) and for the text slot.  B is read only.
 * R_out: float32 [B, H, nc+1, d, d] with nc = vdn_num_chunks(layout);
 * R_out[c] = S_fwd(c) + S_bwd(c), the summed states a non-anchor query frame of
 * chunk c reads, and R_out[nc] = S_x, the full text write (what anchor frames
 * read).  Both states start at S_x / 2 and skip anchor frames.
 * [deepmagic blog, 用兩條分支取代一條; PaperDaily §三, §四] */
vdn_status_t vdn_vda_factor_scan(float* A_io, const float* B, const float* alpha,
                                 const vdn_layout_t* layout, float* R_out,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* The layer's first stage, the whole VDA branch as the layer runs it, up to
 * the summed states: for bf16 layouts with d >= 32 one pass computes every
 * frame's statistics and factor (A stays on chip; G = (I + A)^-1 is kept as
 * bf16 hi and lo planes), then the bidirectional scan and the sum of the two
 * states; other layouts run vdn_vda_gram's and vdn_vda_factor_scan's
 * kernels.  R_out: float32 [B, H, nc+1, d, d], as vdn_vda_factor_scan's.
 * vt_out (may be NULL; only for the layouts vdn_softmax_merge_fwd covers):
 * the V^T copy the layer's softmax reads, bf16 [B, H, d, T*P + L] (row d of
 * head h: value d of every video token, then of every text token), written
 * by the same pass.  Inputs as vdn_hybrid_attn_fwd's; workspace as
 * vdn_hybrid_attn_fwd's (vdn_hybrid_attn_workspace_size bytes, caller-owned,
 * contents undefined afterwards).  Outputs must not alias the workspace.
 * [deepmagic blog, 用兩條分支取代一條; PaperDaily §三, §四] */
vdn_status_t vdn_vda_branch(const void* k, const void* v, const void* text_k,
                            const void* text_v, const float* beta, const float* alpha,
                            const vdn_layout_t* layout, float* R_out, void* vt_out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The layer's second stage: vdn_softmax_merge_fwd with V given as the V^T
 * copy vdn_vda_branch wrote (vt, bf16 [B, H, d, T*P + L]) instead of v and
 * text_v; one kernel, no workspace.  vdn_vda_branch followed by this call is
 * vdn_hybrid_attn_fwd, bit for bit.  [PaperDaily §二, §三] */
vdn_status_t vdn_softmax_merge_fwd_vt(const void* q, const void* k, const void* text_k,
                                      const void* vt, const float* R,
                                      const float* gate_logits, const vdn_layout_t* layout,
                                      void* o, hipStream_t stream);

/* Read + RMSNorm + gates + merge: o = sigmoid(g0) * o_soft
 *   + sigmoid(g1) * RMSNorm(R[c] q), with R from vdn_vda_factor_scan
 * (slot nc for anchor frames).  o may equal o_soft (in place); otherwise no
 * aliasing.  [PaperDaily §三] */
vdn_status_t vdn_merge(const void* q, const void* o_soft, const float* R,
                       const float* gate_logits, const vdn_layout_t* layout,
                       void* o, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VDN_H */
