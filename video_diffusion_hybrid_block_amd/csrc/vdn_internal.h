// Internal definitions shared by the host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vdn.h"

namespace vdn {

// ---------------------------------------------------------------------------
// Frame geometry [PaperDaily "伯克利与Impossible视频生成" §二, §三].
// Chunk c holds frames [c*C, min((c+1)*C, T)).  The window of chunk c is the
// frame interval [win_lo(c), win_hi(c)] covering chunks c-w .. c+w.  Anchors
// are frame 0 and frame T-1 (each optional).  A non-anchor query frame of
// chunk c sees win ∪ anchors in softmax; its forward state folds the
// non-anchor frames below win_lo(c) in ascending order, its backward state
// the non-anchor frames above win_hi(c) in descending order.  Anchor query
// frames see every frame and read the text write only.
// ---------------------------------------------------------------------------
struct Geo {
  int T, P, C, w, af, al, L, nc;
};

__host__ __device__ inline Geo make_geo(const vdn_layout_t& l) {
  Geo g;
  g.T = l.frames; g.P = l.tokens_per_frame; g.C = l.chunk_frames; g.w = l.window_chunks;
  g.af = l.anchor_first ? 1 : 0; g.al = l.anchor_last ? 1 : 0; g.L = l.text_tokens;
  g.nc = (g.T + g.C - 1) / g.C;
  return g;
}

__host__ __device__ inline int imax(int a, int b) { return a > b ? a : b; }
__host__ __device__ inline int imin(int a, int b) { return a < b ? a : b; }

__host__ __device__ inline int win_lo(const Geo& g, int c) {
  long v = (long)(c - g.w) * g.C;
  return v < 0 ? 0 : (int)v;
}
__host__ __device__ inline int win_hi(const Geo& g, int c) {
  long v = (long)(c + g.w + 1) * g.C;
  return (v > g.T ? g.T : (int)v) - 1;
}
__host__ __device__ inline bool is_anchor(const Geo& g, int t) {
  return (g.af && t == 0) || (g.al && t == g.T - 1);
}

// Video key segments (token ranges, merged where adjacent) visible to query
// frame t.  Returns the number of segments (1..3); seg_start/seg_len in tokens.
__host__ __device__ inline int key_segments(const Geo& g, int t, int seg_start[3], int seg_len[3]) {
  if (is_anchor(g, t)) {
    seg_start[0] = 0; seg_len[0] = g.T * g.P;
    return 1;
  }
  int c = t / g.C;
  int lo = win_lo(g, c), hi = win_hi(g, c);
  int n = 0;
  // frame 0 anchor, merged into the window when adjacent
  if (g.af && lo > 0) {
    if (lo == 1) lo = 0;
    else { seg_start[n] = 0; seg_len[n] = g.P; ++n; }
  }
  bool tail = false;
  if (g.al && hi < g.T - 1) {
    if (hi == g.T - 2) hi = g.T - 1;
    else tail = true;
  }
  seg_start[n] = lo * g.P; seg_len[n] = (hi - lo + 1) * g.P; ++n;
  if (tail) { seg_start[n] = (g.T - 1) * g.P; seg_len[n] = g.P; ++n; }
  return n;
}

// True when chunk c holds at least one non-anchor frame (a frame that reads
// the linear states).  Only the first and last chunk can fail this.
__host__ __device__ inline bool chunk_has_query(const Geo& g, int c) {
  int first = c * g.C, last = imin(g.T, (c + 1) * g.C) - 1;
  int n = last - first + 1;
  int na = (g.af && first == 0) ? 1 : 0;
  if (g.al && last == g.T - 1 && !(g.af && g.T - 1 == 0)) ++na;
  return n > na;
}

// Frames the scans fold: forward uses non-anchor frames below the window
// start of the last chunk that has query frames; backward uses non-anchor
// frames above the window end of the first such chunk (both exclusive bounds).
__host__ __device__ inline int fwd_scan_end(const Geo& g) {
  for (int c = g.nc - 1; c >= 0; --c)
    if (chunk_has_query(g, c)) return win_lo(g, c);
  return 0;
}
__host__ __device__ inline int bwd_scan_begin(const Geo& g) {
  for (int c = 0; c < g.nc; ++c)
    if (chunk_has_query(g, c)) return win_hi(g, c);
  return g.T - 1;
}

__host__ __device__ inline bool frame_needs_stats(const Geo& g, int f) {
  if (is_anchor(g, f)) return false;
  return f < fwd_scan_end(g) || f > bwd_scan_begin(g);
}

// Anchor frames below m / above m (the anchor set {0, T-1} without repeats).
__host__ __device__ inline int anchors_below(const Geo& g, int m) {
  int n = (g.af && 0 < m) ? 1 : 0;
  if (g.al && g.T - 1 < m && !(g.af && g.T == 1)) ++n;
  return n;
}
__host__ __device__ inline int anchors_above(const Geo& g, int m) {
  int n = (g.al && g.T - 1 > m) ? 1 : 0;
  if (g.af && 0 > m && !(g.al && g.T == 1)) ++n;
  return n;
}
// Position j (1-based) of frame f in the fold order of direction dir (0:
// forward, ascending; 1: backward, descending), 0 when that state does not
// fold f.
__host__ __device__ inline int fold_index(const Geo& g, int dir, int f) {
  if (is_anchor(g, f)) return 0;
  if (dir == 0) return f < fwd_scan_end(g) ? f + 1 - anchors_below(g, f + 1) : 0;
  return f > bwd_scan_begin(g) ? g.T - f - anchors_above(g, f - 1) : 0;
}
// Index j of the state chunk c's snapshot holds in direction dir: the number
// of steps before it (non-anchor frames below min(win_lo, fend), resp. above
// max(win_hi, fbeg)).
__host__ __device__ inline int snap_index(const Geo& g, int dir, int c) {
  if (dir == 0) {
    const int m = imin(win_lo(g, c), fwd_scan_end(g));
    return m - anchors_below(g, m);
  }
  const int m = imax(win_hi(g, c), bwd_scan_begin(g));
  return (g.T - 1 - m) - anchors_above(g, m);
}

// Statistics slots of one (batch, head): frames the scans fold (or every
// frame when `all_frames`), then the text block as slot T.  slot_of maps the
// dense index 0..count_slots-1 to the slot.
__host__ __device__ inline int slot_of(const Geo& g, int idx, bool all_frames) {
  if (all_frames) return idx;
  int lo_end = fwd_scan_end(g);
  int hi_begin = bwd_scan_begin(g);
  int f0 = g.af ? 1 : 0;                     // first non-anchor frame
  int f1 = g.al ? g.T - 2 : g.T - 1;         // last non-anchor frame
  int a = imin(lo_end, f1 + 1);
  int n_lo = imax(0, a - f0);
  if (idx < n_lo) return f0 + idx;
  idx -= n_lo;
  int start_hi = imax(hi_begin + 1, imax(f0, a));
  int n_hi = imax(0, f1 + 1 - start_hi);
  if (idx < n_hi) return start_hi + idx;
  return g.T;
}

__host__ __device__ inline int count_slots(const Geo& g, bool all_frames) {
  if (all_frames) return g.T + 1;
  int n = 0;
  for (int f = 0; f < g.T; ++f) n += frame_needs_stats(g, f) ? 1 : 0;
  return n + 1;
}

// Workspace plan (bytes, each region 256-byte aligned).
struct Plan {
  size_t a_off, b_off, sf_off, sb_off, r_off, vt_off, total;
};

__host__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The bf16 MFMA softmax reads V from a transposed copy (V^T, video then text
// tokens per row) when every 8-key chunk of its key sequence lies inside one
// segment, i.e. when P and L are multiples of 8.
__host__ __device__ inline bool softmax_uses_vt(const vdn_layout_t& l) {
  return l.dtype == VDN_BF16 && l.head_dim_k >= 32 && l.tokens_per_frame % 8 == 0 &&
         l.text_tokens % 8 == 0;
}
__host__ inline size_t softmax_ws_bytes(const vdn_layout_t& l) {
  if (!softmax_uses_vt(l)) return 0;
  size_t nl8 = ((size_t)l.frames * l.tokens_per_frame + l.text_tokens + 7) / 8 * 8;
  return align256((size_t)l.batch * l.heads * l.head_dim_k * nl8 * 2);
}

__host__ inline Plan make_plan(const vdn_layout_t& l) {
  Geo g = make_geo(l);
  size_t d = (size_t)l.head_dim_k;
  size_t bh = (size_t)l.batch * l.heads;
  size_t mat = d * d * sizeof(float);
  size_t stats = bh * (size_t)(g.T + 1) * mat;
  size_t snaps = bh * (size_t)(g.nc + 1) * mat;
  Plan p;
  p.a_off = 0;
  p.b_off = align256(p.a_off + stats);
  p.sf_off = align256(p.b_off + stats);
  p.sb_off = align256(p.sf_off + snaps);
  p.r_off = align256(p.sb_off + snaps);
  p.vt_off = align256(p.r_off + snaps);
  p.total = align256(p.vt_off + softmax_ws_bytes(l));
  return p;
}

__host__ inline size_t scan_ws_bytes(const vdn_layout_t& l) {
  Geo g = make_geo(l);
  size_t d = (size_t)l.head_dim_k;
  size_t snaps = (size_t)l.batch * l.heads * (size_t)(g.nc + 1) * d * d * sizeof(float);
  return 2 * align256(snaps);
}

// ---------------------------------------------------------------------------
// Kernel launchers (one translation unit each).  All return hipError_t of the
// launch.  Pointers are device pointers; shapes were validated by the caller.
// ---------------------------------------------------------------------------
hipError_t launch_softmax(const void* q, const void* k, const void* v, const void* tk,
                          const void* tv, const vdn_layout_t& l, float scale, void* o, void* ws,
                          hipStream_t s);
hipError_t launch_gram(const void* k, const void* v, const void* tk, const void* tv,
                       const float* beta, const vdn_layout_t& l, bool all_frames, float* A,
                       float* B, hipStream_t s);
hipError_t launch_factor(float* A, const vdn_layout_t& l, bool all_frames, hipStream_t s);
// Layer forward path (bf16, d >= 32): statistics and factor in one pass.
// Gp [B*H][T+1][2][d][d] bf16 receives G = (I + A)^-1 of every slot the scans
// fold (and the text block) as hi and lo planes, B [B*H][T+1][d][d] fp32 the
// writes; with vt non-null (only when softmax_uses_vt) the same pass writes
// the softmax's V^T copy [B][H][d][nl8] (every frame, then the text).
hipError_t launch_vda_stats(const void* k, const void* v, const void* tk, const void* tv,
                            const float* beta, const vdn_layout_t& l, void* Gp, float* B,
                            void* vt, hipStream_t s);
// The bidirectional scan and R = S_f + S_b from those planes (bf16, d >= 32).
hipError_t launch_scan_split(const void* Gp, const float* B, const float* alpha,
                             const vdn_layout_t& l, float* Sf, float* Sb, float* R, hipStream_t s);
// states (backward pass, bf16 MFMA path only; may be null): every chain's
// state after each of its steps, [B*H][2][T+1][d][d] fp32, step 0 = start.
hipError_t launch_scan(const float* G, const float* B, const float* alpha, const vdn_layout_t& l,
                       float* Sf, float* Sb, float* R, hipStream_t s, float* states = nullptr);
// Backward pass of the scan: dspost [B*H][2][T+1][d][d] gets, per chain, the
// gradient of its state after every step j (j = 0: the start), from dR
// [B*H][nc+1][d][d] (the gradients of the read slots).  bf16, d >= 32.
hipError_t launch_scan_bwd(const float* G, const float* dR, const float* alpha,
                           const vdn_layout_t& l, float* dspost, hipStream_t s);
hipError_t launch_merge(const void* q, const void* o_soft, const float* R, const float* gates,
                        const vdn_layout_t& l, float eps, void* o, hipStream_t s);
// Softmax branch with the merge fused into its epilogue (bf16, V^T path only):
// o = sigmoid(g0) softmax + sigmoid(g1) RMSNorm(R q), or with `split` the two
// gated branches side by side, o [B][N][2][H][d] (softmax branch first).
bool softmax_merge_fusable(const vdn_layout_t& l);
// fp32 layouts, d >= 32: the softmax on fp32 MFMA with the merge in its
// epilogue, o [B][N][H][d] fp32.
bool softmax_merge_f32_fusable(const vdn_layout_t& l);
hipError_t launch_softmax_merge_f32(const void* q, const void* k, const void* v, const void* tk,
                                    const void* tv, const float* R, const float* gates,
                                    const vdn_layout_t& l, float scale, float eps, void* o,
                                    hipStream_t s);
// vt_ready: ws already holds the V^T copy (written by launch_vda_stats).
hipError_t launch_softmax_merge(const void* q, const void* k, const void* v, const void* tk,
                                const void* tv, const float* R, const float* gates,
                                const vdn_layout_t& l, float scale, float eps, bool split, void* o,
                                void* ws, hipStream_t s, bool vt_ready = false);
// Extra operands of the softmax kernel's epilogue.
// Merge backward (backward pass): for every video token-head, dgates
// [B,N,H,2] fp32, dos = sigmoid(l0) dO [B,N,H,d] bf16, dlin = gradient of the
// linear read before RMSNorm [B,N,H,d] fp32, and per (b, h, token) the
// softmax's log-sum-exp in exp2 units, negated (nlse = -lse), and -D with
// D = dos . O_soft (dvec), [B,H,N] fp32: the backward's score and dP
// products start their accumulators from them.
// MXFP8 branches: mx_scales [B*N][2*H*d/32] receives the E8M0 block scales
// (the E4M3 codes go to the kernel's output pointer, [B*N][2*H*d] bytes).
// Training forward: o_soft = O_soft and o_lin = RMSNorm(R q), [B,N,H,d] fp32,
// and per (b, h, token) nlse (as above) and rinv = 1 / r, [B,H,N] fp32.
struct EpilogueIO {
  const __bf16* dO;
  float* dgates;
  __bf16* dos;
  float* dlin;
  float* dvec;
  float* nlse;
  uint8_t* mx_scales;
  float* o_soft;
  float* o_lin;
  float* rinv;
};
// Training forward: the merged output of launch_softmax_merge plus the
// residuals named under EpilogueIO (o_soft, o_lin, nlse, rinv).
hipError_t launch_softmax_merge_train(const void* q, const void* k, const void* v,
                                      const void* tk, const void* tv, const float* R,
                                      const float* gates, const vdn_layout_t& l, float scale,
                                      float eps, void* o, const EpilogueIO& io, void* ws,
                                      hipStream_t s);
// Merge backward from the training forward's residuals (bf16 dO, d = 32, 64
// or 128): dgates, dos, dlin and dvec as the backward softmax epilogue
// writes them, from o_soft, o_lin and rinv instead of a recomputation.
hipError_t launch_merge_bwd_saved(const void* dO, const float* gates, const float* o_soft,
                                  const float* o_lin, const float* rinv, const vdn_layout_t& l,
                                  float* dgates, void* dos, float* dlin, float* dvec,
                                  hipStream_t s);
// The two gated branches as MXFP8 (E4M3 codes, one E8M0 scale per 32
// consecutive d of one head and branch), quantized in the epilogue from the
// fp32 values: codes [B*N][2*H*d] bytes (softmax branch first, as x2),
// scales [B*N][2*H*d/32].  The activation operand of the FP8 projection.
hipError_t launch_softmax_branches_mxfp8(const void* q, const void* k, const void* v,
                                         const void* tk, const void* tv, const float* R,
                                         const float* gates, const vdn_layout_t& l, float scale,
                                         float eps, void* codes, void* scales, void* ws,
                                         hipStream_t s, bool vt_ready = false);
hipError_t launch_softmax_merge_bwd(const void* q, const void* k, const void* v, const void* tk,
                                    const void* tv, const float* R, const float* gates,
                                    const vdn_layout_t& l, float scale, float eps,
                                    const EpilogueIO& bio, void* ws, hipStream_t s);
// Transposed copy xt[b][h][d][n] of x [B,N,H,D] followed by tx [B,L,H,D]
// (tokens along the row, zero-padded to a multiple of 8), bf16.
hipError_t launch_transpose(const void* x, const void* tx, int B, int H, int D, int N, int L,
                            void* xt, hipStream_t s);
// Softmax backward (bf16, d in {32, 64, 128}, P and L multiples of 8):
// dq += scale * sum_j dS_ij k_j (dq fp32, already holding the linear read's
// part), dk/dv and dtk/dtv (text keys) added (fp32, holding the statistics'
// part from gram_bwd), from dos,
// the row statistics nlse/dvec, and transposed copies kt (keys + text), qt and
// dost (video tokens).
hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* tk,
                           const void* tv, const void* dos, const float* nlse, const float* dvec,
                           const void* kt, const void* qt, const void* dost,
                           const vdn_layout_t& l, float scale, float* dq, float* dk, float* dv,
                           float* dtk, float* dtv, hipStream_t s);
// VDA backward: dR / dq (written; dRp holds per-chunk partials of dR,
// vda_bwd_partial_bytes), reverse scan, per-frame dA (over G), dB (over B),
// dalpha; then gram_bwd writes dk, dv, dtk, dtv (zero for tokens of frames no
// chain folds) and dbeta, before the softmax backward adds its part.
size_t vda_bwd_partial_bytes(const vdn_layout_t& l);
hipError_t launch_vda_bwd(const void* q, const void* k, const void* v, const void* tk,
                          const void* tv, const float* beta, const float* alpha,
                          const float* dlin, const float* R, float* GA, float* BB,
                          const float* states, float* dRp, float* dR, float* dspost, float* dq,
                          float* dalpha, const vdn_layout_t& l, hipStream_t s);
hipError_t launch_gram_bwd(const void* k, const void* v, const void* tk, const void* tv,
                           const float* beta, const float* dA, const float* dB, float* dk,
                           float* dv, float* dtk, float* dtv, float* dbeta, const vdn_layout_t& l,
                           hipStream_t s);
// Output projections: y[m][n] = sum_k x[m][k] w[n][k] (bf16 in and out, fp32
// accumulation); needs K a positive multiple of 64 and N a multiple of 8.
bool proj_shape_ok(long M, int K, int N);
hipError_t launch_proj(const void* x, const void* w, long M, int K, int N, void* y, hipStream_t s);
// MXFP8 (E4M3 codes + one E8M0 scale per 32 values along K): quantization of
// a bf16 [M][K] matrix (K a multiple of 32) and the product from quantized
// operands (K a multiple of 128, N of 8).
bool mx_quant_shape_ok(long M, int K);
hipError_t launch_mx_quant(const void* x, long M, int K, void* q, void* scales, hipStream_t s);
bool proj_mxfp8_shape_ok(long M, int K, int N);
hipError_t launch_proj_mxfp8(const void* xq, const void* xs, const void* wq, const void* ws,
                             long M, int K, int N, void* y, hipStream_t s);

}  // namespace vdn
