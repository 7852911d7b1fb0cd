// Backward pass of the linear (VDA) branch, after the merge backward:
//
//  1. read slots (dr_mfma_kernel + dr_sum_kernel): each video token reads
//     o = R_c q with R_c its chunk's summed state (slot nc, the text write,
//     for anchor frames), so dR_c = sum_i do_i q_i^T over the slot's tokens
//     and q_i gets R_c^T do_i (written as the first part of dq);
//  2. the reverse scan (k_scan.hip) turns dR into dS_j, the gradient of each
//     chain's state after each step;
//  3. per frame (vda_frame_bwd_kernel): a step S_j = X_j G_j with
//     X_j = alpha_f S_{j-1} + B_f gives dX = dS_j G_j (G symmetric), so
//     dB_f += dX, dalpha_f += <dX, S_{j-1}>, dG_f += X_j^T dS_j, summed over
//     the chains that fold f; G = (I + A)^-1 gives dA_f = -G dG_f G.  The text
//     write S_x = B_x G_x starts both chains at S_x / 2, so
//     dS_x = (dS_0^fwd + dS_0^bwd) / 2, dB_x = dS_x G_x, dG_x = B_x^T dS_x;
//  4. per token (gram_bwd_mfma_kernel): A = sum beta k k^T, B = sum beta v k^T
//     give dk_i = beta_i ((dA + dA^T) k_i + dB^T v_i), dv_i = beta_i dB k_i
//     (written; the softmax backward adds its part afterwards) and
//     dbeta_i = k_i^T dA k_i + v_i^T dB k_i.
// [the forward: deepmagic blog "生成比播放還快", section 用兩條分支取代一條
//  (S = (S̄ + B)(I + A)^-1); PaperDaily "伯克利与Impossible视频生成" §三 (two
//  states from half the text write, summed read), §四 (frame statistics)]
//
// gfx950 design: the per-token products (steps 1 and 4) run on
// v_mfma_f32_32x32x16_bf16 with fp32 operands split into bf16 hi + lo (bf16
// inputs are exact), tiles staged in swizzled LDS and read row-wise
// (ds_read_b128) or column-wise (ds_read_b64_tr_b16) as each product needs;
// the per-frame d x d x d products (step 3, ~1 % of the backward) are fp32
// VALU.
#include "vdn_device.h"
#include "vdn_internal.h"

namespace vdn {

namespace {

// ---------------------------------------------------------------------------
// 1. dR and the linear part of dq.  Workgroup = (batch, head, slot, chunk of
// DR_CH of the slot's tokens); partial dR per chunk, summed by dr_sum_kernel.
// ---------------------------------------------------------------------------
constexpr int DR_CH = 1024;              // tokens per workgroup
constexpr int DR_TT = 64;                // tokens per LDS tile

// Video tokens of read slot `slot`: a chunk's non-anchor frames, which are
// contiguous since only the first and the last frame can be anchors, or for
// slot nc the anchor frames (at most two).  The slot's i-th token is
// base0 + i below `split` and base1 + i from there on; n tokens in all.
struct SlotMap {
  int n, split, base0, base1;
};
__device__ __forceinline__ SlotMap slot_map(const Geo& g, int slot) {
  SlotMap m;
  if (slot < g.nc) {
    int f0 = slot * g.C, f1 = imin(g.T, f0 + g.C);
    if (is_anchor(g, f0)) ++f0;
    if (f1 > f0 && is_anchor(g, f1 - 1)) --f1;
    m.n = imax(0, f1 - f0) * g.P;
    m.split = m.n;
    m.base0 = f0 * g.P;
    m.base1 = 0;
  } else {
    const bool first = g.af, last = g.al && !(g.af && g.T == 1);
    m.n = ((first ? 1 : 0) + (last ? 1 : 0)) * g.P;
    m.split = first ? g.P : 0;
    m.base0 = 0;
    m.base1 = (g.T - 1) * g.P - m.split;
  }
  return m;
}
__device__ __forceinline__ int slot_tok(const SlotMap& m, int i) {
  return i < m.split ? m.base0 + i : m.base1 + i;
}

// Threads of a dR workgroup: its LDS (R hi + lo, three token tiles) allows
// one workgroup per CU at d = 128, so eight waves there (two per SIMD).
constexpr int dr_threads(int d) { return d == 128 ? 512 : 256; }

template <int D>
__global__ void __launch_bounds__(dr_threads(D))
dr_mfma_kernel(const bf16* __restrict__ q, const float* __restrict__ dlin,
               const float* __restrict__ R, float* __restrict__ dRp, float* __restrict__ dq,
               Geo g, int H, int nch) {
  constexpr int MAT = D * D * 2;         // bf16 d x d tile, bytes
  constexpr int TB = DR_TT * D * 2;      // bf16 token tile, bytes
  constexpr int NBK = D / 32;
  constexpr int NT = dr_threads(D), NW = NT / 64;
  __shared__ __attribute__((aligned(16))) char rh[MAT];
  __shared__ __attribute__((aligned(16))) char rl[MAT];
  __shared__ __attribute__((aligned(16))) char qs[TB];
  __shared__ __attribute__((aligned(16))) char dh[TB];
  __shared__ __attribute__((aligned(16))) char dl[TB];
  char VDN_LDS* Rh = (char VDN_LDS*)rh;
  char VDN_LDS* Rl = (char VDN_LDS*)rl;
  char VDN_LDS* Qs = (char VDN_LDS*)qs;
  char VDN_LDS* Dh = (char VDN_LDS*)dh;
  char VDN_LDS* Dl = (char VDN_LDS*)dl;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, half = lane >> 5;
  const int ch = blockIdx.x % nch;
  const int slot = (blockIdx.x / nch) % (g.nc + 1);
  const int bh = blockIdx.x / nch / (g.nc + 1);
  const int b = bh / H, h = bh % H;
  const int N = g.T * g.P;
  const size_t mat = (size_t)D * D;
  const SlotMap sm = slot_map(g, slot);
  const int ntok = sm.n;
  const int i0 = ch * DR_CH;
  const int nmine = imax(0, imin(DR_CH, ntok - i0));
  float* part = dRp + (((size_t)bh * (g.nc + 1) + slot) * nch + ch) * mat;
  // R of the slot, hi + lo, row-major swizzled (read column-wise for dq)
  const float* Rs = R + ((size_t)bh * (g.nc + 1) + slot) * mat;
  for (int i = tid; i < D * D / 8; i += NT) {
    const int r = i / (D / 8), c = (i % (D / 8)) * 8;
    const f32x4 a = *(const f32x4*)(Rs + r * D + c);
    const f32x4 a2 = *(const f32x4*)(Rs + r * D + c + 4);
    const float xv[8] = {a[0], a[1], a[2], a[3], a2[0], a2[1], a2[2], a2[3]};
    bf16x8 hv, lv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16 hi, lo;
      split_bf16(xv[e], hi, lo);
      hv[e] = hi;
      lv[e] = lo;
    }
    *(bf16x8 VDN_LDS*)(Rh + swz_off<D>(r, c)) = hv;
    *(bf16x8 VDN_LDS*)(Rl + swz_off<D>(r, c)) = lv;
  }
  // this wave's dR blocks: (rb, cb) = wave-strided over the NBK x NBK grid
  constexpr int BPW = NBK * NBK >= NW ? NBK * NBK / NW : 1;
  f32x16 acc[BPW];
#pragma unroll
  for (int u = 0; u < BPW; ++u) acc[u] = f32x16{};
  for (int t0 = 0; t0 < nmine; t0 += DR_TT) {
    __syncthreads();                     // previous tile consumed (and R staged)
    for (int i = tid; i < DR_TT * D / 8; i += NT) {
      const int r = i / (D / 8), c = (i % (D / 8)) * 8;
      bf16x8 qv = {}, hv = {}, lv = {};
      if (t0 + r < nmine) {
        const int tok = slot_tok(sm, i0 + t0 + r);
        const size_t off = (((size_t)b * N + tok) * H + h) * D + c;
        qv = *(const bf16x8*)(q + off);
        const f32x4 a = *(const f32x4*)(dlin + off);
        const f32x4 a2 = *(const f32x4*)(dlin + off + 4);
        const float xv[8] = {a[0], a[1], a[2], a[3], a2[0], a2[1], a2[2], a2[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16 hi, lo;
          split_bf16(xv[e], hi, lo);
          hv[e] = hi;
          lv[e] = lo;
        }
      }
      *(bf16x8 VDN_LDS*)(Qs + swz_off<D>(r, c)) = qv;
      *(bf16x8 VDN_LDS*)(Dh + swz_off<D>(r, c)) = hv;
      *(bf16x8 VDN_LDS*)(Dl + swz_off<D>(r, c)) = lv;
    }
    __syncthreads();
    // dR[r][c] += sum_t dlin[t][r] q[t][c]: A = dlin^T, B = q (column reads)
#pragma unroll
    for (int u = 0; u < BPW; ++u) {
      const int blk = wv * BPW + u;
      if (blk >= NBK * NBK) break;       // d = 32: one block, wave 0
      const int rb = blk / NBK, cb = blk % NBK;
#pragma unroll
      for (int ks = 0; ks < DR_TT / 16; ++ks) {
        const bf16x8 ah = lds_col8<D>(Dh, ks * 16, rb * 32, lane);
        const bf16x8 al = lds_col8<D>(Dl, ks * 16, rb * 32, lane);
        const bf16x8 bq = lds_col8<D>(Qs, ks * 16, cb * 32, lane);
        acc[u] = mfma32(ah, bq, acc[u]);
        acc[u] = mfma32(al, bq, acc[u]);
      }
    }
    // dq[t][c] = sum_r dlin[t][r] R[r][c] over (token block, column block)
    // pairs, wave-strided; A = dlin rows, B = R columns
    {
      constexpr int NPAIR = (DR_TT / 32) * NBK;
#pragma unroll
      for (int pi = wv; pi < NPAIR; pi += NW) {
        const int tb = pi / NBK, cb = pi % NBK;
        f32x16 o = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 ah = lds_row8<D>(Dh, tb * 32 + (lane & 31), ks * 2 + half);
          const bf16x8 al = lds_row8<D>(Dl, tb * 32 + (lane & 31), ks * 2 + half);
          const bf16x8 bh_ = lds_col8<D>(Rh, ks * 16, cb * 32, lane);
          const bf16x8 bl_ = lds_col8<D>(Rl, ks * 16, cb * 32, lane);
          o = mfma32(ah, bh_, o);
          o = mfma32(ah, bl_, o);
          o = mfma32(al, bh_, o);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = tb * 32 + (j >> 2) * 8 + half * 4 + (j & 3);
          if (t0 + r < nmine) {
            const int tok = slot_tok(sm, i0 + t0 + r);
            dq[(((size_t)b * N + tok) * H + h) * D + cb * 32 + (lane & 31)] = o[j];
          }
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < BPW; ++u) {
    const int blk = wv * BPW + u;
    if (blk >= NBK * NBK) break;
    const int rb = blk / NBK, cb = blk % NBK;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = rb * 32 + (j >> 2) * 8 + half * 4 + (j & 3);
      part[(size_t)r * D + cb * 32 + (lane & 31)] = acc[u][j];
    }
  }
}

// dR[bh][slot] = sum of the chunks' partials.
__global__ void __launch_bounds__(256)
dr_sum_kernel(const float4* __restrict__ part, float4* __restrict__ dR, int nch, size_t mat4,
              size_t nslot) {
  const size_t n = nslot * mat4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t sl = i / mat4, e = i % mat4;
    const float4* p = part + sl * nch * mat4 + e;
    float4 a = p[0];
    for (int c = 1; c < nch; ++c) {
      const float4 x = p[(size_t)c * mat4];
      a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
    }
    dR[i] = a;
  }
}

// ---------------------------------------------------------------------------
// d x d x d products for the per-frame step: a 32 x 16 thread grid (512
// threads, two waves per SIMD on the one workgroup the LDS allows per CU),
// thread (ti, tj) owning a d/32 x d/16 block.  Rows come in groups of
// WR = min(4, d/32) consecutive rows, group hh at 32 WR hh + WR ti; columns
// in groups of W = min(4, d/16), group hh at 16 W hh + W tj.  Consecutive
// rows / columns let every LDS read be 4 W (4 WR) bytes wide; spreading the
// groups keeps the distinct ti (tj) of a wave on different banks.
// ---------------------------------------------------------------------------
constexpr int FR_NT = 512;

template <int D>
struct Tile {
  static constexpr int RR = D / 32;              // rows per thread
  static constexpr int RB = D / 16;              // columns per thread
  static constexpr int WR = RR < 4 ? RR : 4;     // consecutive rows per group
  static constexpr int W = RB < 4 ? RB : 4;      // consecutive columns per group
  static constexpr int NHR = RR / WR;            // row groups
  static constexpr int NH = RB / W;              // column groups
  static constexpr int LD = D + 4;               // padded LDS row (floats)
  static_assert(D % 32 == 0 && D >= 32 && D <= 128, "d = 32, 64 or 128");
};

template <int W>
using fvec = float __attribute__((ext_vector_type(W)));

// row x in [0, d/32) of thread row index ti in [0, 32)
template <int D>
__device__ __forceinline__ int blk_r(int ti, int x) {
  constexpr int WR = Tile<D>::WR;
  return (x / WR) * 32 * WR + ti * WR + x % WR;
}
// column c in [0, d/16) of thread column index tj in [0, 16)
template <int D>
__device__ __forceinline__ int blk_c(int tj, int c) {
  constexpr int W = Tile<D>::W;
  return (c / W) * 16 * W + tj * W + c % W;
}

// acc += op(A) * B, A and B in LDS ([D][LD]), op(A) = A or A^T.
template <int D, bool TA>
__device__ __forceinline__ void mm_acc(const float* A, const float* B, int ti, int tj,
                                       float (&acc)[D / 32][D / 16]) {
  constexpr int RR = Tile<D>::RR, RB = Tile<D>::RB, W = Tile<D>::W, WR = Tile<D>::WR;
  constexpr int NHR = Tile<D>::NHR, NH = Tile<D>::NH, LD = Tile<D>::LD;
#pragma unroll 2
  for (int k = 0; k < D; k += W) {
    float av[RR][W], bv[W][RB];          // av[row][kk], bv[kk][col]
    if constexpr (TA) {
#pragma unroll
      for (int kk = 0; kk < W; ++kk)
#pragma unroll
        for (int hh = 0; hh < NHR; ++hh) {
          const fvec<WR> x = *(const fvec<WR>*)(A + (k + kk) * LD + hh * 32 * WR + ti * WR);
#pragma unroll
          for (int q = 0; q < WR; ++q) av[hh * WR + q][kk] = x[q];
        }
    } else {
#pragma unroll
      for (int a = 0; a < RR; ++a) {
        const fvec<W> x = *(const fvec<W>*)(A + blk_r<D>(ti, a) * LD + k);
#pragma unroll
        for (int q = 0; q < W; ++q) av[a][q] = x[q];
      }
    }
#pragma unroll
    for (int kk = 0; kk < W; ++kk)
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const fvec<W> x = *(const fvec<W>*)(B + (k + kk) * LD + hh * 16 * W + tj * W);
#pragma unroll
        for (int q = 0; q < W; ++q) bv[kk][hh * W + q] = x[q];
      }
#pragma unroll
    for (int kk = 0; kk < W; ++kk)
#pragma unroll
      for (int a = 0; a < RR; ++a)
#pragma unroll
        for (int c = 0; c < RB; ++c) acc[a][c] = fmaf(av[a][kk], bv[kk][c], acc[a][c]);
  }
}

// dst (LDS, [D][LD]) = f(src0, src1) elementwise over [D][D] global inputs,
// W floats per access
template <int D, typename F>
__device__ __forceinline__ void stage_mat(float* dst, const float* s0, const float* s1, F f,
                                          int tid) {
  constexpr int W = Tile<D>::W, LD = Tile<D>::LD;
  for (int i = tid; i < D * D / W; i += FR_NT) {
    const fvec<W> x = *(const fvec<W>*)(s0 + i * W);
    const fvec<W> y = *(const fvec<W>*)(s1 + i * W);
    fvec<W> r;
#pragma unroll
    for (int q = 0; q < W; ++q) r[q] = f(x[q], y[q]);
    *(fvec<W>*)(dst + (i * W / D) * LD + (i * W) % D) = r;
  }
}

template <int D>
__device__ __forceinline__ void load_mat(float* dst, const float* src, int tid) {
  constexpr int W = Tile<D>::W, LD = Tile<D>::LD;
  for (int i = tid; i < D * D / W; i += FR_NT)
    *(fvec<W>*)(dst + (i * W / D) * LD + (i * W) % D) = *(const fvec<W>*)(src + i * W);
}

// ---------------------------------------------------------------------------
// 3. Per frame (and the text slot T): dA, dB in place of G, B; dalpha.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(FR_NT)
vda_frame_bwd_kernel(float* __restrict__ GA, float* __restrict__ BB,
                     const float* __restrict__ alpha, const float* __restrict__ states,
                     const float* __restrict__ dspost, float* __restrict__ dalpha, Geo g, int H) {
  constexpr int RR = Tile<D>::RR, RB = Tile<D>::RB, LD = Tile<D>::LD;
  __shared__ __attribute__((aligned(16))) float L1[D * LD];
  __shared__ __attribute__((aligned(16))) float L2[D * LD];
  __shared__ float red[FR_NT];
  const int tid = threadIdx.x;
  const int ti = tid >> 4, tj = tid & 15;
  const int slot = blockIdx.x % (g.T + 1);
  const int bh = blockIdx.x / (g.T + 1);
  const int b = bh / H, h = bh % H;
  const size_t mat = (size_t)D * D;
  float* Gs = GA + ((size_t)bh * (g.T + 1) + slot) * mat;
  float* Bs = BB + ((size_t)bh * (g.T + 1) + slot) * mat;
  const bool text = slot == g.T;
  const int j0 = text ? 0 : fold_index(g, 0, slot);
  const int j1 = text ? 0 : fold_index(g, 1, slot);
  const bool live = text ? g.L > 0 : (j0 > 0 || j1 > 0);
  if (!live) {
    // no chain reads this slot: zero gradients (its statistics were never
    // formed)
    for (int i = tid; i < D * D; i += FR_NT) {
      Gs[i] = 0.f;
      Bs[i] = 0.f;
    }
    if (!text && tid == 0) dalpha[((size_t)b * g.T + slot) * H + h] = 0.f;
    return;
  }
  float dB[RR][RB], dG[RR][RB];
#pragma unroll
  for (int a = 0; a < RR; ++a)
#pragma unroll
    for (int c = 0; c < RB; ++c) dB[a][c] = dG[a][c] = 0.f;
  float dal = 0.f;
  const float* post = dspost + (size_t)bh * 2 * (g.T + 1) * mat;
  const float* st = states + (size_t)bh * 2 * (g.T + 1) * mat;
  if (text) {
    // dS_x = (dS_0^fwd + dS_0^bwd) / 2; dB_x = dS_x G_x; dG_x = B_x^T dS_x
    const float* p0 = post;
    const float* p1 = post + (size_t)(g.T + 1) * mat;
    stage_mat<D>(L1, p0, p1, [](float x, float y) { return 0.5f * (x + y); }, tid);
    load_mat<D>(L2, Gs, tid);
    __syncthreads();
    mm_acc<D, false>(L1, L2, ti, tj, dB);
    __syncthreads();
    load_mat<D>(L2, Bs, tid);
    __syncthreads();
    mm_acc<D, true>(L2, L1, ti, tj, dG);
    __syncthreads();
  } else {
    const float a = alpha[((size_t)b * g.T + slot) * H + h];
    for (int dir = 0; dir < 2; ++dir) {
      const int j = dir == 0 ? j0 : j1;
      if (j == 0) continue;
      const float* dSj = post + ((size_t)dir * (g.T + 1) + j) * mat;
      const float* Sp = st + ((size_t)dir * (g.T + 1) + j - 1) * mat;
      load_mat<D>(L1, dSj, tid);
      load_mat<D>(L2, Gs, tid);
      __syncthreads();
      float dX[RR][RB];
#pragma unroll
      for (int x = 0; x < RR; ++x)
#pragma unroll
        for (int c = 0; c < RB; ++c) dX[x][c] = 0.f;
      mm_acc<D, false>(L1, L2, ti, tj, dX);
#pragma unroll
      for (int x = 0; x < RR; ++x)
#pragma unroll
        for (int c = 0; c < RB; ++c) {
          dB[x][c] += dX[x][c];
          dal = fmaf(dX[x][c], Sp[(size_t)blk_r<D>(ti, x) * D + blk_c<D>(tj, c)], dal);
        }
      __syncthreads();
      // X = alpha S_{j-1} + B_f
      stage_mat<D>(L2, Sp, Bs, [a](float x, float y) { return fmaf(a, x, y); }, tid);
      __syncthreads();
      mm_acc<D, true>(L2, L1, ti, tj, dG);
      __syncthreads();
    }
    red[tid] = dal;
    __syncthreads();
    for (int s = FR_NT / 2; s > 0; s >>= 1) {
      if (tid < s) red[tid] += red[tid + s];
      __syncthreads();
    }
    if (tid == 0) dalpha[((size_t)b * g.T + slot) * H + h] = red[0];
  }
  // dA = -G dG G
  load_mat<D>(L2, Gs, tid);
#pragma unroll
  for (int x = 0; x < RR; ++x)
#pragma unroll
    for (int c = 0; c < RB; ++c) L1[blk_r<D>(ti, x) * LD + blk_c<D>(tj, c)] = dG[x][c];
  __syncthreads();
  float t1[RR][RB];
#pragma unroll
  for (int x = 0; x < RR; ++x)
#pragma unroll
    for (int c = 0; c < RB; ++c) t1[x][c] = 0.f;
  mm_acc<D, false>(L2, L1, ti, tj, t1);     // G dG
  __syncthreads();
#pragma unroll
  for (int x = 0; x < RR; ++x)
#pragma unroll
    for (int c = 0; c < RB; ++c) L1[blk_r<D>(ti, x) * LD + blk_c<D>(tj, c)] = t1[x][c];
  __syncthreads();
  float t2[RR][RB];
#pragma unroll
  for (int x = 0; x < RR; ++x)
#pragma unroll
    for (int c = 0; c < RB; ++c) t2[x][c] = 0.f;
  mm_acc<D, false>(L1, L2, ti, tj, t2);     // (G dG) G
  __syncthreads();                          // every read of G_f / B_f done
#pragma unroll
  for (int x = 0; x < RR; ++x)
#pragma unroll
    for (int c = 0; c < RB; ++c) {
      const size_t e = (size_t)blk_r<D>(ti, x) * D + blk_c<D>(tj, c);
      Gs[e] = -t2[x][c];
      Bs[e] = dB[x][c];
    }
}

// ---------------------------------------------------------------------------
// 4. Per token of every frame (slot T: the text tokens): dk, dv, dbeta
// (written; zero for frames no chain folds; the softmax backward adds its
// dk, dv afterwards).  Workgroup = (batch, head, slot, chunk of GB_CH
// tokens: a whole frame up to 1024 tokens, so the staging of As and dB below
// serves as many tokens as possible), GB_NT / 64 waves x 32 tokens at a
// time.  With As = dA + dA^T:
// U = K As^T, W = K dB^T, Z = V dB (tokens x d each) on MFMA, As and dB as
// bf16 hi + lo in swizzled LDS (As and dB rows for U and W, dB columns for
// Z); dk = beta (U + Z), dv = beta W, dbeta = sum_r (k_r U_r / 2 + v_r W_r).
// ---------------------------------------------------------------------------
constexpr int GB_CH = 1024;
constexpr int GB_NT = 512;

template <int D>
__global__ void __launch_bounds__(GB_NT)
gram_bwd_mfma_kernel(const bf16* __restrict__ k, const bf16* __restrict__ v,
                     const bf16* __restrict__ tk, const bf16* __restrict__ tv,
                     const float* __restrict__ beta, const float* __restrict__ dA,
                     const float* __restrict__ dB, float* __restrict__ dk,
                     float* __restrict__ dv, float* __restrict__ dtk, float* __restrict__ dtv,
                     float* __restrict__ dbeta, Geo g, int H, int nch) {
  constexpr int MAT = D * D * 2;
  constexpr int NBK = D / 32;
  // As hi, As lo, dB hi, dB lo; the two dB tiles are adjacent (they first
  // hold dA in fp32)
  __shared__ __attribute__((aligned(16))) char sm[4 * MAT];
  char VDN_LDS* Ah = (char VDN_LDS*)sm;
  char VDN_LDS* Al = Ah + MAT;
  char VDN_LDS* Bh = Ah + 2 * MAT;
  char VDN_LDS* Bl = Ah + 3 * MAT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, half = lane >> 5;
  const int ch = blockIdx.x % nch;
  const int slot = (blockIdx.x / nch) % (g.T + 1);
  const int bh = blockIdx.x / nch / (g.T + 1);
  const int b = bh / H, h = bh % H;
  const int N = g.T * g.P;
  const bool text = slot == g.T;
  const int ntok = text ? g.L : g.P;
  const int i0 = ch * GB_CH;
  const int nmine = imin(GB_CH, ntok - i0);
  if (nmine <= 0) return;
  const int NB = N + g.L;
  float* dbrow = dbeta + ((size_t)b * NB + (text ? N : slot * g.P) + i0) * H + h;
  const bool live = text || frame_needs_stats(g, slot);
  const size_t base = text ? ((size_t)b * g.L + i0) * H + h : ((size_t)b * N + (size_t)slot * g.P + i0) * H + h;
  float* dkb = (text ? dtk : dk) + base * D;
  float* dvb = (text ? dtv : dv) + base * D;
  const size_t HD = (size_t)H * D;
  if (!live) {
    for (int i = tid; i < nmine; i += GB_NT) dbrow[(size_t)i * H] = 0.f;
    for (int i = tid; i < nmine * (D / 4); i += GB_NT) {
      const int t = i / (D / 4), c = (i % (D / 4)) * 4;
      *(f32x4*)(dkb + (size_t)t * HD + c) = f32x4{};
      *(f32x4*)(dvb + (size_t)t * HD + c) = f32x4{};
    }
    return;
  }
  const size_t mat = (size_t)D * D;
  const float* dAs = dA + ((size_t)bh * (g.T + 1) + slot) * mat;
  const float* dBs = dB + ((size_t)bh * (g.T + 1) + slot) * mat;
  // dA in fp32 through the (not yet used) dB region, so that As = dA + dA^T
  // is formed from coalesced row reads
  float VDN_LDS* dAl = (float VDN_LDS*)Bh;            // d x d floats: both dB tiles
#pragma unroll 1
  for (int i = tid; i < D * D / 4; i += GB_NT) *(f32x4 VDN_LDS*)(dAl + i * 4) = *(const f32x4*)(dAs + i * 4);
  __syncthreads();
#pragma unroll 1
  for (int i = tid; i < D * D / 8; i += GB_NT) {
    const int r = i / (D / 8), c = (i % (D / 8)) * 8;
    bf16x8 ah, al;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float a = dAl[r * D + c + e] + dAl[(c + e) * D + r];
      bf16 x, y;
      split_bf16(a, x, y);
      ah[e] = x;
      al[e] = y;
    }
    *(bf16x8 VDN_LDS*)(Ah + swz_off<D>(r, c)) = ah;
    *(bf16x8 VDN_LDS*)(Al + swz_off<D>(r, c)) = al;
  }
  __syncthreads();
#pragma unroll 1
  for (int i = tid; i < D * D / 8; i += GB_NT) {
    const int r = i / (D / 8), c = (i % (D / 8)) * 8;
    const f32x4 b0 = *(const f32x4*)(dBs + (size_t)r * D + c);
    const f32x4 b1 = *(const f32x4*)(dBs + (size_t)r * D + c + 4);
    const float bv[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    bf16x8 bh_, bl_;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16 x, y;
      split_bf16(bv[e], x, y);
      bh_[e] = x;
      bl_[e] = y;
    }
    *(bf16x8 VDN_LDS*)(Bh + swz_off<D>(r, c)) = bh_;
    *(bf16x8 VDN_LDS*)(Bl + swz_off<D>(r, c)) = bl_;
  }
  __syncthreads();
  const bf16* kb = (text ? tk : k) + base * D;
  const bf16* vb = (text ? tv : v) + base * D;
  const float* bt = beta + ((size_t)b * NB + (text ? N : slot * g.P) + i0) * H + h;

  for (int t0 = wv * 32; t0 < nmine; t0 += GB_NT / 2) {
    const int tl = imin(t0 + (lane & 31), nmine - 1);   // A-operand row (clamped)
    bf16x8 ka[D / 16], va[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      ka[ks] = *(const bf16x8*)(kb + (size_t)tl * HD + ks * 16 + half * 8);
      va[ks] = *(const bf16x8*)(vb + (size_t)tl * HD + ks * 16 + half * 8);
    }
    // rows of the result: register j -> token t0 + 8*(j/4) + 4*half + j%4
    float bj[16], dbp[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int t = imin(t0 + (j >> 2) * 8 + half * 4 + (j & 3), nmine - 1);
      bj[j] = bt[(size_t)t * H];
      dbp[j] = 0.f;
    }
#pragma unroll
    for (int nb = 0; nb < NBK; ++nb) {
      f32x16 U = f32x16{}, W = f32x16{}, Z = f32x16{};
      const int r = nb * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a_h = lds_row8<D>(Ah, r, ks * 2 + half);
        const bf16x8 a_l = lds_row8<D>(Al, r, ks * 2 + half);
        const bf16x8 b_h = lds_row8<D>(Bh, r, ks * 2 + half);
        const bf16x8 b_l = lds_row8<D>(Bl, r, ks * 2 + half);
        const bf16x8 c_h = lds_col8<D>(Bh, ks * 16, nb * 32, lane);
        const bf16x8 c_l = lds_col8<D>(Bl, ks * 16, nb * 32, lane);
        U = mfma32(ka[ks], a_h, U);
        U = mfma32(ka[ks], a_l, U);
        W = mfma32(ka[ks], b_h, W);
        W = mfma32(ka[ks], b_l, W);
        Z = mfma32(va[ks], c_h, Z);
        Z = mfma32(va[ks], c_l, Z);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int t = t0 + (j >> 2) * 8 + half * 4 + (j & 3);
        if (t < nmine) {
          const size_t e = (size_t)t * HD + r;
          dkb[e] = bj[j] * (U[j] + Z[j]);
          dvb[e] = bj[j] * W[j];
          dbp[j] = fmaf(0.5f * (float)kb[e], U[j], dbp[j]);
          dbp[j] = fmaf((float)vb[e], W[j], dbp[j]);
        }
      }
    }
    // sum over the 32 columns each half holds, then one lane per token
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float x = dbp[j];
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) x += __shfl_xor(x, o, 32);
      dbp[j] = x;
    }
    if ((lane & 31) == 0) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int t = t0 + (j >> 2) * 8 + half * 4 + (j & 3);
        if (t < nmine) dbrow[(size_t)t * H] = dbp[j];
      }
    }
  }
}

constexpr int dr_chunks(const Geo& g) {
  return (imax(g.C, 2) * g.P + DR_CH - 1) / DR_CH;
}

template <int D>
hipError_t launch_dr_d(const void* q, const float* dlin, const float* R, float* dRp, float* dR,
                       float* dq, const vdn_layout_t& l, hipStream_t s) {
  Geo g = make_geo(l);
  const int nch = dr_chunks(g);
  dr_mfma_kernel<D><<<dim3((unsigned)((long)l.batch * l.heads * (g.nc + 1) * nch)), dim3(dr_threads(D)), 0, s>>>(
      (const bf16*)q, dlin, R, dRp, dq, g, l.heads, nch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t mat4 = (size_t)D * D / 4;
  const size_t nslot = (size_t)l.batch * l.heads * (g.nc + 1);
  const size_t n = nslot * mat4;
  dr_sum_kernel<<<dim3((unsigned)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192)), dim3(256), 0, s>>>(
      (const float4*)dRp, (float4*)dR, nch, mat4, nslot);
  return hipGetLastError();
}

template <int D>
hipError_t launch_frame_d(float* GA, float* BB, const float* alpha, const float* states,
                          const float* dspost, float* dalpha, const vdn_layout_t& l,
                          hipStream_t s) {
  Geo g = make_geo(l);
  vda_frame_bwd_kernel<D><<<dim3((unsigned)((long)l.batch * l.heads * (g.T + 1))), dim3(FR_NT), 0, s>>>(
      GA, BB, alpha, states, dspost, dalpha, g, l.heads);
  return hipGetLastError();
}

template <int D>
hipError_t launch_gram_bwd_d(const void* k, const void* v, const void* tk, const void* tv,
                             const float* beta, const float* dA, const float* dB, float* dk,
                             float* dv, float* dtk, float* dtv, float* dbeta,
                             const vdn_layout_t& l, hipStream_t s) {
  Geo g = make_geo(l);
  const int nch = (imax(g.P, g.L) + GB_CH - 1) / GB_CH;
  gram_bwd_mfma_kernel<D><<<dim3((unsigned)((long)l.batch * l.heads * (g.T + 1) * nch)), dim3(GB_NT), 0, s>>>(
      (const bf16*)k, (const bf16*)v, (const bf16*)tk, (const bf16*)tv, beta, dA, dB, dk, dv,
      dtk, dtv, dbeta, g, l.heads, nch);
  return hipGetLastError();
}

}  // namespace

size_t vda_bwd_partial_bytes(const vdn_layout_t& l) {
  Geo g = make_geo(l);
  return (size_t)l.batch * l.heads * (g.nc + 1) * dr_chunks(g) * l.head_dim_k * l.head_dim_k *
         sizeof(float);
}

hipError_t launch_vda_bwd(const void* q, const void* k, const void* v, const void* tk,
                          const void* tv, const float* beta, const float* alpha,
                          const float* dlin, const float* R, float* GA, float* BB,
                          const float* states, float* dRp, float* dR, float* dspost, float* dq,
                          float* dalpha, const vdn_layout_t& l, hipStream_t s) {
  hipError_t e = hipErrorInvalidValue;
  switch (l.head_dim_k) {
    case 128: e = launch_dr_d<128>(q, dlin, R, dRp, dR, dq, l, s); break;
    case 64: e = launch_dr_d<64>(q, dlin, R, dRp, dR, dq, l, s); break;
    case 32: e = launch_dr_d<32>(q, dlin, R, dRp, dR, dq, l, s); break;
  }
  if (e != hipSuccess) return e;
  e = launch_scan_bwd(GA, dR, alpha, l, dspost, s);
  if (e != hipSuccess) return e;
  switch (l.head_dim_k) {
    case 128: e = launch_frame_d<128>(GA, BB, alpha, states, dspost, dalpha, l, s); break;
    case 64: e = launch_frame_d<64>(GA, BB, alpha, states, dspost, dalpha, l, s); break;
    case 32: e = launch_frame_d<32>(GA, BB, alpha, states, dspost, dalpha, l, s); break;
  }
  return e;
}

hipError_t launch_gram_bwd(const void* k, const void* v, const void* tk, const void* tv,
                           const float* beta, const float* dA, const float* dB, float* dk,
                           float* dv, float* dtk, float* dtv, float* dbeta, const vdn_layout_t& l,
                           hipStream_t s) {
  switch (l.head_dim_k) {
    case 128: return launch_gram_bwd_d<128>(k, v, tk, tv, beta, dA, dB, dk, dv, dtk, dtv, dbeta, l, s);
    case 64: return launch_gram_bwd_d<64>(k, v, tk, tv, beta, dA, dB, dk, dv, dtk, dtv, dbeta, l, s);
    case 32: return launch_gram_bwd_d<32>(k, v, tk, tv, beta, dA, dB, dk, dv, dtk, dtv, dbeta, l, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace vdn
