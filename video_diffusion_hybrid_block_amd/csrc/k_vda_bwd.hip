// Backward pass of the linear (VDA) branch, after the merge backward:
//
//  1. read slots (dr_kernel): each video token reads o = R_c q with R_c its
//     chunk's summed state (slot nc, the text write, for anchor frames), so
//     dR_c = sum_i do_i q_i^T over the slot's tokens and q_i gets R_c^T do_i
//     (written as the first part of dq);
//  2. the reverse scan (k_scan.hip) turns dR into dS_j, the gradient of each
//     chain's state after each step;
//  3. per frame (vda_frame_bwd_kernel): a step S_j = X_j G_j with
//     X_j = alpha_f S_{j-1} + B_f gives dX = dS_j G_j (G symmetric), so
//     dB_f += dX, dalpha_f += <dX, S_{j-1}>, dG_f += X_j^T dS_j, summed over
//     the chains that fold f; G = (I + A)^-1 gives dA_f = -G dG_f G.  The text
//     write S_x = B_x G_x starts both chains at S_x / 2, so
//     dS_x = (dS_0^fwd + dS_0^bwd) / 2, dB_x = dS_x G_x, dG_x = B_x^T dS_x;
//  4. per token (gram_bwd_kernel): A = sum beta k k^T, B = sum beta v k^T give
//     dk_i += beta_i ((dA + dA^T) k_i + dB^T v_i), dv_i += beta_i dB k_i,
//     dbeta_i = k_i^T dA k_i + v_i^T dB k_i.
// [the forward: deepmagic blog "生成比播放還快", section 用兩條分支取代一條
//  (S = (S̄ + B)(I + A)^-1); PaperDaily "伯克利与Impossible视频生成" §三 (two
//  states from half the text write, summed read), §四 (frame statistics)]
//
// These are fp32 VALU kernels: their work (a few d x d x d products per
// frame, three d x d matrix-vector products per token) is a few percent of
// the softmax backward.
#include "vdn_device.h"
#include "vdn_internal.h"

namespace vdn {

namespace {

// ---------------------------------------------------------------------------
// 1. dR and the linear part of dq.  One workgroup per (batch, head, slot).
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
dr_kernel(const bf16* __restrict__ q, const float* __restrict__ dlin, const float* __restrict__ R,
          float* __restrict__ dR, float* __restrict__ dq, Geo g, int H) {
  constexpr int TT = 32;                 // tokens per tile
  constexpr int RB = D / 16;             // dR block per thread: RB x RB
  constexpr int QC = D / 8;              // dq columns per thread
  constexpr int LD = D + 4;
  __shared__ __attribute__((aligned(16))) float Rs[D * D];
  __shared__ __attribute__((aligned(16))) float dl[TT * LD];
  __shared__ __attribute__((aligned(16))) float qs[TT * LD];
  const int tid = threadIdx.x;
  const int slot = blockIdx.x % (g.nc + 1);
  const int bh = blockIdx.x / (g.nc + 1);
  const int b = bh / H, h = bh % H;
  const size_t mat = (size_t)D * D;
  const float* Rc = R + ((size_t)bh * (g.nc + 1) + slot) * mat;
  for (int i = tid; i < D * D; i += 256) Rs[i] = Rc[i];
  const int N = g.T * g.P;
  const int ti = tid >> 4, tj = tid & 15;
  float acc[RB][RB];
#pragma unroll
  for (int a = 0; a < RB; ++a)
#pragma unroll
    for (int c = 0; c < RB; ++c) acc[a][c] = 0.f;
  // frames of the slot: the chunk's non-anchor frames, or the anchors
  int f0, f1;
  if (slot < g.nc) {
    f0 = slot * g.C;
    f1 = imin(g.T, f0 + g.C);
  } else {
    f0 = 0;
    f1 = g.T;
  }
  for (int f = f0; f < f1; ++f) {
    if ((slot < g.nc) == is_anchor(g, f)) continue;
    for (int t0 = 0; t0 < g.P; t0 += TT) {
      const int nt = imin(TT, g.P - t0);
      __syncthreads();                   // previous tile consumed (and Rs loaded)
      for (int i = tid; i < TT * D; i += 256) {
        const int r = i / D, c = i % D;
        float dv = 0.f, qv = 0.f;
        if (r < nt) {
          const size_t off = (((size_t)b * N + (size_t)f * g.P + t0 + r) * H + h) * D + c;
          dv = dlin[off];
          qv = (float)q[off];
        }
        dl[r * LD + c] = dv;
        qs[r * LD + c] = qv;
      }
      __syncthreads();
      // dR block (rows ti*RB.., cols tj*RB..) += dlin^T q over the tile
      for (int r = 0; r < nt; ++r) {
        float dv[RB], qv[RB];
#pragma unroll
        for (int a = 0; a < RB; ++a) dv[a] = dl[r * LD + ti * RB + a];
#pragma unroll
        for (int c = 0; c < RB; ++c) qv[c] = qs[r * LD + tj * RB + c];
#pragma unroll
        for (int a = 0; a < RB; ++a)
#pragma unroll
          for (int c = 0; c < RB; ++c) acc[a][c] = fmaf(dv[a], qv[c], acc[a][c]);
      }
      // dq_i = R^T dlin_i: 8 threads per token, QC columns each
      const int tok = tid >> 3, cg = (tid & 7) * QC;
      if (tok < nt) {
        float o[QC];
#pragma unroll
        for (int e = 0; e < QC; ++e) o[e] = 0.f;
        for (int r = 0; r < D; ++r) {
          const float dv = dl[tok * LD + r];
#pragma unroll
          for (int e = 0; e < QC; ++e) o[e] = fmaf(Rs[r * D + cg + e], dv, o[e]);
        }
        float* dst = dq + (((size_t)b * N + (size_t)f * g.P + t0 + tok) * H + h) * D + cg;
#pragma unroll
        for (int e = 0; e < QC; e += 4) *(f32x4*)(dst + e) = f32x4{o[e], o[e + 1], o[e + 2], o[e + 3]};
      }
    }
  }
  float* dst = dR + ((size_t)bh * (g.nc + 1) + slot) * mat;
#pragma unroll
  for (int a = 0; a < RB; ++a)
#pragma unroll
    for (int c = 0; c < RB; ++c) dst[(size_t)(ti * RB + a) * D + tj * RB + c] = acc[a][c];
}

// ---------------------------------------------------------------------------
// d x d x d products for the per-frame step: a 16 x 16 thread grid, thread
// (ti, tj) owning the RB x RB block at rows ti*RB, columns tj*RB.
// ---------------------------------------------------------------------------
template <int D>
struct Tile {
  static constexpr int RB = D / 16;
  static constexpr int LD = D + 1;       // padded LDS row (floats)
};

// acc += op(A) * B, A and B in LDS ([D][LD]), op(A) = A or A^T.
template <int D, bool TA>
__device__ __forceinline__ void mm_acc(const float* A, const float* B, int ti, int tj,
                                       float (&acc)[D / 16][D / 16]) {
  constexpr int RB = D / 16, LD = D + 1;
  for (int k = 0; k < D; ++k) {
    float av[RB], bv[RB];
#pragma unroll
    for (int a = 0; a < RB; ++a) av[a] = TA ? A[k * LD + ti * RB + a] : A[(ti * RB + a) * LD + k];
#pragma unroll
    for (int c = 0; c < RB; ++c) bv[c] = B[k * LD + tj * RB + c];
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
      for (int c = 0; c < RB; ++c) acc[a][c] = fmaf(av[a], bv[c], acc[a][c]);
  }
}

template <int D>
__device__ __forceinline__ void load_mat(float* dst, const float* src, float scale, int tid) {
  constexpr int LD = D + 1;
  for (int i = tid; i < D * D; i += 256) dst[(i / D) * LD + i % D] = scale * src[i];
}

// ---------------------------------------------------------------------------
// 3. Per frame (and the text slot T): dA, dB in place of G, B; dalpha.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
vda_frame_bwd_kernel(float* __restrict__ GA, float* __restrict__ BB,
                     const float* __restrict__ alpha, const float* __restrict__ states,
                     const float* __restrict__ dspost, float* __restrict__ dalpha, Geo g, int H) {
  constexpr int RB = D / 16, LD = D + 1;
  __shared__ float L1[D * LD];
  __shared__ float L2[D * LD];
  __shared__ float red[256];
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
    for (int i = tid; i < D * D; i += 256) {
      Gs[i] = 0.f;
      Bs[i] = 0.f;
    }
    if (!text && tid == 0) dalpha[((size_t)b * g.T + slot) * H + h] = 0.f;
    return;
  }
  float dB[RB][RB], dG[RB][RB];
#pragma unroll
  for (int a = 0; a < RB; ++a)
#pragma unroll
    for (int c = 0; c < RB; ++c) dB[a][c] = dG[a][c] = 0.f;
  float dal = 0.f;
  const float* post = dspost + (size_t)bh * 2 * (g.T + 1) * mat;
  const float* st = states + (size_t)bh * 2 * (g.T + 1) * mat;
  if (text) {
    // dS_x = (dS_0^fwd + dS_0^bwd) / 2; dB_x = dS_x G_x; dG_x = B_x^T dS_x
    const float* p0 = post;
    const float* p1 = post + (size_t)(g.T + 1) * mat;
    for (int i = tid; i < D * D; i += 256) L1[(i / D) * LD + i % D] = 0.5f * (p0[i] + p1[i]);
    load_mat<D>(L2, Gs, 1.0f, tid);
    __syncthreads();
    mm_acc<D, false>(L1, L2, ti, tj, dB);
    __syncthreads();
    load_mat<D>(L2, Bs, 1.0f, tid);
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
      load_mat<D>(L1, dSj, 1.0f, tid);
      load_mat<D>(L2, Gs, 1.0f, tid);
      __syncthreads();
      float dX[RB][RB];
#pragma unroll
      for (int x = 0; x < RB; ++x)
#pragma unroll
        for (int c = 0; c < RB; ++c) dX[x][c] = 0.f;
      mm_acc<D, false>(L1, L2, ti, tj, dX);
#pragma unroll
      for (int x = 0; x < RB; ++x)
#pragma unroll
        for (int c = 0; c < RB; ++c) {
          dB[x][c] += dX[x][c];
          dal = fmaf(dX[x][c], Sp[(size_t)(ti * RB + x) * D + tj * RB + c], dal);
        }
      __syncthreads();
      // X = alpha S_{j-1} + B_f
      for (int i = tid; i < D * D; i += 256) L2[(i / D) * LD + i % D] = fmaf(a, Sp[i], Bs[i]);
      __syncthreads();
      mm_acc<D, true>(L2, L1, ti, tj, dG);
      __syncthreads();
    }
    red[tid] = dal;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (tid < s) red[tid] += red[tid + s];
      __syncthreads();
    }
    if (tid == 0) dalpha[((size_t)b * g.T + slot) * H + h] = red[0];
  }
  // dA = -G dG G
  load_mat<D>(L2, Gs, 1.0f, tid);
#pragma unroll
  for (int x = 0; x < RB; ++x)
#pragma unroll
    for (int c = 0; c < RB; ++c) L1[(ti * RB + x) * LD + tj * RB + c] = dG[x][c];
  __syncthreads();
  float t1[RB][RB];
#pragma unroll
  for (int x = 0; x < RB; ++x)
#pragma unroll
    for (int c = 0; c < RB; ++c) t1[x][c] = 0.f;
  mm_acc<D, false>(L2, L1, ti, tj, t1);     // G dG
  __syncthreads();
#pragma unroll
  for (int x = 0; x < RB; ++x)
#pragma unroll
    for (int c = 0; c < RB; ++c) L1[(ti * RB + x) * LD + tj * RB + c] = t1[x][c];
  __syncthreads();
  float t2[RB][RB];
#pragma unroll
  for (int x = 0; x < RB; ++x)
#pragma unroll
    for (int c = 0; c < RB; ++c) t2[x][c] = 0.f;
  mm_acc<D, false>(L1, L2, ti, tj, t2);     // (G dG) G
  __syncthreads();                          // every read of G_f / B_f done
#pragma unroll
  for (int x = 0; x < RB; ++x)
#pragma unroll
    for (int c = 0; c < RB; ++c) {
      const size_t e = (size_t)(ti * RB + x) * D + tj * RB + c;
      Gs[e] = -t2[x][c];
      Bs[e] = dB[x][c];
    }
}

// ---------------------------------------------------------------------------
// 4. Per token of every frame (slot T: the text tokens): dk, dv (added),
// dbeta (written; zero for frames no chain folds).
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
gram_bwd_kernel(const bf16* __restrict__ k, const bf16* __restrict__ v,
                const bf16* __restrict__ tk, const bf16* __restrict__ tv,
                const float* __restrict__ beta, const float* __restrict__ dA,
                const float* __restrict__ dB, float* __restrict__ dk, float* __restrict__ dv,
                float* __restrict__ dtk, float* __restrict__ dtv, float* __restrict__ dbeta,
                Geo g, int H) {
  constexpr int LD = D + 1;
  constexpr int TT = 16;                 // tokens per pass
  constexpr int RPT = D / 16;            // output rows per thread
  __shared__ float As[D * LD];           // dA + dA^T
  __shared__ float Bs[D * LD];           // dB
  __shared__ float kv[TT][2][D];
  const int tid = threadIdx.x;
  const int slot = blockIdx.x % (g.T + 1);
  const int bh = blockIdx.x / (g.T + 1);
  const int b = bh / H, h = bh % H;
  const int N = g.T * g.P;
  const bool text = slot == g.T;
  const int ntok = text ? g.L : g.P;
  if (ntok == 0) return;
  const int NB = N + g.L;
  float* dbrow = dbeta + ((size_t)b * NB + (text ? N : slot * g.P)) * H + h;
  const bool live = text || frame_needs_stats(g, slot);
  if (!live) {
    for (int i = tid; i < ntok; i += 256) dbrow[(size_t)i * H] = 0.f;
    return;
  }
  const size_t mat = (size_t)D * D;
  const float* dAs = dA + ((size_t)bh * (g.T + 1) + slot) * mat;
  const float* dBs = dB + ((size_t)bh * (g.T + 1) + slot) * mat;
  for (int i = tid; i < D * D; i += 256) {
    const int r = i / D, c = i % D;
    As[r * LD + c] = dAs[i] + dAs[(size_t)c * D + r];
    Bs[r * LD + c] = dBs[i];
  }
  const bf16* kb = text ? tk + ((size_t)b * g.L * H + h) * D : k + (((size_t)b * N + (size_t)slot * g.P) * H + h) * D;
  const bf16* vb = text ? tv + ((size_t)b * g.L * H + h) * D : v + (((size_t)b * N + (size_t)slot * g.P) * H + h) * D;
  float* dkb = text ? dtk + ((size_t)b * g.L * H + h) * D : dk + (((size_t)b * N + (size_t)slot * g.P) * H + h) * D;
  float* dvb = text ? dtv + ((size_t)b * g.L * H + h) * D : dv + (((size_t)b * N + (size_t)slot * g.P) * H + h) * D;
  const float* btok = beta + ((size_t)b * NB + (text ? N : slot * g.P)) * H + h;
  const int tk_ = tid >> 4, rl = tid & 15;
  for (int t0 = 0; t0 < ntok; t0 += TT) {
    __syncthreads();                     // previous tokens consumed (and matrices loaded)
    for (int i = tid; i < TT * D; i += 256) {
      const int t = i / D, c = i % D;
      float kx = 0.f, vx = 0.f;
      if (t0 + t < ntok) {
        kx = (float)kb[(size_t)(t0 + t) * H * D + c];
        vx = (float)vb[(size_t)(t0 + t) * H * D + c];
      }
      kv[t][0][c] = kx;
      kv[t][1][c] = vx;
    }
    __syncthreads();
    const int t = t0 + tk_;
    // rows r = rl + 16 m: u = (dA + dA^T) k, w = dB k, z = dB^T v
    float u[RPT], w[RPT], z[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) u[m] = w[m] = z[m] = 0.f;
    for (int c = 0; c < D; ++c) {
      const float kc = kv[tk_][0][c], vc = kv[tk_][1][c];
#pragma unroll
      for (int m = 0; m < RPT; ++m) {
        const int r = rl + 16 * m;
        u[m] = fmaf(As[r * LD + c], kc, u[m]);
        w[m] = fmaf(Bs[r * LD + c], kc, w[m]);
        z[m] = fmaf(Bs[c * LD + r], vc, z[m]);
      }
    }
    // dbeta = k^T dA k + v^T dB k = k . u / 2 + v . w
    float db = 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int r = rl + 16 * m;
      db = fmaf(0.5f * kv[tk_][0][r], u[m], db);
      db = fmaf(kv[tk_][1][r], w[m], db);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) db += __shfl_xor(db, o, 16);
    if (t < ntok) {
      const float bt = btok[(size_t)t * H];
      float* dkr = dkb + (size_t)t * H * D;
      float* dvr = dvb + (size_t)t * H * D;
#pragma unroll
      for (int m = 0; m < RPT; ++m) {
        const int r = rl + 16 * m;
        dkr[r] += bt * (u[m] + z[m]);
        dvr[r] += bt * w[m];
      }
      if (rl == 0) dbrow[(size_t)t * H] = db;
    }
  }
}

template <int D>
hipError_t launch_dr_d(const void* q, const float* dlin, const float* R, float* dR, float* dq,
                       const vdn_layout_t& l, hipStream_t s) {
  Geo g = make_geo(l);
  dr_kernel<D><<<dim3((unsigned)((long)l.batch * l.heads * (g.nc + 1))), dim3(256), 0, s>>>(
      (const bf16*)q, dlin, R, dR, dq, g, l.heads);
  return hipGetLastError();
}

template <int D>
hipError_t launch_frame_d(float* GA, float* BB, const float* alpha, const float* states,
                          const float* dspost, float* dalpha, const vdn_layout_t& l,
                          hipStream_t s) {
  Geo g = make_geo(l);
  vda_frame_bwd_kernel<D><<<dim3((unsigned)((long)l.batch * l.heads * (g.T + 1))), dim3(256), 0, s>>>(
      GA, BB, alpha, states, dspost, dalpha, g, l.heads);
  return hipGetLastError();
}

template <int D>
hipError_t launch_gram_bwd_d(const void* k, const void* v, const void* tk, const void* tv,
                             const float* beta, const float* dA, const float* dB, float* dk,
                             float* dv, float* dtk, float* dtv, float* dbeta,
                             const vdn_layout_t& l, hipStream_t s) {
  Geo g = make_geo(l);
  gram_bwd_kernel<D><<<dim3((unsigned)((long)l.batch * l.heads * (g.T + 1))), dim3(256), 0, s>>>(
      (const bf16*)k, (const bf16*)v, (const bf16*)tk, (const bf16*)tv, beta, dA, dB, dk, dv,
      dtk, dtv, dbeta, g, l.heads);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_vda_bwd(const void* q, const void* k, const void* v, const void* tk,
                          const void* tv, const float* beta, const float* alpha,
                          const float* dlin, const float* R, float* GA, float* BB,
                          const float* states, float* dR, float* dspost, float* dq, float* dk,
                          float* dv, float* dtk, float* dtv, float* dbeta, float* dalpha,
                          const vdn_layout_t& l, hipStream_t s) {
  hipError_t e = hipErrorInvalidValue;
  switch (l.head_dim_k) {
    case 128: e = launch_dr_d<128>(q, dlin, R, dR, dq, l, s); break;
    case 64: e = launch_dr_d<64>(q, dlin, R, dR, dq, l, s); break;
    case 32: e = launch_dr_d<32>(q, dlin, R, dR, dq, l, s); break;
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
