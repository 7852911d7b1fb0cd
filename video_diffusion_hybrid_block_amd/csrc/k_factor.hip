// Per-frame factor of the VDA update: G = (I + A)^-1 for every frame the scans
// fold and for the text block, so the sequential scan only multiplies.
// (I + A) is symmetric positive definite with every eigenvalue >= 1 (A is a
// beta-weighted Gram), so Cholesky needs no pivoting: I + A = L L^T, then
// X = L^-1 by forward substitution, then G = X^T X.  G has spectral norm <= 1,
// the non-expansive transition of the update.
// [deepmagic blog "生成比播放還快：Video DeltaNet 用 11 秒產出 14 秒 768p 影片",
//  section 用兩條分支取代一條 (S = (S̄ + B)(I + A)^-1, non-expansive);
//  PaperDaily "伯克利与Impossible视频生成" §四 (the (I+A) inverse couples the
//  tokens of one frame)]
//
// gfx950 design: one workgroup of 256 threads per (batch, head, slot), laid out
// as a 16 x 16 grid; thread (ti, tk) keeps the (d/16) x (d/16) block of rows
// ti, columns tk of the matrix in registers for the whole factorisation.  Each
// elimination step broadcasts one column (Cholesky) or one row (substitution)
// through LDS with double-buffered vectors: one barrier per step.  L is kept in
// LDS for the substitution; X replaces it for the product.  All fp32.
#include "vdn_device.h"
#include "vdn_internal.h"

namespace vdn {

namespace {

template <int D>
__global__ void __launch_bounds__(256)
factor_kernel(float* __restrict__ A, Geo g, int nslots, bool all_frames) {
  constexpr int BS = D / 16;
  constexpr int LD = D + 1;
  __shared__ float Ls[D * LD];
  __shared__ float vec[2][D];

  const int tid = threadIdx.x;
  const int ti = tid >> 4, tk = tid & 15;
  const int r0 = ti * BS, c0 = tk * BS;
  const int task = blockIdx.x;
  const int bh = task / nslots;
  const int slot = slot_of(g, task % nslots, all_frames);
  float* Mg = A + ((size_t)bh * (g.T + 1) + slot) * D * D;

  // M = I + A, owned block in registers.
  float m[BS][BS];
#pragma unroll
  for (int i = 0; i < BS; ++i)
#pragma unroll
    for (int j = 0; j < BS; ++j) {
      float x = Mg[(size_t)(r0 + i) * D + c0 + j];
      m[i][j] = x + ((r0 + i) == (c0 + j) ? 1.0f : 0.0f);
    }

  // ---- Cholesky, right-looking, one column per step ----
  for (int j = 0; j < D; ++j) {
    float* col = vec[j & 1];
    if (tk == j / BS && ti >= j / BS) {
      const int jm = j % BS;
#pragma unroll
      for (int i = 0; i < BS; ++i) {
        float val = 0.f;
#pragma unroll
        for (int c = 0; c < BS; ++c) val = (c == jm) ? m[i][c] : val;
        if (r0 + i >= j) col[r0 + i] = val;
      }
    }
    __syncthreads();
    const float piv = col[j];
    const float rs = rsqrtf(piv);
    if (ti >= j / BS) {
      float li[BS], lk[BS];
#pragma unroll
      for (int i = 0; i < BS; ++i) li[i] = (r0 + i >= j) ? col[r0 + i] * rs : 0.f;
#pragma unroll
      for (int c = 0; c < BS; ++c) lk[c] = (c0 + c > j) ? col[c0 + c] * rs : 0.f;
#pragma unroll
      for (int i = 0; i < BS; ++i)
#pragma unroll
        for (int c = 0; c < BS; ++c) {
          if (c0 + c == j) {
            if (r0 + i >= j) {
              m[i][c] = li[i];               // final L[i][j]
              Ls[(r0 + i) * LD + j] = li[i];
            }
          } else if (r0 + i >= c0 + c) {
            m[i][c] = fmaf(-li[i], lk[c], m[i][c]);
          }
        }
    }
  }
  __syncthreads();

  // ---- X = L^-1 (lower), forward substitution, one row per step ----
  float x[BS][BS];
#pragma unroll
  for (int i = 0; i < BS; ++i)
#pragma unroll
    for (int c = 0; c < BS; ++c) x[i][c] = (r0 + i == c0 + c) ? 1.0f : 0.0f;
  for (int kk = 0; kk < D; ++kk) {
    float* row = vec[kk & 1];
    if (ti == kk / BS && tk <= ti) {
      const float inv = 1.0f / Ls[kk * LD + kk];
      const int im = kk % BS;
#pragma unroll
      for (int i = 0; i < BS; ++i) {
        if (i != im) continue;
#pragma unroll
        for (int c = 0; c < BS; ++c) {
          if (c0 + c <= kk) {
            x[i][c] *= inv;
            row[c0 + c] = x[i][c];
          }
        }
      }
    }
    __syncthreads();
    if (tk <= ti && r0 + BS - 1 > kk && c0 <= kk) {
#pragma unroll
      for (int i = 0; i < BS; ++i) {
        if (r0 + i > kk) {
          const float lik = Ls[(r0 + i) * LD + kk];
#pragma unroll
          for (int c = 0; c < BS; ++c)
            if (c0 + c <= kk) x[i][c] = fmaf(-lik, row[c0 + c], x[i][c]);
        }
      }
    }
  }
  __syncthreads();
  // X (lower, zeros above) replaces L in LDS.
#pragma unroll
  for (int i = 0; i < BS; ++i)
#pragma unroll
    for (int c = 0; c < BS; ++c)
      Ls[(r0 + i) * LD + c0 + c] = (tk <= ti && r0 + i >= c0 + c) ? x[i][c] : 0.0f;
  __syncthreads();

  // ---- G = X^T X, block (ti, tk) ----
  float gacc[BS][BS];
#pragma unroll
  for (int i = 0; i < BS; ++i)
#pragma unroll
    for (int c = 0; c < BS; ++c) gacc[i][c] = 0.f;
  const int kstart = (ti > tk ? ti : tk) * BS;
  for (int kk = kstart; kk < D; ++kk) {
    float xa[BS], xb[BS];
#pragma unroll
    for (int i = 0; i < BS; ++i) xa[i] = Ls[kk * LD + r0 + i];
#pragma unroll
    for (int c = 0; c < BS; ++c) xb[c] = Ls[kk * LD + c0 + c];
#pragma unroll
    for (int i = 0; i < BS; ++i)
#pragma unroll
      for (int c = 0; c < BS; ++c) gacc[i][c] = fmaf(xa[i], xb[c], gacc[i][c]);
  }
#pragma unroll
  for (int i = 0; i < BS; ++i)
#pragma unroll
    for (int c = 0; c < BS; ++c) Mg[(size_t)(r0 + i) * D + c0 + c] = gacc[i][c];
}

template <int D>
hipError_t launch_d(float* A, const vdn_layout_t& l, bool all_frames, hipStream_t s) {
  Geo g = make_geo(l);
  int nslots = count_slots(g, all_frames);
  long grid = (long)l.batch * l.heads * nslots;
  factor_kernel<D><<<dim3((unsigned)grid), dim3(256), 0, s>>>(A, g, nslots, all_frames);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_factor(float* A, const vdn_layout_t& l, bool all_frames, hipStream_t s) {
  switch (l.head_dim_k) {
    case 128: return launch_d<128>(A, l, all_frames, s);
    case 64: return launch_d<64>(A, l, all_frames, s);
    case 32: return launch_d<32>(A, l, all_frames, s);
    case 16: return launch_d<16>(A, l, all_frames, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace vdn
