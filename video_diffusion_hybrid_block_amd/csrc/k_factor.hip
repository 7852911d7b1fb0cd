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
// through LDS with double-buffered vectors: one barrier per step.  The step
// loop is unrolled by the block size so every register index is static (no
// divergent selects), and waves own column groups so a wave whose columns are
// finished skips the step.  L is kept in LDS for the substitution; X replaces
// it for the product.  All fp32.
#include "vdn_device.h"
#include "vdn_internal.h"

namespace vdn {

namespace {

template <int D>
__global__ void __launch_bounds__(256)
factor_kernel(float* __restrict__ A, Geo g, int nslots, bool all_frames) {
  constexpr int BS = D / 16;       // rows / columns per thread block
  constexpr int LD = D + 1;
  __shared__ float Ls[D * LD];
  __shared__ __attribute__((aligned(16))) float vec[2][D];

  const int tid = threadIdx.x;
  // Waves own column groups (tk = 4w .. 4w+3), so a wave whose columns are
  // finished skips a step as a whole.
  const int ti = tid & 15, tk = tid >> 4;
  const int wq = tid >> 6;
  const int r0 = ti * BS, c0 = tk * BS;
  const int task = blockIdx.x;
  const int bh = task / nslots;
  const int slot = slot_of(g, task % nslots, all_frames);
  float* Mg = A + ((size_t)bh * (g.T + 1) + slot) * D * D;

  float m[BS][BS];
#pragma unroll
  for (int i = 0; i < BS; ++i)
#pragma unroll
    for (int j = 0; j < BS; ++j)
      m[i][j] = Mg[(size_t)(r0 + i) * D + c0 + j] + ((r0 + i) == (c0 + j) ? 1.0f : 0.0f);

  // ---- Cholesky I + A = L L^T, right-looking, one column per step ----
  // Step j: the owners of column j publish it; every thread then forms
  // l_i = M[i][j] / sqrt(M[j][j]) for its rows (zero above j) and applies the
  // rank-1 update to its columns > j.  Column j of L (zeros above the
  // diagonal) goes to LDS.
  for (int kb = 0; kb < 16; ++kb) {
#pragma unroll
    for (int km = 0; km < BS; ++km) {
      const int j = kb * BS + km;
      float* col = vec[j & 1];
      if (tk == kb) {
#pragma unroll
        for (int i = 0; i < BS; ++i) col[r0 + i] = m[i][km];
      }
      __syncthreads();
      if (4 * wq + 3 >= kb) {
        const float rs = rsqrtf(col[j]);
        float li[BS], lk[BS];
#pragma unroll
        for (int i = 0; i < BS; ++i) {
          const float v = col[r0 + i];
          li[i] = (r0 + i >= j) ? v * rs : 0.f;
        }
#pragma unroll
        for (int c = 0; c < BS; ++c) {
          const float v = col[c0 + c];
          lk[c] = (c0 + c > j) ? v * rs : 0.f;
        }
#pragma unroll
        for (int i = 0; i < BS; ++i)
#pragma unroll
          for (int c = 0; c < BS; ++c) m[i][c] = fmaf(-li[i], lk[c], m[i][c]);
        if (tk == kb) {
#pragma unroll
          for (int i = 0; i < BS; ++i) Ls[(r0 + i) * LD + j] = li[i];
        }
      }
    }
  }
  __syncthreads();

  // ---- X = L^-1 (lower triangular), forward substitution by rows ----
  float x[BS][BS];
#pragma unroll
  for (int i = 0; i < BS; ++i)
#pragma unroll
    for (int c = 0; c < BS; ++c) x[i][c] = (r0 + i == c0 + c) ? 1.0f : 0.0f;
  for (int kb = 0; kb < 16; ++kb) {
#pragma unroll
    for (int km = 0; km < BS; ++km) {
      const int k = kb * BS + km;
      float* row = vec[k & 1];
      if (ti == kb) {
        const float inv = 1.0f / Ls[k * LD + k];
#pragma unroll
        for (int c = 0; c < BS; ++c) {
          x[km][c] *= inv;
          row[c0 + c] = x[km][c];
        }
      }
      __syncthreads();
      if (4 * wq <= kb) {
        float lik[BS], rv[BS];
#pragma unroll
        for (int i = 0; i < BS; ++i) {
          const float v = Ls[(r0 + i) * LD + k];
          lik[i] = (r0 + i > k) ? v : 0.f;
        }
#pragma unroll
        for (int c = 0; c < BS; ++c) rv[c] = row[c0 + c];
#pragma unroll
        for (int i = 0; i < BS; ++i)
#pragma unroll
          for (int c = 0; c < BS; ++c) x[i][c] = fmaf(-lik[i], rv[c], x[i][c]);
      }
    }
  }
  __syncthreads();
  // X (exactly lower triangular) replaces L in LDS.
#pragma unroll
  for (int i = 0; i < BS; ++i)
#pragma unroll
    for (int c = 0; c < BS; ++c) Ls[(r0 + i) * LD + c0 + c] = x[i][c];
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
