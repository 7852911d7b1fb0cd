// Per-frame factor of the VDA update: G = (I + A)^-1 for every frame the scans
// fold and for the text block, so the sequential scan only multiplies.
// (I + A) is symmetric positive definite with every eigenvalue >= 1 (A is a
// beta-weighted Gram), so elimination needs no pivoting.
// G is formed by a symmetric sweep (below).  G has spectral norm <= 1, the
// non-expansive transition of the update.
// [deepmagic blog "生成比播放還快：Video DeltaNet 用 11 秒產出 14 秒 768p 影片",
//  section 用兩條分支取代一條 (S = (S̄ + B)(I + A)^-1, non-expansive);
//  PaperDaily "伯克利与Impossible视频生成" §四 (the (I+A) inverse couples the
//  tokens of one frame)]
//
// gfx950 design: one workgroup of 256 threads per (batch, head, slot), laid out
// as a 16 x 16 grid; thread (ti, tk) keeps the (d/16) x (d/16) block of rows
// ti, columns tk of the matrix in registers.  The inverse is formed in place
// by the symmetric sweep (Gauss-Jordan elimination on an SPD matrix, pivots
// taken in order, all positive): sweeping pivot k maps M to B with
//   B[i][j] = M[i][j] - M[i][k] M[k][j] / M[k][k]   (i, j != k)
//   B[i][k] = B[k][i] = M[i][k] / M[k][k],   B[k][k] = -1 / M[k][k],
// and sweeping every pivot once leaves -M^-1.  Every intermediate stays
// symmetric, so one row broadcast through LDS per pivot gives each thread the
// column values it needs too: one barrier per pivot, d in all (a Cholesky,
// triangular inverse and X^T X take 2d barrier steps plus a product).  With
// w = M[k][.] / sqrt(M[k][k]) the update is m[i][j] -= w_i w_j, bitwise
// symmetric, so G comes out exactly symmetric (the scan reads its rows as
// columns).  The row loop is unrolled by the block size so every register
// index is static.  All fp32; 2*d floats of LDS, so several workgroups share a
// CU.
#include "vdn_device.h"
#include "vdn_internal.h"

namespace vdn {

namespace {

template <int D>
__global__ void __launch_bounds__(256)
factor_kernel(float* __restrict__ A, Geo g, int nslots, bool all_frames) {
  constexpr int BS = D / 16;       // rows / columns per thread block
  __shared__ __attribute__((aligned(16))) float rowbuf[2][D];

  const int tid = threadIdx.x;
  const int ti = tid & 15, tk = tid >> 4;
  const int r0 = ti * BS, c0 = tk * BS;
  const int task = blockIdx.x;
  const int bh = task / nslots;
  const int slot = slot_of(g, task % nslots, all_frames);
  float* Mg = A + ((size_t)bh * (g.T + 1) + slot) * D * D;

  // I + A from the lower triangle of A (the Gram's two triangles can differ in
  // the last bit), so the swept matrix is exactly symmetric.
  float m[BS][BS];
#pragma unroll
  for (int i = 0; i < BS; ++i)
#pragma unroll
    for (int j = 0; j < BS; ++j) {
      const int r = r0 + i, c = c0 + j;
      m[i][j] = Mg[(size_t)(r >= c ? r : c) * D + (r >= c ? c : r)] + (r == c ? 1.0f : 0.0f);
    }

  if (ti == 0) {
#pragma unroll
    for (int c = 0; c < BS; ++c) rowbuf[0][c0 + c] = m[0][c];
  }
  __syncthreads();
  for (int kb = 0; kb < 16; ++kb) {
#pragma unroll
    for (int km = 0; km < BS; ++km) {
      const int k = kb * BS + km;
      const float* rk = rowbuf[k & 1];
      const float sk = rsqrtf(rk[k]);
      float wi[BS], wc[BS];
#pragma unroll
      for (int i = 0; i < BS; ++i) wi[i] = rk[r0 + i] * sk;
#pragma unroll
      for (int c = 0; c < BS; ++c) wc[c] = rk[c0 + c] * sk;
#pragma unroll
      for (int i = 0; i < BS; ++i)
#pragma unroll
        for (int c = 0; c < BS; ++c) m[i][c] = fmaf(-wi[i], wc[c], m[i][c]);
      if (ti == kb) {                       // row k: M[k][c] / M[k][k]
#pragma unroll
        for (int c = 0; c < BS; ++c) m[km][c] = wc[c] * sk;
      }
      if (tk == kb) {                       // column k
#pragma unroll
        for (int i = 0; i < BS; ++i) m[i][km] = wi[i] * sk;
        if (ti == kb) m[km][km] = -sk * sk;
      }
      // the owners of row k+1 publish it (after this pivot) for the next step
      if (km + 1 < BS) {
        if (ti == kb) {
#pragma unroll
          for (int c = 0; c < BS; ++c) rowbuf[(k + 1) & 1][c0 + c] = m[(km + 1) % BS][c];
        }
      } else if (kb + 1 < 16) {
        if (ti == kb + 1) {
#pragma unroll
          for (int c = 0; c < BS; ++c) rowbuf[(k + 1) & 1][c0 + c] = m[0][c];
        }
      }
      __syncthreads();
    }
  }
  // G = (I + A)^-1 = -B
#pragma unroll
  for (int i = 0; i < BS; ++i)
#pragma unroll
    for (int c = 0; c < BS; ++c) Mg[(size_t)(r0 + i) * D + c0 + c] = -m[i][c];
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
