// Frame statistics and factor of the VDA branch in one pass, for the layer's
// forward path: for every frame the scans fold (and the text block)
//   A = sum_i beta_i k_i k_i^T   (the key Gram of the frame),
//   B = sum_i beta_i v_i k_i^T   (its write),
//   G = (I + A)^-1               (the non-expansive transition),
// with A kept on chip: it goes from the MFMA accumulators through LDS into
// the inverse and never reaches HBM.  The same pass writes the V^T copy the
// softmax reads (every frame and the text block), from the V tiles it has in
// LDS anyway, so V is read from HBM once for both branches.
// [deepmagic blog "生成比播放還快：Video DeltaNet 用 11 秒產出 14 秒 768p 影片",
//  section 用兩條分支取代一條 (closed form S = (S̄ + B)(I + A)^-1, non-expansive);
//  PaperDaily "伯克利与Impossible视频生成" §四 (A holds the key correlation of
//  the spatial tokens of one frame; the (I + A) inverse couples them)]
//
// gfx950 design (bf16, d in {32, 64, 128}): one workgroup of 8 waves per
// (batch, head, slot); two workgroups per CU, so one streams its tiles while
// the other inverts.
//  * Tiles of 32 tokens go global -> LDS with 16-byte direct-to-LDS loads into
//    an XOR-swizzled [token][d] layout, four slots in a ring: tiles t+1 ..
//    t+3 are in flight while tile t is used, one barrier per tile.  beta*k is formed in
//    fp32 and split into bf16 hi + lo in registers, from the K fragment the
//    wave reads for its block column, so A = K^T (bK)_hi + K^T (bK)_lo and B
//    likewise with V (two bf16 MFMA passes; a single rounding of beta*k moves
//    the small eigen-directions of I + A on ill-conditioned key sets).  At
//    d = 128 a wave owns one block column (four 32 x 32 blocks of A or B).
//  * V^T: ds_read_b64_tr_b16 pairs give each lane 8 consecutive tokens of one
//    d, stored as 16 bytes into row d of the copy.
//  * Inverse: I + A is read from A's lower triangle (exactly symmetric) into
//    a 16 x 32 thread grid, (d/16) x (d/32) values per thread, and inverted
//    in place by the symmetric sweep (Gauss-Jordan on an SPD matrix, pivots
//    in order, all positive; sweeping every pivot leaves -(I + A)^-1).  With
//    w = M[k][.] / sqrt(M[k][k]) the update is m[i][j] -= w_i w_j, bitwise
//    symmetric; one pivot row broadcast through LDS per step.
//  * G is stored as two bf16 planes, hi and lo (hi + lo = G to 2^-16), the
//    operand format of the scan's three-pass products, so the scan converts
//    nothing per step.
#include "vdn_device.h"
#include "vdn_internal.h"

namespace vdn {

namespace {

template <int D>
__global__ void __launch_bounds__(512, 4)
vda_stats_kernel(const bf16* __restrict__ k, const bf16* __restrict__ v,
                 const bf16* __restrict__ tk, const bf16* __restrict__ tv,
                 const float* __restrict__ beta, bf16* __restrict__ Gp, float* __restrict__ Bout,
                 bf16* __restrict__ vt, int nl8, Geo g, int H, int nitems) {
  constexpr int BT = 32;                     // tokens per tile
  constexpr int NBUF = 4;                    // K / V / beta ring depth
  constexpr int AHEAD = NBUF - 1;            // tiles in flight past the one in use
  constexpr int KCH = D / 8;                 // 16-byte chunks per token row
  constexpr int TILE = BT * D * 2;
  constexpr int NW = 8, NT = 64 * NW;
  constexpr int NCH = BT * KCH;              // 16-byte chunks per operand tile
  constexpr int NLW = NCH >= NT ? NW : NCH / 64;   // waves that copy an operand tile
  constexpr int NI = NCH >= NT ? NCH / NT : 1;     // copies per lane per operand
  static_assert(NCH % 64 == 0 && (NCH < NT || NCH % NT == 0), "copy split");
  constexpr int NB = D / 32;
  constexpr int NBLK = 2 * NB * NB;          // 32 x 32 blocks of A and B
  constexpr int BLK_PER_WAVE = NBLK >= NW ? NBLK / NW : 1;
  constexpr int ABYTES = D * D * 4;
  constexpr int BOFF = 2 * NBUF * TILE;      // after the K and V rings: beta ring
  constexpr int ROWOFF = ABYTES;             // sweep's pivot rows, after A
  constexpr int SMEM_T = BOFF + NBUF * BT * 4;
  constexpr int SMEM_S = ROWOFF + 2 * D * 4;
  constexpr int SMEM = SMEM_T > SMEM_S ? SMEM_T : SMEM_S;
  constexpr int NVT = (BT / 16) * NB;        // 16-token x 32-d transposed reads per tile
  constexpr int RB = D / 16, CB = D / 32;    // sweep: rows / columns per thread
  static_assert(RB == 2 * CB, "sweep grid");
  constexpr int BETA_WAVE = NW - 1;          // the wave that copies beta
  // One array for everything: with a second __shared__ array the compiler
  // orders LDS reads after every direct-to-LDS copy in flight.
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  char VDN_LDS* lds = (char VDN_LDS*)smem;
  float VDN_LDS* bring = (float VDN_LDS*)(lds + BOFF);
  float VDN_LDS* rowbuf = (float VDN_LDS*)(lds + ROWOFF);   // [2][D], sweep only

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int N = g.T * g.P;
  const int task = blockIdx.x;
  const int bh = task / nitems;
  const int b = bh / H, h = bh % H;
  const int idx = task % nitems;
  const int slot = vt ? idx : slot_of(g, idx, false);
  const bool text = slot == g.T;
  const bool stats = text || frame_needs_stats(g, slot);
  const int ntok = text ? g.L : g.P;
  const bf16* kb = text ? tk : k;
  const bf16* vb = text ? tv : v;
  const int tok0 = text ? 0 : slot * g.P;
  const int rows_total = text ? g.L : N;
  const float* bptr = beta + (size_t)b * (N + g.L) * H + h + (size_t)(text ? N : slot * g.P) * H;
  // V^T row d of this head; the slot's tokens start at column vcol0
  bf16* vtbh = vt ? vt + (size_t)bh * D * nl8 : nullptr;
  const int vcol0 = text ? N : slot * g.P;
  const int ntiles = (ntok + BT - 1) / BT;

  // 32 x 32 output blocks of this wave: matrix (0: A, rows from K; 1: B,
  // rows from V), block row bi, block column bj.  A wave keeps one block
  // column, so per 16 tokens it forms one column-side operand, beta k split
  // into bf16 hi + lo, in registers, and reads one row-side fragment per
  // block.
  auto block_of = [&](int i, int& mat, int& bi, int& bj) {
    if constexpr (NB == 4) {
      mat = wv >> 2;
      bi = i;
      bj = wv & 3;
      return true;
    } else {
      const int blk = wv * BLK_PER_WAVE + i;
      mat = blk / (NB * NB);
      bi = (blk / NB) % NB;
      bj = blk % NB;
      return blk < NBLK;
    }
  };
  int mat0, bi0, bj0;
  const bool has_blk = block_of(0, mat0, bi0, bj0);
  f32x16 acc[BLK_PER_WAVE];
#pragma unroll
  for (int i = 0; i < BLK_PER_WAVE; ++i) acc[i] = f32x16{};

  // Copies of tile t into ring slot t % NBUF: waves 0 .. NLW-1 NI 16-byte
  // chunks of K (statistics slots only) and of V per lane, rows past the
  // slot's end reading its first token; BETA_WAVE the tile's beta values (4
  // bytes per lane; lanes past the end write 0 instead).  Tile t+1 is issued
  // once every wave is done with tile t-1 and lands while tile t is used.
  const bool copier = sgpr(wv) < NLW;
  const bool beta_wave = stats && sgpr(wv) == BETA_WAVE;
  // this lane's chunks: row (token in the tile) and swizzled 16-byte chunk
  const uint32_t rstride = (uint32_t)H * D * 2;      // bytes between tokens
  uint32_t coff[NI];
  int crow[NI];
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int p = (ii * NLW + wv) * 64 + lane;
    crow[ii] = p / KCH;
    coff[ii] = (uint32_t)(((p % KCH) ^ swz<D>(crow[ii])) * 16);
  }
  const size_t slot_row0 = (size_t)b * rows_total + tok0;
  auto issue = [&](int t) {
    const int t0 = t * BT, sl = t % NBUF;
    const int last = sgpr(ntok - 1 - t0);           // rows past it read it
    if (beta_wave) {
      float VDN_LDS* bs = bring + sl * BT;
      const uint32_t ln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      if ((int)ln < BT) {
        if ((int)ln <= last) dma4s(sgpr_ptr(bptr + (size_t)t0 * H), ln * (uint32_t)(H * 4), bs);
        else bs[ln] = 0.f;
      }
    }
    if (copier) {
      const size_t e0 = ((slot_row0 + t0) * H + h) * D;
      const bf16* kbase = (const bf16*)sgpr_ptr(kb + e0);
      const bf16* vbase = (const bf16*)sgpr_ptr(vb + e0);
#pragma unroll
      for (int ii = 0; ii < NI; ++ii) {
        const int blk = ii * NLW + wv;
        const uint32_t off = (uint32_t)(crow[ii] < last ? crow[ii] : last) * rstride + coff[ii];
        if (stats) dma16s(kbase, off, lds + sl * TILE + blk * 1024);
        dma16s(vbase, off, lds + (NBUF + sl) * TILE + blk * 1024);
      }
    }
  };
  // Vector memory operations of this wave per tile (wave-uniform): its
  // copies (K and V chunks, beta) and its V^T stores.  They complete in
  // issue order, so "tile t has landed" is a wait until at most the
  // operations issued after tile t's copies are pending: the copies of the
  // (up to two) later tiles already issued and the stores of the last
  // min(t, 3) tiles.  Only the last tile can skip a store (rows past the
  // slot's end), and no wait follows it.
  const int ncopy = sgpr((copier ? (stats ? 2 : 1) * NI : 0) + (beta_wave ? 1 : 0));
  int nstore = 0;
  if (vtbh) {
#pragma unroll
    for (int u = 0; u < (NVT + NW - 1) / NW; ++u) nstore += u * NW + wv < NVT ? 1 : 0;
  }
  nstore = sgpr(nstore);
  for (int i = 0; i < AHEAD; ++i)
    if (i < ntiles) issue(i);
  for (int t = 0; t < ntiles; ++t) {
    const int t0 = t * BT, sl = t % NBUF;
    const char VDN_LDS* Kt = lds + sl * TILE;
    const char VDN_LDS* Vt = lds + (NBUF + sl) * TILE;
    wait_vmcnt(ncopy * ((t + 1 < ntiles) + (t + 2 < ntiles)) + nstore * (t < 3 ? t : 3));
    // tile t is in LDS for every wave, and every wave is done with tile t-1,
    // whose ring slot receives tile t+3
    lds_barrier();
    if (t + AHEAD < ntiles) issue(t + AHEAD);
    if (vtbh) {
      // lane l gets V[t0 + r0 + 8 (l / 32) + e][c0 + l % 32], e = 0..7: 16
      // bytes of V^T row c0 + l % 32
#pragma unroll
      for (int u = 0; u < (NVT + NW - 1) / NW; ++u) {
        const int call = u * NW + wv;
        if (call >= NVT) break;
        const int r0 = (call / NB) * 16, c0 = (call % NB) * 32;
        const bf16x8 val = lds_col8<D>(Vt, r0, c0, lane);
        const int tt = t0 + r0 + 8 * (lane >> 5);
        if (tt < ntok)
          *(bf16x8*)(vtbh + (size_t)(c0 + (lane & 31)) * nl8 + vcol0 + tt) = val;
      }
    }
    if (!stats || !has_blk) continue;
    const float VDN_LDS* bt_ = bring + sl * BT;
#pragma unroll
    for (int ks = 0; ks < BT / 16; ++ks) {
      // column side: beta k of 8 tokens in column bj0 * 32 + l % 32, split
      // into bf16 hi + lo
      const bf16x8 kc = lds_col8<D>(Kt, ks * 16, bj0 * 32, lane);
      const f32x4 b0 = *(const f32x4 VDN_LDS*)(bt_ + ks * 16 + 8 * (lane >> 5));
      const f32x4 b1 = *(const f32x4 VDN_LDS*)(bt_ + ks * 16 + 8 * (lane >> 5) + 4);
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16 x, y;
        split_bf16((float)kc[e] * (e < 4 ? b0[e] : b1[e - 4]), x, y);
        hi[e] = x;
        lo[e] = y;
      }
#pragma unroll
      for (int i = 0; i < BLK_PER_WAVE; ++i) {
        int mat, bi, bj;
        if (!block_of(i, mat, bi, bj)) continue;
        const bf16x8 a = lds_col8<D>(mat == 0 ? Kt : Vt, ks * 16, bi * 32, lane);
        acc[i] = mfma32(a, hi, acc[i]);
        acc[i] = mfma32(a, lo, acc[i]);
      }
    }
  }
  if (!stats) return;

  // B to HBM; A into LDS (fp32, row-major) for the inverse
  lds_barrier();                              // every wave is done with the tiles
  float VDN_LDS* Al = (float VDN_LDS*)smem;
  const size_t mat_off = ((size_t)bh * (g.T + 1) + slot) * D * D;
  const int half = lane >> 5;
#pragma unroll
  for (int i = 0; i < BLK_PER_WAVE; ++i) {
    int mat, bi, bj;
    if (!block_of(i, mat, bi, bj)) continue;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = bi * 32 + (j >> 2) * 8 + half * 4 + (j & 3);
      const int c = bj * 32 + (lane & 31);
      if (mat == 0) Al[r * D + c] = acc[i][j];
      else Bout[mat_off + (size_t)r * D + c] = acc[i][j];
    }
  }
  lds_barrier();

  const int ti = tid & 15, tc = tid >> 4;     // 16 x 32 thread grid
  const int r0 = ti * RB, c0 = tc * CB;
  float m[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int r = r0 + i, c = c0 + j;
      m[i][j] = Al[(r >= c ? r : c) * D + (r >= c ? c : r)] + (r == c ? 1.0f : 0.0f);
    }
  if (ti == 0) {
#pragma unroll
    for (int j = 0; j < CB; ++j) rowbuf[c0 + j] = m[0][j];
  }
  lds_barrier();
  for (int kb = 0; kb < 16; ++kb) {
#pragma unroll
    for (int km = 0; km < RB; ++km) {
      const int kk = kb * RB + km;
      const float VDN_LDS* rk = rowbuf + (kk & 1) * D;
      // pivots are diagonals of Schur complements of I + A: all >= 1
      const float sk = __builtin_amdgcn_rsqf(rk[kk]);
      float wi[RB], wc[CB];
#pragma unroll
      for (int i = 0; i < RB; ++i) wi[i] = rk[r0 + i] * sk;
#pragma unroll
      for (int j = 0; j < CB; ++j) wc[j] = rk[c0 + j] * sk;
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) m[i][j] = fmaf(-wi[i], wc[j], m[i][j]);
      if (ti == kb) {                         // row kk: M[kk][.] / M[kk][kk]
#pragma unroll
        for (int j = 0; j < CB; ++j) m[km][j] = wc[j] * sk;
      }
      if (tc == kb * 2 + km / CB) {           // column kk (local column km % CB)
#pragma unroll
        for (int i = 0; i < RB; ++i) m[i][km % CB] = wi[i] * sk;
        if (ti == kb) m[km][km % CB] = -sk * sk;
      }
      // the owners of row kk + 1 publish it for the next pivot
      if (km + 1 < RB) {
        if (ti == kb) {
#pragma unroll
          for (int j = 0; j < CB; ++j) rowbuf[((kk + 1) & 1) * D + c0 + j] = m[(km + 1) % RB][j];
        }
      } else if (kb + 1 < 16) {
        if (ti == kb + 1) {
#pragma unroll
          for (int j = 0; j < CB; ++j) rowbuf[((kk + 1) & 1) * D + c0 + j] = m[0][j];
        }
      }
      lds_barrier();
    }
  }
  // G = (I + A)^-1 = -M, as bf16 hi and lo planes
  bf16* gh = Gp + 2 * mat_off;
  bf16* gl = gh + (size_t)D * D;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    bf16 hv[CB], lv[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) split_bf16(-m[i][j], hv[j], lv[j]);
    const size_t o = (size_t)(r0 + i) * D + c0;
    if constexpr (CB == 4) {
      *(bf16x4*)(gh + o) = bf16x4{hv[0], hv[1], hv[2], hv[3]};
      *(bf16x4*)(gl + o) = bf16x4{lv[0], lv[1], lv[2], lv[3]};
    } else if constexpr (CB == 2) {
      *(bf16x2*)(gh + o) = bf16x2{hv[0], hv[1]};
      *(bf16x2*)(gl + o) = bf16x2{lv[0], lv[1]};
    } else {
      gh[o] = hv[0];
      gl[o] = lv[0];
    }
  }
}

template <int D>
hipError_t launch_d(const void* k, const void* v, const void* tk, const void* tv,
                    const float* beta, const vdn_layout_t& l, void* Gp, float* B, void* vt,
                    hipStream_t s) {
  const Geo g = make_geo(l);
  const int nitems = vt ? g.T + 1 : count_slots(g, false);
  const long grid = (long)l.batch * l.heads * nitems;
  const int nl8 = (g.T * g.P + g.L + 7) / 8 * 8;
  vda_stats_kernel<D><<<dim3((unsigned)grid), dim3(512), 0, s>>>(
      (const bf16*)k, (const bf16*)v, (const bf16*)tk, (const bf16*)tv, beta, (bf16*)Gp, B,
      (bf16*)vt, nl8, g, l.heads, nitems);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_vda_stats(const void* k, const void* v, const void* tk, const void* tv,
                            const float* beta, const vdn_layout_t& l, void* Gp, float* B,
                            void* vt, hipStream_t s) {
  if (l.dtype != VDN_BF16) return hipErrorNotSupported;
  if (vt && !softmax_uses_vt(l)) return hipErrorInvalidValue;
  switch (l.head_dim_k) {
    case 128: return launch_d<128>(k, v, tk, tv, beta, l, Gp, B, vt, s);
    case 64: return launch_d<64>(k, v, tk, tv, beta, l, Gp, B, vt, s);
    case 32: return launch_d<32>(k, v, tk, tv, beta, l, Gp, B, vt, s);
  }
  return hipErrorNotSupported;
}

}  // namespace vdn
