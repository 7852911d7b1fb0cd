// Backward pass of the softmax branch.  With P_ij = exp(s_ij - lse_i) the
// forward's attention weights (s_ij = scale q_i . k_j over the keys query i
// sees: its window and anchor frames and every text key), dO_s the gradient
// of O_soft and D_i = dO_s,i . O_soft,i:
//   dP_ij = dO_s,i . v_j,   dS_ij = P_ij (dP_ij - D_i),
//   dq_i += scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i,
//   dv_j = sum_i P_ij dO_s,i.
// The forward's merge backward stores -D_i, and dP_ij - D_i accumulates on
// the MFMA starting from it (no subtraction per score).
// The keys query frame t sees are the video tokens of its visible frames and
// the text; since frame t sees frame f exactly when f sees t, the queries that
// see key frame f are the tokens of f's own visible frames (text keys: every
// video query).
// [PaperDaily "伯克利与Impossible视频生成:14.3秒视频6.70秒去噪" §二 (window and
//  anchors, symmetric by construction); arXiv listing "Video DeltaNet", abstract
//  (text keeps softmax)]
//
// gfx950 design (bf16, d in {32, 64, 128}; P and L multiples of 8):
//  * dq kernel: the forward's work items (256 queries of one frame, 8 waves x
//    32 queries, one lane per query) and key walk.  Per 64-key tile:
//    S^T = K Q^T and dP^T = V dO_s^T on v_mfma_f32_32x32x16_bf16 (Q^T and
//    dO_s^T stay in registers), P^T = exp2(scale log2e S^T - lse) with the
//    forward's log-sum-exp (stored negated), dS^T lane-local, dq^T += K^T dS^T.
//    The scores are exact fp32 products of q and k as given, like the
//    training forward's, so P is consistent with its log-sum-exp.  K rows are
//    permuted inside 32-key blocks so the dS^T registers are the B operand of
//    the last product; K^T comes from a transposed copy.
//  * dk/dv kernel: 256 keys of one frame (or text) per workgroup, 8 waves x 32
//    keys, one lane per key (K^T, V^T in registers), walking the 64-query tiles
//    that see them twice: S = Q K^T, dv^T += dO_s^T P in one pass;
//    S, dP = dO_s V^T, dk^T += Q^T dS in the other, with Q / dO_s rows permuted
//    the same way and Q^T / dO_s^T from transposed copies; the tile's -lse and -D
//    ride along in one more direct-to-LDS block (-D starts the dP
//    accumulators).
//  * Tiles move with 16-byte direct-to-LDS loads into two buffers (the next
//    tile in flight during this one); rows padded to 2d+16 bytes and
//    transposed rows to 144 bytes so every ds_read_b128 is conflict-free.
#include "softmax_common.h"
#include "vdn_device.h"
#include "vdn_internal.h"

namespace vdn {

namespace {

template <int D>
struct BT {
  static constexpr int KCH = D / 8;                 // 16-byte chunks of a row
  static constexpr int KST = 2 * D + 16;            // padded row, bytes
  static constexpr int KSL = KST / 16;              // ... in 16-byte slots
  static constexpr int VST = 144, VSL = 9;          // transposed row: 64 positions + pad
  static constexpr int RBLK = KSL;                  // 1 KB blocks of a 64-row tile
  static constexpr int TBLK = (D * VSL + 63) / 64;  // ... of a D x 64 transposed tile
};

// Per-lane sources of chunk `lane` of block `blk` of a tile starting at
// sequence position p0, resolved row by row: a 64-row tile (row, chunk
// clamped; the pad slot reloads the last chunk) and a D x 64 transposed tile
// from a transposed copy xt[d][x] (x = video token, then N + text token).
// The pass that has registers to spare keeps these loop-invariant pointers;
// the others use the packed form below.
template <int D>
__device__ __forceinline__ const bf16* row_src(const KeyAddr& a, int p0, int blk, int lane,
                                               const bf16* vid, const bf16* txt, int HD) {
  const int slot = blk * 64 + lane;
  const int row = slot / BT<D>::KSL;
  const int ch = imin(slot % BT<D>::KSL, BT<D>::KCH - 1);
  const int r = key_row(a, p0 + row);
  const bool t = (r & 0x40000000) != 0;
  return (t ? txt : vid) + (size_t)(unsigned)((r & 0x3FFFFFFF) * HD) + ch * 8;
}
template <int D>
__device__ __forceinline__ const bf16* tr_src(const KeyAddr& a, int p0, int blk, int lane,
                                              const bf16* xt, int nl8, int N) {
  const int slot = blk * 64 + lane;
  const int d = imin(slot / BT<D>::VSL, D - 1);
  const int c = imin(slot % BT<D>::VSL, 7);
  const int r = key_row(a, p0 + c * 8);
  const int tok = (r & 0x3FFFFFFF) + ((r & 0x40000000) ? N : 0);
  return xt + (size_t)d * nl8 + tok;
}

// Per-lane part of a tile copy, packed in 32 bits so that nothing 64-bit per
// lane is loop-invariant (the compiler would hoist such pointers and, short
// of registers, spill them; a scratch reload then waits for every copy in
// flight).  The issue loops mark the packed words as rewritten each tile, so
// the offsets decoded from them are not hoisted either.  Row blocks: position of the lane's row in the tile (bits 0-7)
// and its 16-byte chunk (bits 8-15); transposed blocks: the position of the
// lane's 8-token chunk (bits 0-7) and its d row (bits 8-15).
template <int D>
__device__ __forceinline__ uint32_t row_pack(int blk, int lane) {
  const int slot = blk * 64 + lane;
  return (uint32_t)(slot / BT<D>::KSL) | ((uint32_t)imin(slot % BT<D>::KSL, BT<D>::KCH - 1) << 8);
}
template <int D>
__device__ __forceinline__ uint32_t tr_pack(int blk, int lane) {
  const int slot = blk * 64 + lane;
  return (uint32_t)(imin(slot % BT<D>::VSL, 7) * 8) | ((uint32_t)imin(slot / BT<D>::VSL, D - 1) << 8);
}
// Byte offsets from the tile's first row / first position when the tile lies
// in one key segment (rows HD elements apart; transposed rows nl8 apart).
__device__ __forceinline__ uint32_t row_boff(uint32_t pk, int HD) {
  return ((pk & 0xFFu) * (uint32_t)HD + (pk >> 8) * 8u) * 2u;
}
__device__ __forceinline__ uint32_t tr_boff(uint32_t pk, int nl8) {
  return ((pk >> 8) * (uint32_t)nl8 + (pk & 0xFFu)) * 2u;
}
// Per-lane sources for a tile that straddles segments (key rows resolved one
// by one): row blocks from the video or text tensor, transposed blocks from a
// transposed copy xt[d][x] (x = video token, then N + text token).
__device__ __forceinline__ const bf16* row_gen(const KeyAddr& a, int p0, uint32_t pk,
                                               const bf16* vid, const bf16* txt, int HD) {
  const int r = key_row(a, p0 + (int)(pk & 0xFFu));
  const bool t = (r & 0x40000000) != 0;
  return (t ? txt : vid) + (size_t)(unsigned)((r & 0x3FFFFFFF) * HD) + (pk >> 8) * 8;
}
__device__ __forceinline__ const bf16* tr_gen(const KeyAddr& a, int p0, uint32_t pk,
                                              const bf16* xt, int nl8, int N) {
  const int r = key_row(a, p0 + (int)(pk & 0xFFu));
  const int tok = (r & 0x3FFFFFFF) + ((r & 0x40000000) ? N : 0);
  return xt + (size_t)(pk >> 8) * nl8 + tok;
}
// Segment of virtual position kv (0..2 video, 3 text, 4 past the end).
__device__ __forceinline__ int seg_of(const KeyAddr& a, int kv) {
  return (int)(((uint32_t)(a.e0 - 1 - kv) >> 31) + ((uint32_t)(a.e1 - 1 - kv) >> 31) +
               ((uint32_t)(a.e2 - 1 - kv) >> 31) + ((uint32_t)(a.nkeys - 1 - kv) >> 31));
}

// ---------------------------------------------------------------------------
// dq kernel
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(512)
attn_bwd_dq_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                   const bf16* __restrict__ v, const bf16* __restrict__ tk,
                   const bf16* __restrict__ tv, const bf16* __restrict__ dos,
                   const float* __restrict__ nlse, const float* __restrict__ dvec,
                   const bf16* __restrict__ kt, int nl8, float* __restrict__ dq, Geo g, int B,
                   int H, int tpf, float c, float scale) {
  using T = BT<D>;
  constexpr int NW = 8, BN = 64;
  constexpr int NB = 2 * T::RBLK + T::TBLK;          // blocks per tile
  constexpr int NI = (NB + NW - 1) / NW;             // DMA instructions per wave
  constexpr int VOFF = T::RBLK * 1024, TOFF = 2 * T::RBLK * 1024;
  constexpr int BUFB = (NB + 1) * 1024;              // + one spare block
  __shared__ __attribute__((aligned(1024))) char smem[2 * BUFB];
  char VDN_LDS* lds = (char VDN_LDS*)smem;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int N = g.T * g.P;
  WorkItem w = decode_work_xcd(g, B, H, tpf);
  w.b = sgpr(w.b); w.h = sgpr(w.h); w.t = sgpr(w.t); w.tile = sgpr(w.tile);
  KeyAddr ka = key_addr(key_map(g, w.t));
  ka.e0 = sgpr(ka.e0); ka.e1 = sgpr(ka.e1); ka.e2 = sgpr(ka.e2); ka.nkeys = sgpr(ka.nkeys);
  ka.d0 = sgpr(ka.d0); ka.d1 = sgpr(ka.d1); ka.d2 = sgpr(ka.d2); ka.clamp_tok = sgpr(ka.clamp_tok);
  const int nkeys = ka.nkeys;

  const int qlocal = w.tile * (NW * 32) + wv * 32 + (lane & 31);
  const bool qvalid = qlocal < g.P;
  const int qrow = w.t * g.P + (qvalid ? qlocal : 0);
  const size_t qoff = ((size_t)(w.b * (size_t)N + qrow) * H + w.h) * D;
  bf16x8 qreg[D / 16], dreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qreg[ks] = *(const bf16x8*)(q + qoff + ks * 16 + half * 8);
    dreg[ks] = *(const bf16x8*)(dos + qoff + ks * 16 + half * 8);
  }
  const size_t ri = (size_t)(w.b * H + w.h) * N + qrow;
  const float nlq = nlse[ri];   // -lse
  // dvec holds -D: dP - D accumulates on the MFMA from a block of -D
  f32x16 ndq;
#pragma unroll
  for (int e = 0; e < 16; ++e) ndq[e] = dvec[ri];

  const int HD = H * D;
  const bf16* kbh = k + ((size_t)w.b * N * H + w.h) * D;
  const bf16* vbh = v + ((size_t)w.b * N * H + w.h) * D;
  const bf16* tkbh = tk + ((size_t)w.b * g.L * H + w.h) * D;
  const bf16* tvbh = tv + ((size_t)w.b * g.L * H + w.h) * D;
  const bf16* ktbh = kt + ((size_t)w.b * H + w.h) * D * (size_t)nl8;

  const int ntiles = sgpr((nkeys + BN - 1) / BN);
  // Copy i of this wave fills block i * NW + wv of the tile: K rows, V rows,
  // K^T, or the spare block (a reload of K block 0).
  uint32_t pk[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int blk = i * NW + wv;
    pk[i] = blk < T::RBLK ? row_pack<D>(blk, lane)
          : blk < 2 * T::RBLK ? row_pack<D>(blk - T::RBLK, lane)
          : blk < NB ? tr_pack<D>(blk - 2 * T::RBLK, lane) : row_pack<D>(0, lane);
  }
  auto issue = [&](int tile, int buf) {
    char VDN_LDS* bb = lds + buf * BUFB;
    const int p0 = imin(tile, ntiles - 1) * BN;
    // keep the offsets derived from pk inside the loop (see row_pack)
#pragma unroll
    for (int i = 0; i < NI; ++i) asm volatile("" : "+v"(pk[i]));
    const int s0 = seg_of(ka, p0), s1 = seg_of(ka, p0 + BN - 1);
    if (s0 == s1 && s0 < 4) {
      // the whole tile in one segment: wave-uniform bases
      const bool txt = s0 == 3;
      const int dl = s0 == 0 ? ka.d0 : (s0 == 1 ? ka.d1 : (s0 == 2 ? ka.d2 : -ka.e2));
      const size_t r0 = (size_t)(p0 + dl) * HD;
      const char* kb = sgpr_ptr((txt ? tkbh : kbh) + r0);
      const char* vb = sgpr_ptr((txt ? tvbh : vbh) + r0);
      const char* tb = sgpr_ptr(ktbh + (p0 + (txt ? N - ka.e2 : dl)));
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int blk = i * NW + wv;                 // uniform
        if (blk < T::RBLK) g2lds16(kb + row_boff(pk[i], HD), bb + blk * 1024);
        else if (blk < 2 * T::RBLK) g2lds16(vb + row_boff(pk[i], HD), bb + blk * 1024);
        else if (blk < NB) g2lds16(tb + tr_boff(pk[i], nl8), bb + blk * 1024);
        else g2lds16(kb + row_boff(pk[i], HD), bb + NB * 1024);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int blk = i * NW + wv;                   // uniform
      const bf16* src;
      if (blk < T::RBLK) src = row_gen(ka, p0, pk[i], kbh, tkbh, HD);
      else if (blk < 2 * T::RBLK) src = row_gen(ka, p0, pk[i], vbh, tvbh, HD);
      else if (blk < NB) src = tr_gen(ka, p0, pk[i], ktbh, nl8, N);
      else src = row_gen(ka, p0, pk[i], kbh, tkbh, HD);
      g2lds16(src, bb + (blk < NB ? blk : NB) * 1024);
    }
  };

  const int rread = perm32(lane & 31) * T::KST + half * 16;
  const int tread = TOFF + (lane & 31) * T::VST + half * 16;
  const bool partial = (nkeys & (BN - 1)) != 0;
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  issue(0, 0);
  for (int it = 0; it < ntiles; ++it) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 1 < ntiles) issue(it + 1, (it + 1) & 1);
    const char VDN_LDS* bb = lds + (it & 1) * BUFB;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        kf[ks] = *(const bf16x8 VDN_LDS*)(bb + rread + kb * 32 * T::KST + ks * 32);
        vf[ks] = *(const bf16x8 VDN_LDS*)(bb + VOFF + rread + kb * 32 * T::KST + ks * 32);
      }
      s[kb] = f32x16{};
      dp[kb] = ndq;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        s[kb] = mfma32(kf[ks], qreg[ks], s[kb]);
        dp[kb] = mfma32(vf[ks], dreg[ks], dp[kb]);
      }
    }
    if (partial && it == ntiles - 1) {
      const int lim = sgpr(nkeys - it * BN) - half * 8;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (kb * 32 + ((j >> 3) << 4) + (j & 7) >= lim) s[kb][j] = -INFINITY;
    }
    bf16x8 pk[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = fast_exp2(fmaf(s[kb][j], c, nlq));
        pk[kb * 2 + (j >> 3)][j & 7] = (bf16)(p * dp[kb][j]);
      }
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 tf = *(const bf16x8 VDN_LDS*)(bb + tread + db * 32 * T::VST + sp * 32);
        acc[db] = mfma32(tf, pk[sp], acc[db]);
      }
  }
  if (qvalid) {
    float* row = dq + qoff;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = db * 32 + jj * 8 + half * 4;
        f32x4 o = *(const f32x4*)(row + d);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = fmaf(scale, acc[db][jj * 4 + e], o[e]);
        *(f32x4*)(row + d) = o;
      }
  }
}

// ---------------------------------------------------------------------------
// dk / dv kernel
// ---------------------------------------------------------------------------
// Two passes over the query tiles, 8 waves x 32 keys = 256 keys per
// workgroup, two waves per SIMD.  PASS 0 accumulates dv^T += dO_s^T P (needs
// Q rows, dO_s^T, nlse); PASS 1 dk^T += Q^T dS (Q rows, dO_s rows, Q^T, nlse, D).
// Both add to dk / dv, which already hold the statistics' part.
// Each pass holds one d x 32 accumulator per lane, so it fits two waves per
// SIMD, and every query tile it streams serves 256 keys.  (A single pass
// holding both accumulators needs one wave per SIMD and 128 keys per
// workgroup: it measured 47.7 ms at 768p against 36-37 ms for the two
// passes.)
template <int D, int PASS>
__global__ void __launch_bounds__(512)
attn_bwd_dkv2_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                     const bf16* __restrict__ v, const bf16* __restrict__ tk,
                     const bf16* __restrict__ tv, const bf16* __restrict__ dos,
                     const float* __restrict__ nlse, const float* __restrict__ dvec,
                     const bf16* __restrict__ qt, const bf16* __restrict__ dost, int nq8,
                     float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dtk,
                     float* __restrict__ dtv, Geo g, int B, int H, int tpk, int ntx, float c,
                     float scale) {
  using T = BT<D>;
  constexpr int NW = 8, BM = 64;
  // blocks: Q rows, [dO_s rows], transposed tile (dO_s^T or Q^T), nlse / D
  constexpr int DOFF = T::RBLK * 1024;
  constexpr int TOFF = (PASS == 0 ? 1 : 2) * T::RBLK * 1024;
  constexpr int SOFF = TOFF + T::TBLK * 1024;
  constexpr int NB = SOFF / 1024 + 1;
  constexpr int NI = (NB + NW - 1) / NW;
  constexpr int BUFB = (NB + 1) * 1024;
  __shared__ __attribute__((aligned(1024))) char smem[2 * BUFB];
  char VDN_LDS* lds = (char VDN_LDS*)smem;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int N = g.T * g.P;
  const int G = B * H;
  const int gi = sgpr((int)(blockIdx.x % G));
  const int j = sgpr((int)(blockIdx.x / G));
  const int b = gi / H, h = gi % H;
  const int na = (g.af ? 1 : 0) + ((g.al && !(g.af && g.T == 1)) ? 1 : 0);
  int f, tile;
  bool text;
  if (j < na * tpk) {
    text = false;
    f = (j / tpk == 0 && g.af) ? 0 : g.T - 1;
    tile = j % tpk;
  } else if (j < na * tpk + ntx) {
    text = true;
    f = -1;
    tile = j - na * tpk;
  } else {
    text = false;
    const int r = j - na * tpk - ntx;
    f = r / tpk + (g.af ? 1 : 0);
    tile = r % tpk;
  }
  f = sgpr(f);
  tile = sgpr(tile);
  KeyAddr qa;
  if (text) {
    qa.e0 = qa.e1 = qa.e2 = qa.nkeys = N;
    qa.d0 = qa.d1 = qa.d2 = 0;
    qa.clamp_tok = 0;
  } else {
    qa = key_addr(key_map(g, f));
    qa.nkeys = qa.e2;
  }
  const int nq = sgpr(qa.nkeys);
  const int nkr = text ? g.L : g.P;
  const int klocal = tile * (NW * 32) + wv * 32 + (lane & 31);
  const bool kvalid = klocal < nkr;
  const int krow = kvalid ? klocal : 0;
  const size_t koff = text ? ((size_t)(b * (size_t)g.L + krow) * H + h) * D
                           : ((size_t)(b * (size_t)N + (size_t)f * g.P + krow) * H + h) * D;
  bf16x8 kreg[D / 16], vreg[PASS == 1 ? D / 16 : 1];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    kreg[ks] = *(const bf16x8*)((text ? tk : k) + koff + ks * 16 + half * 8);
    if constexpr (PASS == 1) vreg[ks] = *(const bf16x8*)((text ? tv : v) + koff + ks * 16 + half * 8);
  }

  const int HD = H * D;
  const bf16* qbh = q + ((size_t)b * N * H + h) * D;
  const bf16* dbh = dos + ((size_t)b * N * H + h) * D;
  const bf16* trbh = (PASS == 0 ? dost : qt) + ((size_t)b * H + h) * D * (size_t)nq8;
  const float* lbh = nlse + (size_t)(b * H + h) * N;
  const float* dvbh = dvec + (size_t)(b * H + h) * N;

  const int ntiles = sgpr((nq + BM - 1) / BM);
  // Copy i of this wave fills block i * NW + wv: Q rows, [dO_s rows], the
  // transposed tile, nlse / D, or the spare block (a reload of Q block 0).
  uint32_t pk[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int blk = i * NW + wv;
    pk[i] = blk < T::RBLK ? row_pack<D>(blk, lane)
          : (PASS == 1 && blk < 2 * T::RBLK) ? row_pack<D>(blk - T::RBLK, lane)
          : blk < SOFF / 1024 ? tr_pack<D>(blk - TOFF / 1024, lane) : row_pack<D>(0, lane);
  }
  auto issue = [&](int tile_, int buf) {
    char VDN_LDS* bb = lds + buf * BUFB;
    const int p0 = imin(tile_, ntiles - 1) * BM;
    if constexpr (PASS == 0) {
      // one accumulator and no dO_s rows: registers to spare for per-lane
      // pointers (measured faster here than the packed form)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int blk = i * NW + wv;                 // uniform
        const void* src;
        int dst = blk * 1024;
        if (blk < T::RBLK) {
          src = row_src<D>(qa, p0, blk, lane, qbh, qbh, HD);
        } else if (blk < SOFF / 1024) {
          src = tr_src<D>(qa, p0, blk - TOFF / 1024, lane, trbh, nq8, N);
        } else if (blk < NB) {
          const int ch = lane & 15;
          const int tok = key_row(qa, p0 + ch * 4) & 0x3FFFFFFF;
          src = (((lane >> 4) & 1) ? dvbh : lbh) + tok;
        } else {
          src = row_src<D>(qa, p0, 0, lane, qbh, qbh, HD);
          dst = NB * 1024;
        }
        g2lds16(src, bb + dst);
      }
      return;
    }
    // keep the offsets derived from pk inside the loop (see row_pack)
#pragma unroll
    for (int i = 0; i < NI; ++i) asm volatile("" : "+v"(pk[i]));
    const int s0 = seg_of(qa, p0), s1 = seg_of(qa, p0 + BM - 1);
    if (s0 == s1 && s0 < 3) {
      // the whole query tile in one video segment: wave-uniform bases
      // token offset of the segment (a select between the struct's members
      // would be compiled into an indexed load from a stack copy)
      const int dl = (key_row(qa, p0) & 0x3FFFFFFF) - p0;
      const size_t r0 = (size_t)(p0 + dl) * HD;
      const char* qb = sgpr_ptr(qbh + r0);
      const char* db = sgpr_ptr(dbh + r0);
      const char* tb = sgpr_ptr(trbh + (p0 + dl));
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int blk = i * NW + wv;                 // uniform
        if (blk < T::RBLK) {
          g2lds16(qb + row_boff(pk[i], HD), bb + blk * 1024);
        } else if (PASS == 1 && blk < 2 * T::RBLK) {
          g2lds16(db + row_boff(pk[i], HD), bb + blk * 1024);
        } else if (blk < SOFF / 1024) {
          g2lds16(tb + tr_boff(pk[i], nq8), bb + blk * 1024);
        } else if (blk < NB) {
          const int tok = p0 + dl + (lane & 15) * 4;
          g2lds16((((lane >> 4) & 1) ? dvbh : lbh) + tok, bb + blk * 1024);
        } else {
          g2lds16(qb + row_boff(pk[i], HD), bb + NB * 1024);
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int blk = i * NW + wv;                   // uniform
      const void* src;
      if (blk < T::RBLK) {
        src = row_gen(qa, p0, pk[i], qbh, qbh, HD);
      } else if (PASS == 1 && blk < 2 * T::RBLK) {
        src = row_gen(qa, p0, pk[i], dbh, dbh, HD);
      } else if (blk < SOFF / 1024) {
        src = tr_gen(qa, p0, pk[i], trbh, nq8, N);
      } else if (blk < NB) {
        const int ch = lane & 15;
        const int tok = key_row(qa, p0 + ch * 4) & 0x3FFFFFFF;
        src = (((lane >> 4) & 1) ? dvbh : lbh) + tok;
      } else {
        src = row_gen(qa, p0, pk[i], qbh, qbh, HD);
      }
      g2lds16(src, bb + (blk < NB ? blk : NB) * 1024);
    }
  };

  const int rread = perm32(lane & 31) * T::KST + half * 16;
  const int tread = TOFF + (lane & 31) * T::VST + half * 16;
  const bool partial = (nq & (BM - 1)) != 0;
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  issue(0, 0);
  for (int it = 0; it < ntiles; ++it) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 1 < ntiles) issue(it + 1, (it + 1) & 1);
    const char VDN_LDS* bb = lds + (it & 1) * BUFB;
    if (partial && it == ntiles - 1) {
      // queries past the end read a negated log-sum-exp of -inf, so their P
      // (and dS) vanish without a per-score mask
      const int nv = nq - it * BM;
      if ((int)threadIdx.x < BM && (int)threadIdx.x >= nv)
        ((float VDN_LDS*)(lds + (it & 1) * BUFB + SOFF))[threadIdx.x] = -INFINITY;
      __syncthreads();
    }
    bf16x8 pk[4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s = f32x16{}, dp = f32x16{};
      if constexpr (PASS == 1) {
        // -D of the block's query rows (register jr: query qb*32 + 16 (jr/8)
        // + 8 half + jr%8): dP - D accumulates on the MFMA from it
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int q0 = qb * 32 + hh * 16 + half * 8;
          const f32x4 d0 = *(const f32x4 VDN_LDS*)(bb + SOFF + 256 + q0 * 4);
          const f32x4 d1 = *(const f32x4 VDN_LDS*)(bb + SOFF + 256 + q0 * 4 + 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dp[hh * 8 + e] = d0[e];
            dp[hh * 8 + 4 + e] = d1[e];
          }
        }
      }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 qf = *(const bf16x8 VDN_LDS*)(bb + rread + qb * 32 * T::KST + ks * 32);
        s = mfma32(qf, kreg[ks], s);
        if constexpr (PASS == 1) {
          const bf16x8 df = *(const bf16x8 VDN_LDS*)(bb + DOFF + rread + qb * 32 * T::KST + ks * 32);
          dp = mfma32(df, vreg[ks], dp);
        }
      }
      // register jr holds query qb*32 + 16*(jr/8) + 8*half + jr%8
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int q0 = qb * 32 + hh * 16 + half * 8;
        const f32x4 l0 = *(const f32x4 VDN_LDS*)(bb + SOFF + q0 * 4);
        const f32x4 l1 = *(const f32x4 VDN_LDS*)(bb + SOFF + q0 * 4 + 16);
        const float nl[8] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
        if constexpr (PASS == 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e) pk[qb * 2 + hh][e] = (bf16)fast_exp2(fmaf(s[hh * 8 + e], c, nl[e]));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = fast_exp2(fmaf(s[hh * 8 + e], c, nl[e]));
            pk[qb * 2 + hh][e] = (bf16)(p * dp[hh * 8 + e]);
          }
        }
      }
    }
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 tf = *(const bf16x8 VDN_LDS*)(bb + tread + db * 32 * T::VST + sp * 32);
        acc[db] = mfma32(tf, pk[sp], acc[db]);
      }
  }
  if (kvalid) {
    float* row = PASS == 0 ? (text ? dtv : dv) + koff : (text ? dtk : dk) + koff;
    const float sc = PASS == 0 ? 1.0f : scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = db * 32 + jj * 8 + half * 4;
        f32x4 o = *(const f32x4*)(row + d);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = fmaf(sc, acc[db][jj * 4 + e], o[e]);
        *(f32x4*)(row + d) = o;
      }
  }
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, const void* tk, const void* tv,
                    const void* dos, const float* nlse, const float* dvec, const void* kt,
                    const void* qt, const void* dost, const vdn_layout_t& l, float scale,
                    float* dq, float* dk, float* dv, float* dtk, float* dtv, hipStream_t s) {
  Geo g = make_geo(l);
  const int N = g.T * g.P;
  const float c = scale * kLog2e;
  const int tpf = (g.P + 255) / 256;
  const long grid_q = (long)l.batch * l.heads * g.T * tpf;
  const int nl8 = (N + g.L + 7) / 8 * 8;
  attn_bwd_dq_kernel<D><<<dim3((unsigned)grid_q), dim3(512), 0, s>>>(
      (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)tk, (const bf16*)tv,
      (const bf16*)dos, nlse, dvec, (const bf16*)kt, nl8, dq, g, l.batch, l.heads, tpf, c, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int tpk = (g.P + 255) / 256;
  const int ntx = (g.L + 255) / 256;
  const long grid_k = (long)l.batch * l.heads * ((long)g.T * tpk + ntx);
  const int nq8 = (N + 7) / 8 * 8;
  attn_bwd_dkv2_kernel<D, 0><<<dim3((unsigned)grid_k), dim3(512), 0, s>>>(
      (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)tk, (const bf16*)tv,
      (const bf16*)dos, nlse, dvec, (const bf16*)qt, (const bf16*)dost, nq8, dk, dv, dtk, dtv, g,
      l.batch, l.heads, tpk, ntx, c, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  attn_bwd_dkv2_kernel<D, 1><<<dim3((unsigned)grid_k), dim3(512), 0, s>>>(
      (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)tk, (const bf16*)tv,
      (const bf16*)dos, nlse, dvec, (const bf16*)qt, (const bf16*)dost, nq8, dk, dv, dtk, dtv, g,
      l.batch, l.heads, tpk, ntx, c, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* tk,
                           const void* tv, const void* dos, const float* nlse, const float* dvec,
                           const void* kt, const void* qt, const void* dost,
                           const vdn_layout_t& l, float scale, float* dq, float* dk, float* dv,
                           float* dtk, float* dtv, hipStream_t s) {
  switch (l.head_dim_k) {
    case 128: return launch_d<128>(q, k, v, tk, tv, dos, nlse, dvec, kt, qt, dost, l, scale, dq, dk, dv, dtk, dtv, s);
    case 64: return launch_d<64>(q, k, v, tk, tv, dos, nlse, dvec, kt, qt, dost, l, scale, dq, dk, dv, dtk, dtv, s);
    case 32: return launch_d<32>(q, k, v, tk, tv, dos, nlse, dvec, kt, qt, dost, l, scale, dq, dk, dv, dtk, dtv, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace vdn
