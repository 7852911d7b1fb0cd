// Softmax branch of the hybrid layer: for every video query, one softmax over
// the keys of its visible frames (own chunk +- window_chunks, plus the first
// and last frame; an anchor frame sees every frame) together with all text
// keys, times the matching values.
// [PaperDaily "伯克利与Impossible视频生成:14.3秒视频6.70秒去噪" §二;
//  arXiv listing "Video DeltaNet: ...", abstract: softmax is kept for every
//  interaction that involves text]
//
// gfx950 design (bf16, d in {32, 64, 128}):
//  * One workgroup (4 waves) per 128 query rows of one (batch, head, frame);
//    query tiles never straddle frames, so every row of a tile shares one key
//    set.  The key set is a list of <= 3 contiguous video token ranges plus
//    the text block, walked as one virtual sequence in tiles of 64 keys; only
//    the last tile is partial.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//    so each lane owns one query column: row max / sum need one exchange with
//    lane l^32 per tile instead of 32-lane reductions.  K rows are permuted
//    inside each 32-key block so that the score registers already form the
//    B operand of O^T += V^T P^T without any data movement.
//  * K and V tiles go global -> LDS with 16-byte direct-to-LDS loads into an
//    XOR-swizzled layout, double buffered; V is read transposed from its
//    natural [key][d] layout with ds_read_b64_tr_b16.
//  * exp2 with the scale * log2(e) folded into one FMA; fp32 statistics.
//  * Work order: anchor-frame tiles (the heaviest) first; with B*H a multiple
//    of 8 each XCD gets a fixed set of heads so K/V tiles are shared in its L2.
#include <cstdlib>
#include <type_traits>

#include "softmax_common.h"
#include "vdn_device.h"
#include "vdn_internal.h"

namespace vdn {

namespace {

template <int D, bool VTM>
__global__ void __launch_bounds__(256, 2)
softmax_mfma_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                    const bf16* __restrict__ v, const bf16* __restrict__ tk,
                    const bf16* __restrict__ tv, const bf16* __restrict__ vtg, int nl8,
                    bf16* __restrict__ o, Geo g, int B, int H, int tpf, float c) {
  constexpr int BM = 128, BN = 64;
  constexpr int KCH = D / 8;                         // 16-byte data chunks per row
  // LDS rows are padded (no XOR swizzle): with 64 banks, 16 consecutive K rows
  // read at one 16-byte column by ds_read_b128 fall on distinct banks, and
  // every read address is a per-lane base plus a compile-time offset.
  // V, natural layout (VTM = false): rows of one key, read transposed with
  // ds_read_b64_tr_b16 (4 rows x 64 bytes per half-wave hit distinct banks).
  // V^T layout (VTM = true, from the transposed copy): rows of one d, 64 keys
  // each, padded to 144 bytes, read with ds_read_b128 (about 3x the LDS
  // throughput of the transposed read on gfx950).
  constexpr int KST = 2 * D + 16;                    // K row stride, bytes
  constexpr int VST = VTM ? 144 : (D == 32 ? 64 : 2 * D + 64);   // V row stride, bytes
  constexpr int VROWS = VTM ? D : BN;
  constexpr int KSL = KST / 16, VSL = VST / 16;      // 16-byte slots per row
  constexpr int KT = BN * KST;
  constexpr int VSLOTS = VROWS * VSL;                // slots holding data or padding
  constexpr int VBLK = (VSLOTS + 63) / 64;           // 1 KB DMA blocks per V tile
  constexpr int VT = VBLK * 1024;
  constexpr int BUFB = KT + VT;                      // one K+V buffer
  constexpr int NIK = (KSL + 3) / 4, NIV = (VBLK + 3) / 4;  // DMA instructions per wave
  __shared__ __attribute__((aligned(1024))) char smem[2 * BUFB];
  char VDN_LDS* lds = (char VDN_LDS*)smem;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int half = lane >> 5;
  const int N = g.T * g.P;
  const WorkItem w = decode_work_xcd(g, B, H, tpf);
  const KeyMap km = key_map(g, w.t);
  const KeyAddr ka = key_addr(km);

  // Query rows of this wave (B operand of S^T = K Q^T, kept in registers).
  const int qlocal = w.tile * BM + wv * 32 + (lane & 31);
  const bool qvalid = qlocal < g.P;
  const int qrow = w.t * g.P + (qvalid ? qlocal : 0);
  const size_t qoff = ((size_t)(w.b * (size_t)N + qrow) * H + w.h) * D;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qreg[ks] = *(const bf16x8*)(q + qoff + ks * 16 + half * 8);

  const int HD = H * D;
  const bf16* kbh = k + ((size_t)w.b * N * H + w.h) * D;
  const bf16* vbh = v + ((size_t)w.b * N * H + w.h) * D;
  const bf16* tkbh = tk + ((size_t)w.b * g.L * H + w.h) * D;
  const bf16* tvbh = tv + ((size_t)w.b * g.L * H + w.h) * D;

  // Per-lane DMA slots: instruction i of this wave fills LDS slot
  // j = (4i + wv) * 64 + lane, i.e. row j / SLOTS, chunk j % SLOTS (pad slots
  // repeat the row's last chunk).  koff / voff: element offset of that chunk
  // relative to the row's token.
  int krow[NIK], kch[NIK], vrow[NIV], vch[NIV];
#pragma unroll
  for (int i = 0; i < NIK; ++i) {
    const int j = (i * 4 + wv) * 64 + lane;
    krow[i] = j / KSL;
    kch[i] = imin(j % KSL, KCH - 1) * 8;
  }
#pragma unroll
  for (int i = 0; i < NIV; ++i) {
    const int j = (i * 4 + wv) * 64 + lane;
    if constexpr (VTM) {
      // V^T slot: d row j / 9, 8-key chunk j % 9 (chunk 8 is padding)
      const bool pad = j >= VSLOTS;
      vrow[i] = pad ? 0 : j / VSL;
      vch[i] = pad ? 0 : imin(j % VSL, BN / 8 - 1) * 8;
    } else {
      vrow[i] = j / VSL;
      vch[i] = imin(j % VSL, KCH - 1) * 8;
    }
  }
  const bf16* vtbh = VTM ? vtg + ((size_t)w.b * H + w.h) * D * (size_t)nl8 : nullptr;

  auto seg_of = [=](int kv) {
    return (kv >= ka.e0) + (kv >= ka.e1) + (kv >= ka.e2) + (kv >= ka.nkeys);
  };
  auto issue_load = [=](int kb0, char VDN_LDS* kt) {
    char VDN_LDS* vt = kt + KT;
    const int s0 = seg_of(kb0), s1 = seg_of(kb0 + BN - 1);
    if (s0 == s1 && s0 < 4) {
      // whole tile inside one segment: token = kv + d (uniform)
      const bool txt = s0 == 3;
      const int d = s0 == 0 ? ka.d0 : (s0 == 1 ? ka.d1 : (s0 == 2 ? ka.d2 : -ka.e2));
      const size_t tok0 = (size_t)(kb0 + d) * HD;
      const bf16* kb = (txt ? tkbh : kbh) + tok0;
#pragma unroll
      for (int i = 0; i < NIK; ++i)
        if (i * 4 + wv < KSL) g2lds16(kb + (krow[i] * HD + kch[i]), kt + (i * 4 + wv) * 1024);
      if constexpr (VTM) {
        // V^T row d holds video tokens then text tokens: text token x sits
        // at column N + x
        const bf16* vb = vtbh + (kb0 + (txt ? N - ka.e2 : d));
#pragma unroll
        for (int i = 0; i < NIV; ++i)
          if (i * 4 + wv < VBLK) g2lds16(vb + (vrow[i] * nl8 + vch[i]), vt + (i * 4 + wv) * 1024);
      } else {
        const bf16* vb = (txt ? tvbh : vbh) + tok0;
#pragma unroll
        for (int i = 0; i < NIV; ++i)
          if (i * 4 + wv < VBLK) g2lds16(vb + (vrow[i] * HD + vch[i]), vt + (i * 4 + wv) * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NIK; ++i) {
        if (i * 4 + wv >= KSL) continue;
        const int r = key_row(ka, kb0 + krow[i]);
        const bool txt = (r & 0x40000000) != 0;
        const size_t off = (size_t)(unsigned)((r & 0x3FFFFFFF) * HD) + kch[i];
        g2lds16((txt ? tkbh : kbh) + off, kt + (i * 4 + wv) * 1024);
      }
#pragma unroll
      for (int i = 0; i < NIV; ++i) {
        if (i * 4 + wv >= VBLK) continue;
        if constexpr (VTM) {
          // 8-key chunk: all 8 keys lie in one segment (P and L are multiples of 8)
          const int r = key_row(ka, kb0 + vch[i]);
          const int tok = (r & 0x3FFFFFFF) + ((r & 0x40000000) ? N : 0);
          g2lds16(vtbh + ((size_t)vrow[i] * nl8 + tok), vt + (i * 4 + wv) * 1024);
        } else {
          const int r = key_row(ka, kb0 + vrow[i]);
          const bool txt = (r & 0x40000000) != 0;
          const size_t off = (size_t)(unsigned)((r & 0x3FFFFFFF) * HD) + vch[i];
          g2lds16((txt ? tvbh : vbh) + off, vt + (i * 4 + wv) * 1024);
        }
      }
    }
  };

  // Per-lane LDS read bases.  K (A operand of S^T): row perm32(l%32) of each
  // 32-key block, chunk 2*ks + half.  V (transposed reads, A operand of
  // O^T += V^T P^T): lane s of 16-lane group g addresses row 8*(g/2) + s/4,
  // columns 16*(g%2) + 4*(s%4) .. +3 of the 16-key step.
  const int kread = perm32(lane & 31) * KST + half * 16;
  const int gq = lane >> 4, sq = lane & 15;
  // V^T: lane reads row d = l%32 (+32 db), keys 16 sp + 8 half .. +7
  const int vread = VTM ? (lane & 31) * VST + half * 16
                        : (8 * (gq >> 1) + (sq >> 2)) * VST + (16 * (gq & 1) + 4 * (sq & 3)) * 2;

  float m_run = -1e30f, l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};

  const int ntiles = (km.nkeys + BN - 1) / BN;
  const int nfull = km.nkeys / BN;
  const bf16x2 ones2 = {(bf16)1.0f, (bf16)1.0f};

  // One 64-key tile: scores, online softmax, P V.  BUFC: LDS buffer (0/1,
  // compile time); MASKED: the partial last tile.
  auto tile = [&](int it, auto bufc, auto masked) {
    constexpr int bsel = decltype(bufc)::value;
    wait_vmem();
    __syncthreads();
    if (it + 1 < ntiles) issue_load((it + 1) * BN, lds + (1 - bsel) * BUFB);
    const char VDN_LDS* kt = lds + bsel * BUFB + kread;
    const char VDN_LDS* vt = lds + bsel * BUFB + KT + vread;

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = *(const bf16x8 VDN_LDS*)(kt + kb * 32 * KST + ks * 32);
        s[kb] = mfma32(a, qreg[ks], s[kb]);
      }
    }
    if constexpr (decltype(masked)::value) {
      const int base = it * BN;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = base + kb * 32 + ((j >> 3) << 4) + half * 8 + (j & 7);
          if (key >= km.nkeys) s[kb][j] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, s[0][j]);
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[1][j]);
    mx = xhalf_max(mx);
    // Lazy rescale: the exponent offset m_run only moves when some query's
    // max grows by more than 2^8 (in exp2 units); until then p <= 256, which
    // bf16 P and the fp32 sums carry exactly as well.
    if (__builtin_amdgcn_ballot_w64((mx - m_run) * c > 8.0f) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float corr = fast_exp2((m_run - m_new) * c);
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= corr;
      m_run = m_new;
    }
    const float mc = m_run * c;
    bf16x8 pk[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        pk[kb * 2 + (j >> 3)][j & 7] = (bf16)fast_exp2(fmaf(s[kb][j], c, -mc));
    // row sum of the rounded weights (the ones P V uses): 16 bf16 dot2
#pragma unroll
    for (int sp = 0; sp < 4; ++sp) {
      const bf16x2* p2 = (const bf16x2*)&pk[sp];
#pragma unroll
      for (int e = 0; e < 4; ++e) l_run = __builtin_amdgcn_fdot2_f32_bf16(p2[e], ones2, l_run, false);
    }
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        bf16x8 a;
        if constexpr (VTM) {
          a = *(const bf16x8 VDN_LDS*)(vt + db * 32 * VST + sp * 32);
        } else {
          const char VDN_LDS* pv = vt + sp * 16 * VST + db * 64;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 VDN_LDS*)pv);
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 VDN_LDS*)(pv + 4 * VST));
          a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        oacc[db] = mfma32(a, pk[sp], oacc[db]);
      }
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  issue_load(0, lds);
  int it = 0;
  for (; it + 2 <= nfull; it += 2) {
    tile(it, B0{}, std::false_type{});
    tile(it + 1, B1{}, std::false_type{});
  }
  if (it < nfull) {
    tile(it, B0{}, std::false_type{});
    ++it;
  }
  if (it < ntiles) {
    if (it & 1) tile(it, B1{}, std::true_type{});
    else tile(it, B0{}, std::true_type{});
  }

  const float inv = 1.0f / xhalf_sum(l_run);
  if (qvalid) {
    bf16* orow = o + qoff;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = db * 32 + jj * 8 + half * 4;
        bf16x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = (bf16)(oacc[db][jj * 4 + e] * inv);
        *(bf16x4*)(orow + d) = val;
      }
  }
}

// Plain VALU path for float tensors and head sizes without an MFMA path: one
// wave per 64 query rows of a frame, keys staged through LDS 32 at a time.
template <typename T, int D>
__global__ void __launch_bounds__(64)
softmax_valu_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                    const T* __restrict__ tk, const T* __restrict__ tv, T* __restrict__ o, Geo g,
                    int B, int H, int tpf, float scale) {
  constexpr int BN = 32;
  __shared__ float Ks[BN][D];
  __shared__ float Vs[BN][D];
  const int N = g.T * g.P;
  int i = blockIdx.x;
  int gi = i % (B * H), rest = i / (B * H);
  int b = gi / H, h = gi % H;
  int t = rest / tpf, tile = rest % tpf;
  KeyMap km = key_map(g, t);
  int ql = tile * 64 + threadIdx.x;
  bool valid = ql < g.P;
  int qrow = t * g.P + (valid ? ql : 0);
  size_t qoff = ((size_t)(b * (size_t)N + qrow) * H + h) * D;
  float qv[D], ov[D];
  for (int d = 0; d < D; ++d) {
    qv[d] = Elem<T>::to_f(q[qoff + d]) * scale;
    ov[d] = 0.f;
  }
  float m_run = -1e30f, l_run = 0.f;
  for (int kb = 0; kb < km.nkeys; kb += BN) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < BN * D; idx += 64) {
      int r = idx / D, d = idx % D;
      size_t off;
      bool txt = key_src(km, kb + r, b, h, H, N, g.L, D, off);
      Ks[r][d] = Elem<T>::to_f((txt ? tk : k)[off + d]);
      Vs[r][d] = Elem<T>::to_f((txt ? tv : v)[off + d]);
    }
    __syncthreads();
    int nk = km.nkeys - kb < BN ? km.nkeys - kb : BN;
    float s[BN];
    float mx = m_run;
    for (int j = 0; j < BN; ++j) {
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(qv[d], Ks[j][d], acc);
      s[j] = j < nk ? acc : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    float corr = __expf(m_run - mx);
    l_run *= corr;
    for (int d = 0; d < D; ++d) ov[d] *= corr;
    for (int j = 0; j < nk; ++j) {
      float p = __expf(s[j] - mx);
      l_run += p;
      for (int d = 0; d < D; ++d) ov[d] = fmaf(p, Vs[j][d], ov[d]);
    }
    m_run = mx;
  }
  if (valid) {
    float inv = 1.0f / l_run;
    for (int d = 0; d < D; ++d) o[qoff + d] = Elem<T>::from_f(ov[d] * inv);
  }
}

template <typename T, int D>
hipError_t launch_valu(const void* q, const void* k, const void* v, const void* tk,
                       const void* tv, const vdn_layout_t& l, float scale, void* o,
                       hipStream_t s) {
  Geo g = make_geo(l);
  int tpf = (g.P + 63) / 64;
  long grid = (long)l.batch * l.heads * g.T * tpf;
  softmax_valu_kernel<T, D><<<dim3((unsigned)grid), dim3(64), 0, s>>>(
      (const T*)q, (const T*)k, (const T*)v, (const T*)tk, (const T*)tv, (T*)o, g, l.batch,
      l.heads, tpf, scale);
  return hipGetLastError();
}

// Softmax kernel for the V^T path (P and L multiples of 8).
//  * 8 waves x 32 queries = 256 query rows per workgroup, one workgroup per
//    CU (two waves per SIMD): every K / V^T tile in LDS feeds 256 queries.
//  * 64-key tiles in a 3-deep LDS ring; the DMA for tile i+2 is issued while
//    tile i is processed.  A wave issues the same number of DMA instructions
//    (NIW or NIW - 1) every tile, so "tile i+1 landed" is one s_waitcnt
//    vmcnt on that count.
//  * All K fragments of a tile are read from LDS before its score MFMAs (the
//    next tile's copies are issued while they are in flight) and all V^T
//    fragments before the softmax VALU work, so LDS latency overlaps MFMA /
//    VALU work instead of stalling each MFMA pair.
//  * LDS rows: K padded to 2d+16 bytes, V^T (one d, 64 keys) to 144 bytes;
//    both read with ds_read_b128 at base + immediate, conflict-free.
//  * Inference modes: q is multiplied by scale * log2(e) and rounded to bf16
//    once per work item, and each score chain starts from -m (the query's
//    exponent offset) instead of 0, so the MFMAs leave s * scale * log2(e) - m
//    and the weights are one v_exp_f32 each: no FMA per score.  The rounding
//    of the scaled q perturbs each score by about 2^-9 of the size of its
//    terms: invisible at the scale of unit keys against N(0, 1) queries, and
//    up to 4x the layer's error against the oracle when q . k spans tens of
//    exp2 units (still a third of the bf16 bound).  The linear read R q uses q
//    as given (reloaded in the epilogue).  The training modes keep exact
//    fp32 scores, since their log-sum-exp drives the backward.
// MODE 0 writes the softmax branch O_soft; MODE 1 the merged output
// sigmoid(l0) O_soft + sigmoid(l1) RMSNorm(R q); MODE 2 the two gated branches
// side by side, o[b][n][0][h][:] = sigmoid(l0) O_soft and
// o[b][n][1][h][:] = sigmoid(l1) RMSNorm(R q), the input of the per-branch
// output projections.  MODE 3 (backward pass) takes the upstream gradient dO
// of the merged output instead and writes what the backward needs: the gate
// logits' gradients, dO_soft = sigmoid(l0) dO (bf16), the row statistics of
// the softmax (its log-sum-exp in exp2 units and D = dO_soft . O_soft, both
// negated) and the gradient of the linear read before RMSNorm.  MODE 4 writes
// the two gated branches of MODE 2 as MXFP8 codes and block scales (the
// activation operand of the FP8 output projection), quantized from the fp32
// values.  MODE 6 is MODE 1 with exact fp32 scores (the layer's output as the
// training forward computes it).
// MODE 5 (training forward) writes MODE 1's output and keeps, for a later
// backward, O_soft and n = RMSNorm(R q) in fp32 and per row the negated
// log-sum-exp and the RMS factor 1/r.
// Maximum of the 16 scores of one accumulator block: eight dependent
// v_max3_f32 in one asm statement (one statement per chain: as separate
// statements the compiler pads each with a wait state).
__device__ __forceinline__ float max16_raw(const f32x16& x) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3\n\t"
      "v_max3_f32 %0, %0, %4, %5\n\t"
      "v_max3_f32 %0, %0, %6, %7\n\t"
      "v_max3_f32 %0, %0, %8, %9\n\t"
      "v_max3_f32 %0, %0, %10, %11\n\t"
      "v_max3_f32 %0, %0, %12, %13\n\t"
      "v_max3_f32 %0, %0, %14, %15\n\t"
      "v_max_f32 %0, %0, %16"
      : "=&v"(r)
      : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]),
        "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]),
        "v"(x[14]), "v"(x[15]));
  return r;
}

template <int D, int MODE>
__global__ void __launch_bounds__(512)
softmax_vt_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                  const bf16* __restrict__ tk, const bf16* __restrict__ vtg, int nl8,
                  bf16* __restrict__ o, Geo g, int B, int H, int tpf, float c,
                  const float* __restrict__ R, const float* __restrict__ gates, float eps,
                  EpilogueIO bio) {
  constexpr int NW = 8, BM = 32 * NW, BN = 64, NBUF = 3;
  constexpr int KCH = D / 8;
  constexpr int KST = 2 * D + 16, KSL = KST / 16;    // K row stride (bytes), slots
  constexpr int VST = 144, VSL = 9;                  // V^T row: 64 keys + pad
  constexpr int KBLK = (BN * KSL + 63) / 64;         // 1 KB DMA blocks of the K tile
  constexpr int VBLK = (D * VSL + 63) / 64;          // ... of the V^T tile
  constexpr int NBLK = KBLK + VBLK;
  constexpr int NWH = NW / 2;                        // waves per half (K half, V^T half)
  constexpr int NIK = (KBLK + NWH - 1) / NWH, NIV = (VBLK + NWH - 1) / NWH;
  constexpr int NIW = NIK > NIV ? NIK : NIV;         // DMA instructions per wave per tile
  constexpr int VOFF = KBLK * 1024;
  constexpr int BUFB = (NBLK + 1) * 1024;            // + one dummy block
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * BUFB];
  char VDN_LDS* lds = (char VDN_LDS*)smem;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int N = g.T * g.P;
  WorkItem w = decode_work_xcd(g, B, H, tpf);
  w.b = sgpr(w.b); w.h = sgpr(w.h); w.t = sgpr(w.t); w.tile = sgpr(w.tile);
  const KeyMap km = key_map(g, w.t);
  // Segment bounds are workgroup-uniform: keep them in SGPRs so the per-tile
  // address logic runs on the scalar unit.
  KeyAddr ka = key_addr(km);
  ka.e0 = sgpr(ka.e0); ka.e1 = sgpr(ka.e1); ka.e2 = sgpr(ka.e2); ka.nkeys = sgpr(ka.nkeys);
  ka.d0 = sgpr(ka.d0); ka.d1 = sgpr(ka.d1); ka.d2 = sgpr(ka.d2); ka.clamp_tok = sgpr(ka.clamp_tok);
  const int nkeys = ka.nkeys;

  const int qlocal = w.tile * BM + wv * 32 + (lane & 31);
  const bool qvalid = qlocal < g.P;
  const int qrow = w.t * g.P + (qvalid ? qlocal : 0);
  const size_t qoff = ((size_t)(w.b * (size_t)N + qrow) * H + w.h) * D;
  // PS: the scores' B operand is q * c rounded to bf16 and each score chain
  // starts from -m (inference modes).  The training modes (3: merge
  // backward, 5: training forward) keep exact fp32 scores, s * c - m by one
  // FMA per score: their log-sum-exp feeds the backward, which recomputes
  // the weights from q and k as given.
  constexpr bool PS = MODE != 3 && MODE != 5 && MODE != 6;
  bf16x8 qreg[D / 16];   // the scores' B operand
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 x = *(const bf16x8*)(q + qoff + ks * 16 + half * 8);
    if constexpr (PS) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qreg[ks][e] = (bf16)((float)x[e] * c);
    } else {
      qreg[ks] = x;
    }
  }

  const int HD = H * D;
  const bf16* kbh = k + ((size_t)w.b * N * H + w.h) * D;
  const bf16* tkbh = tk + ((size_t)w.b * g.L * H + w.h) * D;
  const bf16* vtbh = vtg + ((size_t)w.b * H + w.h) * D * (size_t)nl8;

  // Waves 0..NWH-1 move the K tile and waves NWH.. the V^T tile, so each
  // wave's DMA base is uniform.  DMA i of a wave fills block NWH*i + (wv %
  // NWH) of its half; slots past the half's last block reload block 0's chunk
  // into the spare block.  offb[i]: byte offset of the lane's 16-byte chunk
  // from the tile's first token (one-segment tiles), 32-bit so the load takes
  // a scalar base plus a vector offset; ldsb[i]: LDS block (uniform).
  const bool vwave = wv >= NWH;
  // real DMA instructions of this wave per tile: NIW or NIW - 1 (no dummies)
  const int ndma = ((vwave ? VBLK : KBLK) - (wv & (NWH - 1)) + NWH - 1) / NWH;
  const bool full = ndma == NIW;
  uint32_t offb[NIW];
  int ldsb[NIW];
#pragma unroll
  for (int i = 0; i < NIW; ++i) {
    const int blk = i * NWH + (wv & (NWH - 1));
    if (!vwave) {
      const bool ok = blk < KBLK;
      const int jj = (ok ? blk : 0) * 64 + lane;
      offb[i] = (uint32_t)(imin(jj / KSL, BN - 1) * HD + imin(jj % KSL, KCH - 1) * 8) * 2u;
      ldsb[i] = sgpr(ok ? blk * 1024 : NBLK * 1024);
    } else {
      const bool ok = blk < VBLK;
      const int jj = (ok ? blk : 0) * 64 + lane;
      offb[i] = (uint32_t)(imin(jj / VSL, D - 1) * nl8 + imin(jj % VSL, BN / 8 - 1) * 8) * 2u;
      ldsb[i] = sgpr(ok ? VOFF + blk * 1024 : NBLK * 1024);
    }
  }
  // segment of key kv: number of segment ends <= kv (all values >= 0)
  auto seg_of = [=](int kv) {
    return (int)(((uint32_t)(ka.e0 - 1 - kv) >> 31) + ((uint32_t)(ka.e1 - 1 - kv) >> 31) +
                 ((uint32_t)(ka.e2 - 1 - kv) >> 31) + ((uint32_t)(ka.nkeys - 1 - kv) >> 31));
  };
  const int ntiles = sgpr((nkeys + BN - 1) / BN);
  auto issue = [=](int tile, int buf) {
    char VDN_LDS* bb = lds + buf * BUFB;
    const int kb0 = imin(tile, ntiles - 1) * BN;   // tiles past the end reload the last one
    const int s0 = seg_of(kb0), s1 = seg_of(kb0 + BN - 1);
    if (s0 == s1 && s0 < 4) {
      const bool txt = s0 == 3;
      const int dl = s0 == 0 ? ka.d0 : (s0 == 1 ? ka.d1 : (s0 == 2 ? ka.d2 : -ka.e2));
      const char* base = sgpr_ptr(vwave ? (const void*)(vtbh + (kb0 + (txt ? N - ka.e2 : dl)))
                                        : (const void*)((txt ? tkbh : kbh) + (size_t)(kb0 + dl) * HD));
#pragma unroll
      for (int i = 0; i < NIW; ++i)
        if (i < NIW - 1 || full) {
          // the first copy waits for the base (written by v_readfirstlane);
          // the others only for their M0 write
          if (i == 0) dma16s(base, offb[i], bb + ldsb[i]);
          else asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                            :: "v"(offb[i]), "s"(base),
                               "{m0}"(__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(bb + ldsb[i])))
                            : "memory");
        }
    } else {
      // tiles over a segment boundary (rare): the bases are re-read from
      // SGPRs here, so no VGPR copies of them stay live across the loop
      const bf16 *kbs = kbh, *tkbs = tkbh, *vtbs = vtbh;
      asm volatile("" : "+s"(kbs), "+s"(tkbs), "+s"(vtbs));
#pragma unroll
      for (int i = 0; i < NIW; ++i) {
        if (i == NIW - 1 && !full) break;
        const int blk = i * NWH + (wv & (NWH - 1));
        if (!vwave) {
          const int jj = (blk < KBLK ? blk : 0) * 64 + lane;
          const int r = key_row(ka, kb0 + imin(jj / KSL, BN - 1));
          const bool txt = (r & 0x40000000) != 0;
          const size_t eo = (size_t)(unsigned)((r & 0x3FFFFFFF) * HD) + imin(jj % KSL, KCH - 1) * 8;
          g2lds16((txt ? tkbs : kbs) + eo, bb + ldsb[i]);
        } else {
          const int jj = (blk < VBLK ? blk : 0) * 64 + lane;
          const int d = imin(jj / VSL, D - 1);
          const int r = key_row(ka, kb0 + imin(jj % VSL, BN / 8 - 1) * 8);   // 8 keys, one segment
          const int tok = (r & 0x3FFFFFFF) + ((r & 0x40000000) ? N : 0);
          g2lds16(vtbs + ((size_t)d * nl8 + tok), bb + ldsb[i]);
        }
      }
    }
  };

  const int kread = perm32(lane & 31) * KST + half * 16;
  const int vread = VOFF + (lane & 31) * VST + half * 16;
  const bool partial = (nkeys & (BN - 1)) != 0;

  // m_run: the query's exponent offset (PS: exp2 units, and minit holds
  // -m_run in every element, the first score MFMA's accumulator input;
  // otherwise score units, m_thr = m_run + 8 / c the lazy-rescale bound)
  float m_run = PS ? 0.f : -1e30f, m_thr = -1e30f, l_run = 0.f;
  f32x16 minit = {};
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  const bf16x2 ones2 = {(bf16)1.0f, (bf16)1.0f};

  // S^T = K Q^T for the tile in buffer buf: all K fragments (kreads, in the
  // order the MFMAs consume them), then the MFMAs (scores).  The loop issues
  // the next copies between the two, so their address work overlaps the LDS
  // reads (-0.9 % against copies first).  The fence at the start of soft_pv
  // keeps its V^T reads after the score MFMAs: hoisted into this phase, they
  // would leave too few registers to read all K fragments ahead.
  auto kreads = [&](int buf, bf16x8 (&kf)[2][D / 16]) {
    const char VDN_LDS* kt = lds + buf * BUFB + kread;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kf[kb][ks] = *(const bf16x8 VDN_LDS*)(kt + kb * 32 * KST + ks * 32);
  };
  auto scores = [&](const bf16x8 (&kf)[2][D / 16], f32x16 (&s)[2]) {
    // first step of both chains from minit, written as asm: from the builtin
    // the compiler ties one chain's accumulator to its input and copies minit
    // into it every tile (8 moves); the two products are independent and the
    // next MFMAs read their results as accumulator inputs, which needs no
    // wait states
    if constexpr (PS) {
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %2, %4, %5\n\t"
                   "v_mfma_f32_32x32x16_bf16 %1, %3, %4, %5\n\t"
                   "s_nop 1"
                   : "=&v"(s[0]), "=&v"(s[1])
                   : "v"(kf[0][0]), "v"(kf[1][0]), "v"(qreg[0]), "v"(minit));
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(kf[kb][0], qreg[0], f32x16{});
    }
#pragma unroll
    for (int ks = 1; ks < D / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(kf[kb][ks], qreg[ks], s[kb]);
  };
  // Online softmax of tile `it` (scores s, buffer buf) and O^T += V^T P^T.
  auto soft_pv = [&](int it, int buf, f32x16 (&s)[2]) {
    // V^T fragments, read while the softmax runs on the VALU (not before the
    // score MFMAs: the fence keeps their registers free for the K fragments)
    __builtin_amdgcn_sched_barrier(0);
    const char VDN_LDS* vt = lds + buf * BUFB + vread;
    bf16x8 vf[4][D / 32];
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) vf[sp][db] = *(const bf16x8 VDN_LDS*)(vt + db * 32 * VST + sp * 32);
    if (partial && it == ntiles - 1) {
      // keys past the end score -inf (computed here, not hoisted as masks)
      const int lim = sgpr(nkeys - it * BN) - half * 8;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (kb * 32 + ((j >> 3) << 4) + (j & 7) >= lim) s[kb][j] = -INFINITY;
    }
    // row max: two max3 chains over the 32 scores, then the partner half
    const float ma = max16_raw(s[0]), mb = max16_raw(s[1]);
    float mx = xhalf_max_raw(max_raw(ma, mb));
    // Lazy rescale: the exponent offset moves only when some query's max
    // passes it by more than 8 (exp2 units); until then p <= 256.  The first
    // tile sets it to the tile's max.
    bf16x8 pk[4];
    if constexpr (PS) {
      if (__builtin_amdgcn_ballot_w64(mx > 8.0f) != 0 || it == 0) {
        const float dl = it == 0 ? mx : fmaxf(mx, 0.f);
        const float corr = it == 0 ? 0.f : fast_exp2(-dl);
        l_run *= corr;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= corr;
        m_run += dl;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] -= dl;
#pragma unroll
        for (int j = 0; j < 16; ++j) minit[j] = -m_run;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) pk[kb * 2 + (j >> 3)][j & 7] = (bf16)fast_exp2(s[kb][j]);
    } else {
      if (__builtin_amdgcn_ballot_w64(mx > m_thr) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float corr = fast_exp2((m_run - m_new) * c);
        l_run *= corr;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= corr;
        m_run = m_new;
        m_thr = m_new + 8.0f / c;
      }
      const float mc = m_run * c;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) pk[kb * 2 + (j >> 3)][j & 7] = (bf16)fast_exp2(fmaf(s[kb][j], c, -mc));
    }
#pragma unroll
    for (int sp = 0; sp < 4; ++sp) {
      const bf16x2* p2 = (const bf16x2*)&pk[sp];
#pragma unroll
      for (int e = 0; e < 4; ++e) l_run = __builtin_amdgcn_fdot2_f32_bf16(p2[e], ones2, l_run, false);
    }
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] = mfma32(vf[sp][db], pk[sp], oacc[db]);
  };

  // Tile t sits in buffer t % NBUF.  At the top of iteration t, tile t has
  // landed (own DMAs: vmcnt; everyone's: the barrier) and every wave is done
  // with tile t-1, whose buffer then receives tile t+2.
  issue(0, 0);
  issue(1, 1);
  f32x16 s[2];
  for (int it = 0; it < ntiles; ++it) {
    if (full) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NIW) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NIW - 1) : "memory");
    __syncthreads();
    // the tile's K fragment reads first: the address work and copies of
    // tile it + 2 then run while they are in flight
    bf16x8 kf[2][D / 16];
    kreads(it % NBUF, kf);
    issue(it + 2, (it + 2) % NBUF);
    scores(kf, s);
    soft_pv(it, it % NBUF, s);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  const float inv = 1.0f / xhalf_sum(l_run);
  if constexpr (MODE == 0) {
    if (qvalid) {
      bf16* orow = o + qoff;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d = db * 32 + jj * 8 + half * 4;
          bf16x4 val;
#pragma unroll
          for (int e = 0; e < 4; ++e) val[e] = (bf16)(oacc[db][jj * 4 + e] * inv);
          *(bf16x4*)(orow + d) = val;
        }
    }
  } else {
    // Merge in registers: o = sigmoid(g0) o_soft + sigmoid(g1) RMSNorm(R q),
    // R = the summed VDA state this frame reads (slot nc for anchors).
    // R is staged once per workgroup as bf16 hi + lo rows in the (now idle)
    // ring memory; o_lin^T = R q^T takes q^T from the score B operand, so it
    // lands in the same registers layout as O^T.
    const float* Rs = R + ((size_t)(w.b * H + w.h) * (g.nc + 1) + (is_anchor(g, w.t) ? g.nc : w.t / g.C)) * D * D;
    char VDN_LDS* rh = lds;
    char VDN_LDS* rl = lds + D * KST;
    // all global loads of the epilogue first: gate logits and this thread's
    // share of R (NR chunks of 8 floats)
    const float2 gl = *(const float2*)(gates + ((size_t)(w.b * (size_t)N + qrow) * H + w.h) * 2);
    if constexpr (PS) {
      // reload the unscaled q (the asm keeps the compiler from reusing the
      // first load's registers across the loop)
      const bf16* qr = q;
      asm volatile("" : "+s"(qr));
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) qreg[ks] = *(const bf16x8*)(qr + qoff + ks * 16 + half * 8);
    }
    constexpr int NR = (D * D / 8 + NW * 64 - 1) / (NW * 64);
    float4 xr[NR][2];
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int i = imin(u * NW * 64 + (int)threadIdx.x, D * D / 8 - 1);
      xr[u][0] = *(const float4*)(Rs + i * 8);
      xr[u][1] = *(const float4*)(Rs + i * 8 + 4);
    }
    __syncthreads();                       // every wave is done with the ring
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int i = u * NW * 64 + threadIdx.x;
      if (i >= D * D / 8) break;
      const int r = (i * 8) / D, cc = (i * 8) % D;
      const float xv[8] = {xr[u][0].x, xr[u][0].y, xr[u][0].z, xr[u][0].w,
                           xr[u][1].x, xr[u][1].y, xr[u][1].z, xr[u][1].w};
      bf16x8 hv, lv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16 hi, lo;
        split_bf16(xv[e], hi, lo);
        hv[e] = hi;
        lv[e] = lo;
      }
      *(bf16x8 VDN_LDS*)(rh + r * KST + cc * 2) = hv;
      *(bf16x8 VDN_LDS*)(rl + r * KST + cc * 2) = lv;
    }
    __syncthreads();
    f32x16 lin[D / 32];
#pragma unroll
    for (int rb = 0; rb < D / 32; ++rb) {
      lin[rb] = f32x16{};
      const int ro = (rb * 32 + (lane & 31)) * KST + half * 16;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 ah = *(const bf16x8 VDN_LDS*)(rh + ro + ks * 32);
        const bf16x8 al = *(const bf16x8 VDN_LDS*)(rl + ro + ks * 32);
        lin[rb] = mfma32(ah, qreg[ks], lin[rb]);
        lin[rb] = mfma32(al, qreg[ks], lin[rb]);
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int rb = 0; rb < D / 32; ++rb)
#pragma unroll
      for (int j = 0; j < 16; ++j) ss = fmaf(lin[rb][j], lin[rb][j], ss);
    ss = xhalf_sum(ss);
    const float rinv = rsqrtf(ss * (1.0f / D) + eps);
    if constexpr (MODE == 3) {
      // Merge backward.  With s0, s1 the gate sigmoids, O_s = oacc * inv and
      // n = lin * rinv: dl0 = (dO . O_s) s0 (1 - s0), dl1 = (dO . n) s1 (1 - s1),
      // dO_s = s0 dO, and through RMSNorm (n = o / r, r = sqrt(mean(o^2) + eps))
      // do = (s1 dO - n (s1 dO . n) / d) / r.
      const float s0 = sigmoidf(gl.x), s1 = sigmoidf(gl.y);
      const bf16* dorow = bio.dO + qoff;
      bf16x4 dov[D / 32][4];
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) dov[db][jj] = *(const bf16x4*)(dorow + db * 32 + jj * 8 + half * 4);
      float dot0 = 0.f, dot1 = 0.f, dsum = 0.f;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float dv = (float)dov[db][jj][e];
            const float os = oacc[db][jj * 4 + e] * inv;
            dot0 = fmaf(dv, os, dot0);
            dot1 = fmaf(dv, lin[db][jj * 4 + e] * rinv, dot1);
            dsum = fmaf((float)(bf16)(s0 * dv), os, dsum);
          }
      dot0 = xhalf_sum(dot0);
      dot1 = xhalf_sum(dot1);
      dsum = xhalf_sum(dsum);
      const float nlse2 = -fmaf(m_run, c, __log2f(1.0f / inv));   // -lse
      if (qvalid) {
        bf16* dosrow = bio.dos + qoff;
        float* dlrow = bio.dlin + qoff;
        const float kn = s1 * dot1 * (1.0f / D);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int d = db * 32 + jj * 8 + half * 4;
            bf16x4 vs;
            f32x4 vl;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float dv = (float)dov[db][jj][e];
              vs[e] = (bf16)(s0 * dv);
              vl[e] = rinv * fmaf(-lin[db][jj * 4 + e] * rinv, kn, s1 * dv);
            }
            *(bf16x4*)(dosrow + d) = vs;
            *(f32x4*)(dlrow + d) = vl;
          }
        if (half == 0) {
          const size_t gi = ((size_t)(w.b * (size_t)N + qrow) * H + w.h) * 2;
          *(float2*)(bio.dgates + gi) = make_float2(dot0 * s0 * (1.0f - s0), dot1 * s1 * (1.0f - s1));
          const size_t ri = (size_t)(w.b * H + w.h) * N + qrow;
          bio.dvec[ri] = -dsum;              // -D: the backward's products start from it
          bio.nlse[ri] = nlse2;
        }
      }
      return;
    }
    const float g0 = sigmoidf(gl.x) * inv, g1 = sigmoidf(gl.y) * rinv;
    if constexpr (MODE == 5) {
      // Training forward: besides the merged output, keep what the merge
      // backward needs: O_s = oacc * inv and n = lin * rinv (fp32, the
      // layout of q), and per (b, h, token) the negated log-sum-exp in exp2
      // units and 1 / r.
      if (qvalid) {
        float* osrow = bio.o_soft + qoff;
        float* onrow = bio.o_lin + qoff;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int d = db * 32 + jj * 8 + half * 4;
            f32x4 vs, vn;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              vs[e] = oacc[db][jj * 4 + e] * inv;
              vn[e] = lin[db][jj * 4 + e] * rinv;
            }
            *(f32x4*)(osrow + d) = vs;
            *(f32x4*)(onrow + d) = vn;
          }
        if (half == 0) {
          const size_t ri = (size_t)(w.b * H + w.h) * N + qrow;
          bio.nlse[ri] = -fmaf(m_run, c, __log2f(1.0f / inv));
          bio.rinv[ri] = rinv;
        }
      }
    }
    if constexpr (MODE == 4) {
      // MXFP8 branches: block db of a branch holds d in [32 db, 32 db + 32)
      // of this head, 16 values in this lane and 16 in lane l ^ 32 (same
      // query, so both lanes share qvalid and the block maximum is one swap).
      const size_t row = (size_t)w.b * N + qrow;
      uint8_t* crow = (uint8_t*)o + row * (2 * H * D) + (size_t)w.h * D;
      uint8_t* srow = bio.mx_scales + row * (2 * H * D / 32) + w.h * (D / 32);
#pragma unroll
      for (int br = 0; br < 2; ++br) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          float x[16];
          float amax = 0.f;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            x[j] = br == 0 ? g0 * oacc[db][j] : g1 * lin[db][j];
            amax = fmaxf(amax, fabsf(x[j]));
          }
          const int X = mx_block_exp(xhalf_max(amax));
          if (qvalid) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              *(uint32_t*)(crow + br * H * D + db * 32 + jj * 8 + half * 4) =
                  mx_pack4(x[jj * 4], x[jj * 4 + 1], x[jj * 4 + 2], x[jj * 4 + 3], X);
            if (half == 0) srow[br * (H * D / 32) + db] = (uint8_t)(X + 127);
          }
        }
      }
      return;
    }
    if (qvalid) {
      if constexpr (MODE == 1 || MODE == 5 || MODE == 6) {
        bf16* orow = o + qoff;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int d = db * 32 + jj * 8 + half * 4;
            bf16x4 val;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              val[e] = (bf16)fmaf(g0, oacc[db][jj * 4 + e], g1 * lin[db][jj * 4 + e]);
            *(bf16x4*)(orow + d) = val;
          }
      } else {
        bf16* orow = o + ((size_t)(w.b * (size_t)N + qrow) * 2 * H + w.h) * D;
        bf16* lrow = orow + (size_t)H * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int d = db * 32 + jj * 8 + half * 4;
            bf16x4 vs, vl;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              vs[e] = (bf16)(g0 * oacc[db][jj * 4 + e]);
              vl[e] = (bf16)(g1 * lin[db][jj * 4 + e]);
            }
            *(bf16x4*)(orow + d) = vs;
            *(bf16x4*)(lrow + d) = vl;
          }
      }
    }
  }
}

// V^T copy for the softmax: vt[b][h][d][x] = value d of token x, with the
// T*P video tokens first, then the L text tokens, then zeros up to nl8 (a
// multiple of 8).  One workgroup per (b, h, 64 tokens), staged through LDS.
template <int D>
__global__ void __launch_bounds__(256)
vt_transpose_kernel(const bf16* __restrict__ v, const bf16* __restrict__ tv,
                    bf16* __restrict__ vt, int N, int L, int H, int nl8, int ntile) {
  constexpr int LDR = D + 2;                 // row stride (elements)
  __shared__ bf16 sm[64 * LDR];
  const int tile = blockIdx.x % ntile;
  const int bh = blockIdx.x / ntile;
  const int b = bh / H, h = bh % H;
  const int x0 = tile * 64;
  for (int i = threadIdx.x; i < 64 * (D / 8); i += 256) {
    const int r = i / (D / 8), c8 = (i % (D / 8)) * 8;
    const int x = x0 + r;
    bf16x8 val = {};
    if (x < N) val = *(const bf16x8*)(v + (((size_t)b * N + x) * H + h) * D + c8);
    else if (x < N + L) val = *(const bf16x8*)(tv + (((size_t)b * L + (x - N)) * H + h) * D + c8);
#pragma unroll
    for (int e = 0; e < 8; ++e) sm[r * LDR + c8 + e] = val[e];
  }
  __syncthreads();
  bf16* dst = vt + (size_t)bh * D * nl8;
  for (int i = threadIdx.x; i < D * 8; i += 256) {
    const int d = i / 8, c = i % 8;
    const int x = x0 + c * 8;
    if (x >= nl8) continue;
    bf16x8 val;
#pragma unroll
    for (int e = 0; e < 8; ++e) val[e] = sm[(c * 8 + e) * LDR + d];
    *(bf16x8*)(dst + (size_t)d * nl8 + x) = val;
  }
}

// Softmax for fp32 layouts on the fp32 matrix cores: v_mfma_f32_32x32x2_f32,
// fp32 operands and accumulation, so nothing is rounded below fp32.
//  * Same work items and key walk as the V^T kernel (8 waves x 32 queries,
//    64-key tiles, segments in SGPRs, multi-segment tiles addressed per row),
//    with K and V both in their natural [token][d] layout: K rows and V rows
//    of a tile go global -> LDS with 16-byte direct-to-LDS copies, rows
//    padded to 4d + 16 bytes, two stages (a tile's compute is ~16x longer
//    than in bf16, so one tile in flight hides the copies).
//  * Scores S^T = K Q^T, 2 d-values per MFMA: lane half h takes d in
//    [h d/2, (h + 1) d/2), so a lane's K fragment for four consecutive steps
//    is one 16-byte LDS read and its Q fragment 64 registers at d = 128.
//  * Inside a 32-key block, MFMA row m holds key 8 (m / 8) + 2 (m % 4) +
//    (m / 4) % 2: accumulator element e of lane half h is then key 2e + h,
//    exactly the B operand of step e of O^T += V^T P^T, so the
//    probabilities feed the second product in place.
//  * O^T row m of d-block db is d = (d/32) m + db, so the V^T operand of
//    one step for every block is one LDS read of d/32 consecutive floats of
//    a V row.
// MODE 0 writes O_soft (fp32; the merge follows as its own kernel); MODE 1
// the merged output sigmoid(l0) O_soft + sigmoid(l1) RMSNorm(R q), with
// o_lin^T = R q^T on the same MFMA from the query registers and R staged in
// the idle ring (its rows ordered like O^T's, so o_lin lands in O^T's
// register layout).
template <int D, int MODE>
__global__ void __launch_bounds__(512)
softmax_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                   const float* __restrict__ v, const float* __restrict__ tk,
                   const float* __restrict__ tv, float* __restrict__ o, Geo g, int B, int H,
                   int tpf, float c, const float* __restrict__ R,
                   const float* __restrict__ gates, float eps) {
  constexpr int NW = 8, BM = 32 * NW, BN = 64, NBUF = 2;
  constexpr int ND = D / 32;                         // 32-row blocks of O^T
  constexpr int DCH = D / 4;                         // 16-byte data chunks per row
  constexpr int RST = 4 * D + 16, RSL = RST / 16;    // row stride (bytes), slots
  constexpr int TBLK = (BN * RSL + 63) / 64;         // 1 KB copy blocks per operand tile
  constexpr int NBLK = 2 * TBLK;                     // K tile, then V tile
  constexpr int NWH = NW / 2;                        // waves per operand
  constexpr int NIW = (TBLK + NWH - 1) / NWH;        // copies per wave per tile
  constexpr int VOFF = TBLK * 1024;
  constexpr int BUFB = (NBLK + 1) * 1024;            // + one spare block
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * BUFB];
  char VDN_LDS* lds = (char VDN_LDS*)smem;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, ml = lane & 31;
  const int N = g.T * g.P;
  WorkItem w = decode_work_xcd(g, B, H, tpf);
  w.b = sgpr(w.b); w.h = sgpr(w.h); w.t = sgpr(w.t); w.tile = sgpr(w.tile);
  const KeyMap km = key_map(g, w.t);
  KeyAddr ka = key_addr(km);
  ka.e0 = sgpr(ka.e0); ka.e1 = sgpr(ka.e1); ka.e2 = sgpr(ka.e2); ka.nkeys = sgpr(ka.nkeys);
  ka.d0 = sgpr(ka.d0); ka.d1 = sgpr(ka.d1); ka.d2 = sgpr(ka.d2); ka.clamp_tok = sgpr(ka.clamp_tok);
  const int nkeys = ka.nkeys;

  const int qlocal = w.tile * BM + wv * 32 + ml;
  const bool qvalid = qlocal < g.P;
  const int qrow = w.t * g.P + (qvalid ? qlocal : 0);
  const size_t qoff = ((size_t)(w.b * (size_t)N + qrow) * H + w.h) * D;
  float qreg[D / 2];
#pragma unroll
  for (int j = 0; j < D / 8; ++j) {
    const f32x4 x = *(const f32x4*)(q + qoff + half * (D / 2) + 4 * j);
#pragma unroll
    for (int u = 0; u < 4; ++u) qreg[4 * j + u] = x[u];
  }

  const int HD = H * D;
  const size_t hoff = ((size_t)w.b * N * H + w.h) * D, thoff = ((size_t)w.b * g.L * H + w.h) * D;
  // waves 0 .. NWH-1 copy the K tile, the others the V tile (same rows)
  const bool vwave = wv >= NWH;
  const float* xbh = (vwave ? v : k) + hoff;
  const float* txbh = (vwave ? tv : tk) + thoff;
  const int ndma = (TBLK - (wv & (NWH - 1)) + NWH - 1) / NWH;   // NIW or NIW - 1
  const bool full = ndma == NIW;
  // copy i of a wave fills block NWH i + (wv % NWH) of its tile: lane slot
  // jj = 64 blk + lane is row jj / RSL, chunk jj % RSL (the pad slot and
  // slots past the last row repeat a real chunk into padding)
  uint32_t offb[NIW];
  int ldsb[NIW];
#pragma unroll
  for (int i = 0; i < NIW; ++i) {
    const int blk = i * NWH + (wv & (NWH - 1));
    const bool ok = blk < TBLK;
    const int jj = (ok ? blk : 0) * 64 + lane;
    offb[i] = (uint32_t)(imin(jj / RSL, BN - 1) * HD + imin(jj % RSL, DCH - 1) * 4) * 4u;
    ldsb[i] = sgpr(ok ? (vwave ? VOFF : 0) + blk * 1024 : NBLK * 1024);
  }
  auto seg_of = [=](int kv) {
    return (int)(((uint32_t)(ka.e0 - 1 - kv) >> 31) + ((uint32_t)(ka.e1 - 1 - kv) >> 31) +
                 ((uint32_t)(ka.e2 - 1 - kv) >> 31) + ((uint32_t)(ka.nkeys - 1 - kv) >> 31));
  };
  const int ntiles = sgpr((nkeys + BN - 1) / BN);
  auto issue = [=](int tile, int buf) {
    char VDN_LDS* bb = lds + buf * BUFB;
    const int kb0 = tile * BN;
    const int s0 = seg_of(kb0), s1 = seg_of(kb0 + BN - 1);
    if (s0 == s1 && s0 < 4) {
      const bool txt = s0 == 3;
      const int dl = s0 == 0 ? ka.d0 : (s0 == 1 ? ka.d1 : (s0 == 2 ? ka.d2 : -ka.e2));
      const char* base = sgpr_ptr((txt ? txbh : xbh) + (size_t)(kb0 + dl) * HD);
#pragma unroll
      for (int i = 0; i < NIW; ++i)
        if (i < NIW - 1 || full) g2lds16(base + offb[i], bb + ldsb[i]);
    } else {
#pragma unroll
      for (int i = 0; i < NIW; ++i) {
        if (i == NIW - 1 && !full) break;
        const int blk = i * NWH + (wv & (NWH - 1));
        const int jj = (blk < TBLK ? blk : 0) * 64 + lane;
        const int r = key_row(ka, kb0 + imin(jj / RSL, BN - 1));
        const bool txt = (r & 0x40000000) != 0;
        const size_t eo = (size_t)(unsigned)((r & 0x3FFFFFFF) * HD) + imin(jj % RSL, DCH - 1) * 4;
        g2lds16((txt ? txbh : xbh) + eo, bb + ldsb[i]);
      }
    }
  };

  const int krow = 8 * (ml >> 3) + 2 * (ml & 3) + ((ml >> 2) & 1);
  const int kread = krow * RST + half * (D / 2) * 4;
  const int vread = VOFF + half * RST + ml * ND * 4;
  const bool partial = (nkeys & (BN - 1)) != 0;
  const float thr = 8.0f / c;   // lazy-rescale margin in score units

  float m_run = -1e30f, m_thr = -1e30f, l_run = 0.f;
  f32x16 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = f32x16{};

  issue(0, 0);
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 1 < ntiles) issue(it + 1, buf ^ 1);
    // S^T for the tile's two 32-key blocks
    f32x16 s[2] = {f32x16{}, f32x16{}};
    const char VDN_LDS* kt = lds + buf * BUFB + kread;
#pragma unroll
    for (int j = 0; j < D / 8; ++j) {
      const f32x4 k0 = *(const f32x4 VDN_LDS*)(kt + 16 * j);
      const f32x4 k1 = *(const f32x4 VDN_LDS*)(kt + 32 * RST + 16 * j);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(k0[u], qreg[4 * j + u], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(k1[u], qreg[4 * j + u], s[1], 0, 0, 0);
      }
    }
    if (partial && it == ntiles - 1) {
      const int lim = sgpr(nkeys - it * BN) - half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kb * 32 + 2 * e >= lim) s[kb][e] = -INFINITY;
    }
    float mx = m_run;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; e += 2) mx = max3_raw(mx, s[kb][e], s[kb][e + 1]);
    mx = xhalf_max_raw(mx);
    // lazy rescale, as in the bf16 kernel: p <= 2^8 between rescales
    if (__builtin_amdgcn_ballot_w64(mx > m_thr) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float corr = fast_exp2((m_run - m_new) * c);
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < ND; ++db) oacc[db] *= corr;
      m_run = m_new;
      m_thr = m_new + thr;
    }
    const float mc = m_run * c;
    float la = 0.f, lb = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        s[kb][e] = fast_exp2(fmaf(s[kb][e], c, -mc));
        s[kb][e + 1] = fast_exp2(fmaf(s[kb][e + 1], c, -mc));
        la += s[kb][e];
        lb += s[kb][e + 1];
      }
    l_run += la + lb;
    // O^T += V^T P^T: step e of block kb is keys 32 kb + 2e (lane half 0)
    // and 32 kb + 2e + 1 (half 1)
    const char VDN_LDS* vt = lds + buf * BUFB + vread;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const char VDN_LDS* vr = vt + (kb * 32 + 2 * e) * RST;
        float va[ND];
        if constexpr (ND == 4) {
          const f32x4 x = *(const f32x4 VDN_LDS*)vr;
          va[0] = x[0]; va[1] = x[1]; va[2] = x[2]; va[3] = x[3];
        } else if constexpr (ND == 2) {
          typedef float f32x2 __attribute__((ext_vector_type(2)));
          const f32x2 x = *(const f32x2 VDN_LDS*)vr;
          va[0] = x[0]; va[1] = x[1];
        } else {
          va[0] = *(const float VDN_LDS*)vr;
        }
#pragma unroll
        for (int db = 0; db < ND; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[db], s[kb][e], oacc[db], 0, 0, 0);
      }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  float inv = 1.0f / xhalf_sum(l_run);
  float g1 = 0.f;
  f32x16 lin[ND];
  if constexpr (MODE == 1) {
    // R of the state this frame reads (slot nc for anchors) into the ring:
    // LDS row 32 db + m holds R row (d/32) m + db, rows padded to RST bytes
    const float* Rs = R + ((size_t)(w.b * H + w.h) * (g.nc + 1) + (is_anchor(g, w.t) ? g.nc : w.t / g.C)) * D * D;
    const float2 gl = *(const float2*)(gates + ((size_t)(w.b * (size_t)N + qrow) * H + w.h) * 2);
    constexpr int NRC = (D * D / 4 + NW * 64 - 1) / (NW * 64);   // 16-byte chunks of R per thread
    f32x4 xr[NRC];
#pragma unroll
    for (int u = 0; u < NRC; ++u)
      xr[u] = *(const f32x4*)(Rs + 4 * imin(u * NW * 64 + (int)threadIdx.x, D * D / 4 - 1));
    __syncthreads();                                  // every wave is done with the ring
#pragma unroll
    for (int u = 0; u < NRC; ++u) {
      const int ci = u * NW * 64 + threadIdx.x;
      if (ci >= D * D / 4) break;
      const int r = ci / (D / 4), c4 = ci % (D / 4);
      const int lr = (r % ND) * 32 + r / ND;
      *(f32x4 VDN_LDS*)(lds + lr * RST + c4 * 16) = xr[u];
    }
    __syncthreads();
    // o_lin^T block db = R[rows (d/32) m + db] q^T: the same d split of the
    // contraction as the scores (lane half h: d in [h d/2, (h + 1) d/2))
    float ss = 0.f;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      lin[db] = f32x16{};
      const char VDN_LDS* rr = lds + (db * 32 + ml) * RST + half * (D / 2) * 4;
#pragma unroll
      for (int j = 0; j < D / 8; ++j) {
        const f32x4 r4 = *(const f32x4 VDN_LDS*)(rr + 16 * j);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          lin[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(r4[u], qreg[4 * j + u], lin[db], 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) ss = fmaf(lin[db][e], lin[db][e], ss);
    }
    ss = xhalf_sum(ss);
    const float rinv = rsqrtf(ss * (1.0f / D) + eps);
    inv *= sigmoidf(gl.x);
    g1 = sigmoidf(gl.y) * rinv;
  }
  if (qvalid) {
    // element e of block db: O^T row m = 8 (e / 4) + 4 half + e % 4, d = ND m + db
    float* orow = o + qoff;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      float val[4 * ND];
#pragma unroll
      for (int el = 0; el < 4; ++el)
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const float x = oacc[db][e4 * 4 + el] * inv;
          val[el * ND + db] = MODE == 1 ? fmaf(g1, lin[db][e4 * 4 + el], x) : x;
        }
      float* dst = orow + ND * (8 * e4 + 4 * half);
#pragma unroll
      for (int u = 0; u < ND; ++u) *(f32x4*)(dst + 4 * u) = f32x4{val[4 * u], val[4 * u + 1], val[4 * u + 2], val[4 * u + 3]};
    }
  }
}

template <int D>
hipError_t launch_f32(const void* q, const void* k, const void* v, const void* tk, const void* tv,
                      const vdn_layout_t& l, float scale, void* o, hipStream_t s,
                      const float* R = nullptr, const float* gates = nullptr, float eps = 0.f) {
  Geo g = make_geo(l);
  const int tpf = (g.P + 255) / 256;
  const long grid = (long)l.batch * l.heads * g.T * tpf;
  if (R)
    softmax_f32_kernel<D, 1><<<dim3((unsigned)grid), dim3(512), 0, s>>>(
        (const float*)q, (const float*)k, (const float*)v, (const float*)tk, (const float*)tv,
        (float*)o, g, l.batch, l.heads, tpf, scale * kLog2e, R, gates, eps);
  else
    softmax_f32_kernel<D, 0><<<dim3((unsigned)grid), dim3(512), 0, s>>>(
        (const float*)q, (const float*)k, (const float*)v, (const float*)tk, (const float*)tv,
        (float*)o, g, l.batch, l.heads, tpf, scale * kLog2e, nullptr, nullptr, 0.f);
  return hipGetLastError();
}

// VDN_EXACT_SCORES=1 in the environment (read at every launch): the layer's
// fused softmax + merge forms its scores exactly in fp32, one FMA per score,
// instead of from q * scale * log2(e) rounded to bf16 (about 4 % slower at
// 768p; its output is then the training forward's, bit for bit).
bool exact_scores() {
  const char* e = getenv("VDN_EXACT_SCORES");
  return e && e[0] == '1';
}

template <int D>
hipError_t launch_mfma(const void* q, const void* k, const void* v, const void* tk,
                       const void* tv, const vdn_layout_t& l, float scale, void* o, void* ws,
                       const float* R, const float* gates, float eps, int mode, hipStream_t s,
                       const EpilogueIO& bio = EpilogueIO{}, bool vt_ready = false) {
  Geo g = make_geo(l);
  int tpf = (g.P + 127) / 128;
  long grid = (long)l.batch * l.heads * g.T * tpf;
  if (softmax_uses_vt(l)) {
    const int tpf2 = (g.P + 255) / 256;
    const long grid2 = (long)l.batch * l.heads * g.T * tpf2;
    const int N = g.T * g.P;
    const int nl8 = (N + g.L + 7) / 8 * 8;
    const int ntile = (nl8 + 63) / 64;
    if (!vt_ready) {
      vt_transpose_kernel<D><<<dim3((unsigned)(l.batch * l.heads * ntile)), dim3(256), 0, s>>>(
          (const bf16*)v, (const bf16*)tv, (bf16*)ws, N, g.L, l.heads, nl8, ntile);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (mode == 1 && exact_scores())
      softmax_vt_kernel<D, 6><<<dim3((unsigned)grid2), dim3(512), 0, s>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)tk, (const bf16*)ws, nl8, (bf16*)o, g,
          l.batch, l.heads, tpf2, scale * kLog2e, R, gates, eps, EpilogueIO{});
    else if (mode == 1)
      softmax_vt_kernel<D, 1><<<dim3((unsigned)grid2), dim3(512), 0, s>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)tk, (const bf16*)ws, nl8, (bf16*)o, g,
          l.batch, l.heads, tpf2, scale * kLog2e, R, gates, eps, EpilogueIO{});
    else if (mode == 2)
      softmax_vt_kernel<D, 2><<<dim3((unsigned)grid2), dim3(512), 0, s>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)tk, (const bf16*)ws, nl8, (bf16*)o, g,
          l.batch, l.heads, tpf2, scale * kLog2e, R, gates, eps, EpilogueIO{});
    else if (mode == 3)
      softmax_vt_kernel<D, 3><<<dim3((unsigned)grid2), dim3(512), 0, s>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)tk, (const bf16*)ws, nl8, nullptr, g,
          l.batch, l.heads, tpf2, scale * kLog2e, R, gates, eps, bio);
    else if (mode == 4)
      softmax_vt_kernel<D, 4><<<dim3((unsigned)grid2), dim3(512), 0, s>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)tk, (const bf16*)ws, nl8, (bf16*)o, g,
          l.batch, l.heads, tpf2, scale * kLog2e, R, gates, eps, bio);
    else if (mode == 5)
      softmax_vt_kernel<D, 5><<<dim3((unsigned)grid2), dim3(512), 0, s>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)tk, (const bf16*)ws, nl8, (bf16*)o, g,
          l.batch, l.heads, tpf2, scale * kLog2e, R, gates, eps, bio);
    else
      softmax_vt_kernel<D, 0><<<dim3((unsigned)grid2), dim3(512), 0, s>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)tk, (const bf16*)ws, nl8, (bf16*)o, g,
          l.batch, l.heads, tpf2, scale * kLog2e, nullptr, nullptr, 0.f, EpilogueIO{});
  } else {
    if (mode != 0) return hipErrorNotSupported;
    softmax_mfma_kernel<D, false><<<dim3((unsigned)grid), dim3(256), 0, s>>>(
        (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)tk, (const bf16*)tv,
        nullptr, 0, (bf16*)o, g, l.batch, l.heads, tpf, scale * kLog2e);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax(const void* q, const void* k, const void* v, const void* tk,
                          const void* tv, const vdn_layout_t& l, float scale, void* o, void* ws,
                          hipStream_t s) {
  const int d = l.head_dim_k;
  if (l.dtype == VDN_BF16) {
    switch (d) {
      case 128: return launch_mfma<128>(q, k, v, tk, tv, l, scale, o, ws, nullptr, nullptr, 0.f, 0, s);
      case 64: return launch_mfma<64>(q, k, v, tk, tv, l, scale, o, ws, nullptr, nullptr, 0.f, 0, s);
      case 32: return launch_mfma<32>(q, k, v, tk, tv, l, scale, o, ws, nullptr, nullptr, 0.f, 0, s);
      case 16: return launch_valu<bf16, 16>(q, k, v, tk, tv, l, scale, o, s);
    }
  } else {
    switch (d) {
      case 128: return launch_f32<128>(q, k, v, tk, tv, l, scale, o, s);
      case 64: return launch_f32<64>(q, k, v, tk, tv, l, scale, o, s);
      case 32: return launch_f32<32>(q, k, v, tk, tv, l, scale, o, s);
      case 16: return launch_valu<float, 16>(q, k, v, tk, tv, l, scale, o, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_transpose(const void* x, const void* tx, int B, int H, int D, int N, int L,
                            void* xt, hipStream_t s) {
  const int nl8 = (N + L + 7) / 8 * 8;
  const int ntile = (nl8 + 63) / 64;
  const dim3 grid((unsigned)(B * H * ntile));
  switch (D) {
    case 128:
      vt_transpose_kernel<128><<<grid, dim3(256), 0, s>>>((const bf16*)x, (const bf16*)tx, (bf16*)xt, N, L, H, nl8, ntile);
      break;
    case 64:
      vt_transpose_kernel<64><<<grid, dim3(256), 0, s>>>((const bf16*)x, (const bf16*)tx, (bf16*)xt, N, L, H, nl8, ntile);
      break;
    case 32:
      vt_transpose_kernel<32><<<grid, dim3(256), 0, s>>>((const bf16*)x, (const bf16*)tx, (bf16*)xt, N, L, H, nl8, ntile);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_softmax_merge_bwd(const void* q, const void* k, const void* v, const void* tk,
                                    const void* tv, const float* R, const float* gates,
                                    const vdn_layout_t& l, float scale, float eps,
                                    const EpilogueIO& bio, void* ws, hipStream_t s) {
  if (!softmax_merge_fusable(l)) return hipErrorNotSupported;
  switch (l.head_dim_k) {
    case 128: return launch_mfma<128>(q, k, v, tk, tv, l, scale, nullptr, ws, R, gates, eps, 3, s, bio);
    case 64: return launch_mfma<64>(q, k, v, tk, tv, l, scale, nullptr, ws, R, gates, eps, 3, s, bio);
    case 32: return launch_mfma<32>(q, k, v, tk, tv, l, scale, nullptr, ws, R, gates, eps, 3, s, bio);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_softmax_branches_mxfp8(const void* q, const void* k, const void* v,
                                         const void* tk, const void* tv, const float* R,
                                         const float* gates, const vdn_layout_t& l, float scale,
                                         float eps, void* codes, void* scales, void* ws,
                                         hipStream_t s, bool vt_ready) {
  if (!softmax_merge_fusable(l)) return hipErrorNotSupported;
  EpilogueIO io{};
  io.mx_scales = (uint8_t*)scales;
  switch (l.head_dim_k) {
    case 128: return launch_mfma<128>(q, k, v, tk, tv, l, scale, codes, ws, R, gates, eps, 4, s, io, vt_ready);
    case 64: return launch_mfma<64>(q, k, v, tk, tv, l, scale, codes, ws, R, gates, eps, 4, s, io, vt_ready);
    case 32: return launch_mfma<32>(q, k, v, tk, tv, l, scale, codes, ws, R, gates, eps, 4, s, io, vt_ready);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_softmax_merge_train(const void* q, const void* k, const void* v,
                                      const void* tk, const void* tv, const float* R,
                                      const float* gates, const vdn_layout_t& l, float scale,
                                      float eps, void* o, const EpilogueIO& io, void* ws,
                                      hipStream_t s) {
  if (!softmax_merge_fusable(l)) return hipErrorNotSupported;
  switch (l.head_dim_k) {
    case 128: return launch_mfma<128>(q, k, v, tk, tv, l, scale, o, ws, R, gates, eps, 5, s, io);
    case 64: return launch_mfma<64>(q, k, v, tk, tv, l, scale, o, ws, R, gates, eps, 5, s, io);
    case 32: return launch_mfma<32>(q, k, v, tk, tv, l, scale, o, ws, R, gates, eps, 5, s, io);
  }
  return hipErrorInvalidValue;
}

bool softmax_merge_f32_fusable(const vdn_layout_t& l) {
  return l.dtype == VDN_F32 && l.head_dim_k >= 32;
}

hipError_t launch_softmax_merge_f32(const void* q, const void* k, const void* v, const void* tk,
                                    const void* tv, const float* R, const float* gates,
                                    const vdn_layout_t& l, float scale, float eps, void* o,
                                    hipStream_t s) {
  if (!softmax_merge_f32_fusable(l)) return hipErrorNotSupported;
  switch (l.head_dim_k) {
    case 128: return launch_f32<128>(q, k, v, tk, tv, l, scale, o, s, R, gates, eps);
    case 64: return launch_f32<64>(q, k, v, tk, tv, l, scale, o, s, R, gates, eps);
    case 32: return launch_f32<32>(q, k, v, tk, tv, l, scale, o, s, R, gates, eps);
  }
  return hipErrorInvalidValue;
}

bool softmax_merge_fusable(const vdn_layout_t& l) {
  return softmax_uses_vt(l) && l.head_dim_k >= 32;
}

hipError_t launch_softmax_merge(const void* q, const void* k, const void* v, const void* tk,
                                const void* tv, const float* R, const float* gates,
                                const vdn_layout_t& l, float scale, float eps, bool split, void* o,
                                void* ws, hipStream_t s, bool vt_ready) {
  if (!softmax_merge_fusable(l)) return hipErrorNotSupported;
  const int mode = split ? 2 : 1;
  const EpilogueIO none{};
  switch (l.head_dim_k) {
    case 128: return launch_mfma<128>(q, k, v, tk, tv, l, scale, o, ws, R, gates, eps, mode, s, none, vt_ready);
    case 64: return launch_mfma<64>(q, k, v, tk, tv, l, scale, o, ws, R, gates, eps, mode, s, none, vt_ready);
    case 32: return launch_mfma<32>(q, k, v, tk, tv, l, scale, o, ws, R, gates, eps, mode, s, none, vt_ready);
  }
  return hipErrorInvalidValue;
}

}  // namespace vdn
