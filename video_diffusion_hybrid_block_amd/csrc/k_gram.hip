// Frame statistics of the VDA branch: for every frame the scans fold (and for
// the text block) A = sum_i beta_i k_i k_i^T, the key Gram of the frame, and
// B = sum_i beta_i v_i k_i^T, its write.
// [deepmagic blog "生成比播放還快：Video DeltaNet 用 11 秒產出 14 秒 768p 影片",
//  section 用兩條分支取代一條 (closed form with A and B);
//  PaperDaily "伯克利与Impossible视频生成" §四 (A holds the key correlation of
//  the spatial tokens of one frame)]
//
// gfx950 design (bf16, d in {32, 64, 128}): one workgroup (4 waves) per
// (batch, head, frame); token tiles of 64 stream global -> LDS with 16-byte
// direct-to-LDS loads.  beta*k is formed in fp32 and split into bf16 hi + lo
// (hi + lo = beta*k to 2^-16), so A = K^T (bK)_hi + K^T (bK)_lo and likewise B
// with V: two bf16 MFMA passes keep the statistics close to fp32 even for
// ill-conditioned, low-rank key sets, where a single bf16 rounding of
// sqrt(beta)*k perturbs the small eigen-directions of I + A beyond tolerance.
// All four operands are read with ds_read_b64_tr_b16 (tokens are the
// contraction index, d is contiguous in memory).
#include "vdn_device.h"
#include "vdn_internal.h"

namespace vdn {

namespace {

template <int D>
__global__ void __launch_bounds__(512)
gram_mfma_kernel(const bf16* __restrict__ k, const bf16* __restrict__ v,
                 const bf16* __restrict__ tk, const bf16* __restrict__ tv,
                 const float* __restrict__ beta, float* __restrict__ Aout,
                 float* __restrict__ Bout, Geo g, int H, int nslots, bool all_frames) {
  constexpr int BT = 64;                     // tokens per tile
  constexpr int KCH = D / 8;
  constexpr int TILE = BT * D * 2;
  constexpr int NW = 8;                      // waves per workgroup
  constexpr int NT = 64 * NW;
  constexpr int NI = BT * KCH / NT >= 1 ? BT * KCH / NT : 1;  // DMA instructions per thread
  constexpr int NB = D / 32;                 // 32-wide blocks per matrix side
  constexpr int NBLK = 2 * NB * NB;
  constexpr int BLK_PER_WAVE = NBLK >= NW ? NBLK / NW : 1;
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];
  __shared__ float bsh[BT];
  char VDN_LDS* lds = (char VDN_LDS*)smem;
  char VDN_LDS* Kt = lds;
  char VDN_LDS* Vt = lds + TILE;
  char VDN_LDS* Ht = lds + 2 * TILE;         // (beta k) hi
  char VDN_LDS* Lt = lds + 3 * TILE;         // (beta k) lo

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int N = g.T * g.P;
  const int task = blockIdx.x;
  const int bh = task / nslots;
  const int b = bh / H, h = bh % H;
  const int slot = slot_of(g, task % nslots, all_frames);
  const bool text = slot == g.T;
  const int ntok = text ? g.L : g.P;
  const bf16* kb = text ? tk : k;
  const bf16* vb = text ? tv : v;
  const int tok0 = text ? 0 : slot * g.P;
  const int rows_total = text ? g.L : N;
  const float* bptr = beta + (size_t)b * (N + g.L) * H + h + (size_t)(text ? N : slot * g.P) * H;

  f32x16 acc[BLK_PER_WAVE];
#pragma unroll
  for (int i = 0; i < BLK_PER_WAVE; ++i) acc[i] = f32x16{};

  for (int t0 = 0; t0 < ntok; t0 += BT) {
    __syncthreads();                          // previous tile fully consumed
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
      int blk = ii * NW + wv;
      if (blk * 64 >= BT * KCH) break;
      int p = blk * 64 + lane;
      int row = p / KCH, pch = p % KCH;
      int ch = pch ^ swz<D>(row);
      int tok = t0 + row < ntok ? t0 + row : 0;
      size_t off = ((size_t)(b * (size_t)rows_total + tok0 + tok) * H + h) * D + ch * 8;
      g2lds16(kb + off, Kt + blk * 1024);
      g2lds16(vb + off, Vt + blk * 1024);
    }
    if (threadIdx.x < BT) {
      int tk_ = t0 + threadIdx.x;
      bsh[threadIdx.x] = tk_ < ntok ? bptr[(size_t)tk_ * H] : 0.f;
    }
    wait_vmem();
    __syncthreads();
    // beta*k -> bf16 hi / lo, same swizzled layout as K
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
      if ((ii * NW + wv) * 64 >= BT * KCH) break;
      int p = (ii * NW + wv) * 64 + lane;
      int row = p / KCH;
      const float bt = bsh[row];
      bf16x8 kv = *(const bf16x8 VDN_LDS*)(Kt + p * 16);
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = (float)kv[e] * bt;
        bf16 a, c;
        split_bf16(x, a, c);
        hi[e] = a;
        lo[e] = c;
      }
      *(bf16x8 VDN_LDS*)(Ht + p * 16) = hi;
      *(bf16x8 VDN_LDS*)(Lt + p * 16) = lo;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BT / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < BLK_PER_WAVE; ++i) {
        const int blk = wv * BLK_PER_WAVE + i;  // 0..2*NB*NB-1
        if (blk >= NBLK) continue;
        const int mat = blk / (NB * NB);        // 0: A (rows from K), 1: B (rows from V)
        const int bi = (blk / NB) % NB, bj = blk % NB;
        bf16x8 a = lds_col8<D>(mat == 0 ? Kt : Vt, ks * 16, bi * 32, lane);
        bf16x8 bh_ = lds_col8<D>(Ht, ks * 16, bj * 32, lane);
        bf16x8 bl_ = lds_col8<D>(Lt, ks * 16, bj * 32, lane);
        acc[i] = mfma32(a, bh_, acc[i]);
        acc[i] = mfma32(a, bl_, acc[i]);
      }
    }
  }

  const size_t mat_off = (((size_t)b * H + h) * (g.T + 1) + slot) * D * D;
  const int half = lane >> 5;
#pragma unroll
  for (int i = 0; i < BLK_PER_WAVE; ++i) {
    const int blk = wv * BLK_PER_WAVE + i;
    if (blk >= NBLK) continue;
    const int mat = blk / (NB * NB);
    const int bi = (blk / NB) % NB, bj = blk % NB;
    float* dst = (mat == 0 ? Aout : Bout) + mat_off;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      int r = bi * 32 + (j >> 2) * 8 + half * 4 + (j & 3);
      int cidx = bj * 32 + (lane & 31);
      dst[(size_t)r * D + cidx] = acc[i][j];
    }
  }
}

// VALU path (float tensors, small head sizes): one workgroup per slot, one
// thread per (row, col) pair of A and of B, fp32 accumulation.
template <typename T, int D>
__global__ void __launch_bounds__(256)
gram_valu_kernel(const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ tk,
                 const T* __restrict__ tv, const float* __restrict__ beta,
                 float* __restrict__ Aout, float* __restrict__ Bout, Geo g, int H, int nslots,
                 bool all_frames) {
  const int N = g.T * g.P;
  const int task = blockIdx.x;
  const int bh = task / nslots;
  const int b = bh / H, h = bh % H;
  const int slot = slot_of(g, task % nslots, all_frames);
  const bool text = slot == g.T;
  const int ntok = text ? g.L : g.P;
  const T* kb = text ? tk : k;
  const T* vb = text ? tv : v;
  const int tok0 = text ? 0 : slot * g.P;
  const int rows_total = text ? g.L : N;
  const float* bptr = beta + (size_t)b * (N + g.L) * H + h + (size_t)(text ? N : slot * g.P) * H;
  const size_t mat_off = (((size_t)b * H + h) * (g.T + 1) + slot) * D * D;
  for (int idx = threadIdx.x; idx < D * D; idx += blockDim.x) {
    int r = idx / D, cc = idx % D;
    float a = 0.f, bb = 0.f;
    for (int t = 0; t < ntok; ++t) {
      size_t off = ((size_t)(b * (size_t)rows_total + tok0 + t) * H + h) * D;
      float bk = bptr[(size_t)t * H] * Elem<T>::to_f(kb[off + cc]);
      a = fmaf(Elem<T>::to_f(kb[off + r]), bk, a);
      bb = fmaf(Elem<T>::to_f(vb[off + r]), bk, bb);
    }
    Aout[mat_off + idx] = a;
    Bout[mat_off + idx] = bb;
  }
}

// fp32 path (d in {32, 64, 128}): the same statistics on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32, two tokens per MFMA), nothing rounded below
// fp32.  One workgroup of 8 waves per (batch, head, slot); K and V tiles of
// 32 tokens go global -> LDS with 16-byte direct-to-LDS copies, two stages.
// A wave owns block column bj of A (waves 0-3) or of B (waves 4-7), so per
// token pair it forms one beta*k operand and reuses it for every block row.
// At d = 128 the wave keeps all four block rows with O^T-style row order
// d = 4m + bi, which makes a lane's four row operands one 16-byte LDS read.
template <int D>
__global__ void __launch_bounds__(512)
gram_f32_kernel(const float* __restrict__ k, const float* __restrict__ v,
                const float* __restrict__ tk, const float* __restrict__ tv,
                const float* __restrict__ beta, float* __restrict__ Aout,
                float* __restrict__ Bout, Geo g, int H, int nslots, bool all_frames) {
  constexpr int BT = 32;                       // tokens per tile
  constexpr int NW = 8;
  constexpr int RB = D * 4;                    // row bytes
  constexpr int TILE = BT * RB;                // one operand tile
  constexpr int TBLK = TILE / 1024;            // 1 KB copy blocks per tile
  constexpr int NWH = NW / 2;
  constexpr int NIW = (TBLK + NWH - 1) / NWH;  // copies per wave per tile
  constexpr int NB = D / 32;
  constexpr int STAGE = 2 * TILE + BT * 4;     // K tile, V tile, beta
  static_assert(TILE % 1024 == 0, "tile blocks");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  char VDN_LDS* lds = (char VDN_LDS*)smem;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, ml = lane & 31;
  const int N = g.T * g.P;
  const int task = blockIdx.x;
  const int bh = task / nslots;
  const int b = bh / H, h = bh % H;
  const int slot = slot_of(g, task % nslots, all_frames);
  const bool text = slot == g.T;
  const int ntok = text ? g.L : g.P;
  const int tok0 = text ? 0 : slot * g.P;
  const int rows_total = text ? g.L : N;
  const float* bptr = beta + (size_t)b * (N + g.L) * H + h + (size_t)(text ? N : slot * g.P) * H;
  const size_t rstride = (size_t)H * D;                  // floats between tokens
  const float* xbase = (wv >= NWH ? (text ? tv : v) : (text ? tk : k)) +
                       ((size_t)b * rows_total + tok0) * rstride + (size_t)h * D;

  // blocks of this wave: matrix mat (0: A, rows from K; 1: B, rows from V),
  // block column bj, block rows bi0 .. bi0 + NBW - 1
  constexpr int NBW = NB == 4 ? 4 : 1;
  const int mat = NB == 1 ? wv : wv >> 2;
  const int bj = NB == 4 ? (wv & 3) : (NB == 2 ? (wv & 1) : 0);
  const int bi0 = NB == 2 ? ((wv >> 1) & 1) : 0;
  const bool active = NB != 1 || wv < 2;
  f32x16 acc[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) acc[i] = f32x16{};

  const int ntiles = (ntok + BT - 1) / BT;
  // copy i of a wave: block NWH i + wv % NWH of its tile (K for waves 0-3, V
  // for 4-7); lane slot jj = 64 blk + lane = row jj / (D / 4), chunk jj % (D / 4);
  // rows past the slot's end re-read its last token (their beta is 0)
  auto issue = [&](int t, int st) {
    char VDN_LDS* sb = lds + st * STAGE;
    const int t0 = t * BT;
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int blk = i * NWH + (wv & (NWH - 1));
      if (blk >= TBLK) break;
      const int jj = blk * 64 + lane;
      const int row = jj / (D / 4), ch = jj % (D / 4);
      const int tok = imin(t0 + row, ntok - 1);
      g2lds16(xbase + (size_t)tok * rstride + ch * 4, sb + (wv >= NWH ? TILE : 0) + blk * 1024);
    }
    // the last wave copies the tile's beta (lanes past the slot's end write 0)
    if (wv == NW - 1 && lane < BT) {
      float VDN_LDS* bs = (float VDN_LDS*)(sb + 2 * TILE);
      if (t0 + lane < ntok) dma4s(sgpr_ptr(bptr + (size_t)t0 * H), (uint32_t)lane * (uint32_t)(H * 4), bs);
      else bs[lane] = 0.f;
    }
  };
  if (ntiles > 0) issue(0, 0);
  for (int t = 0; t < ntiles; ++t) {
    const int st = t & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 1 < ntiles) issue(t + 1, st ^ 1);
    if (!active) continue;
    const char VDN_LDS* sb = lds + st * STAGE;
    const char VDN_LDS* Xt = sb + (mat == 0 ? 0 : TILE);   // row operand
    const float VDN_LDS* bs = (const float VDN_LDS*)(sb + 2 * TILE);
#pragma unroll
    for (int s2 = 0; s2 < BT / 2; ++s2) {
      const int row = 2 * s2 + half;
      // column operand: beta * k of token `row` at d = 32 bj + ml
      const float bk = bs[row] * *(const float VDN_LDS*)(sb + row * RB + (bj * 32 + ml) * 4);
      if constexpr (NB == 4) {
        const f32x4 x = *(const f32x4 VDN_LDS*)(Xt + row * RB + ml * 16);
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
          acc[bi] = __builtin_amdgcn_mfma_f32_32x32x2f32(x[bi], bk, acc[bi], 0, 0, 0);
      } else {
        const float x = *(const float VDN_LDS*)(Xt + row * RB + (bi0 * 32 + ml) * 4);
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(x, bk, acc[0], 0, 0, 0);
      }
    }
  }
  if (!active) return;
  // element e of block bi: row m = 8 (e / 4) + 4 half + e % 4 (d = 4m + bi at
  // d = 128, else 32 bi0 + m), column d = 32 bj + ml
  const size_t mat_off = (((size_t)b * H + h) * (g.T + 1) + slot) * D * D;
  float* dst = (mat == 0 ? Aout : Bout) + mat_off + bj * 32 + ml;
#pragma unroll
  for (int bi = 0; bi < NBW; ++bi)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = 8 * (e >> 2) + 4 * half + (e & 3);
      const int r = NB == 4 ? 4 * m + bi : bi0 * 32 + m;
      dst[(size_t)r * D] = acc[bi][e];
    }
}

template <int D>
hipError_t launch_f32(const void* k, const void* v, const void* tk, const void* tv,
                      const float* beta, const vdn_layout_t& l, bool all_frames, float* A,
                      float* B, hipStream_t s) {
  Geo g = make_geo(l);
  int nslots = count_slots(g, all_frames);
  long grid = (long)l.batch * l.heads * nslots;
  gram_f32_kernel<D><<<dim3((unsigned)grid), dim3(512), 0, s>>>(
      (const float*)k, (const float*)v, (const float*)tk, (const float*)tv, beta, A, B, g,
      l.heads, nslots, all_frames);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mfma(const void* k, const void* v, const void* tk, const void* tv,
                       const float* beta, const vdn_layout_t& l, bool all_frames, float* A,
                       float* B, hipStream_t s) {
  Geo g = make_geo(l);
  int nslots = count_slots(g, all_frames);
  long grid = (long)l.batch * l.heads * nslots;
  gram_mfma_kernel<D><<<dim3((unsigned)grid), dim3(512), 0, s>>>(
      (const bf16*)k, (const bf16*)v, (const bf16*)tk, (const bf16*)tv, beta, A, B, g, l.heads,
      nslots, all_frames);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_valu(const void* k, const void* v, const void* tk, const void* tv,
                       const float* beta, const vdn_layout_t& l, bool all_frames, float* A,
                       float* B, hipStream_t s) {
  Geo g = make_geo(l);
  int nslots = count_slots(g, all_frames);
  long grid = (long)l.batch * l.heads * nslots;
  gram_valu_kernel<T, D><<<dim3((unsigned)grid), dim3(256), 0, s>>>(
      (const T*)k, (const T*)v, (const T*)tk, (const T*)tv, beta, A, B, g, l.heads, nslots,
      all_frames);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gram(const void* k, const void* v, const void* tk, const void* tv,
                       const float* beta, const vdn_layout_t& l, bool all_frames, float* A,
                       float* B, hipStream_t s) {
  const int d = l.head_dim_k;
  if (l.dtype == VDN_BF16) {
    switch (d) {
      case 128: return launch_mfma<128>(k, v, tk, tv, beta, l, all_frames, A, B, s);
      case 64: return launch_mfma<64>(k, v, tk, tv, beta, l, all_frames, A, B, s);
      case 32: return launch_mfma<32>(k, v, tk, tv, beta, l, all_frames, A, B, s);
      case 16: return launch_valu<bf16, 16>(k, v, tk, tv, beta, l, all_frames, A, B, s);
    }
  } else {
    switch (d) {
      case 128: return launch_f32<128>(k, v, tk, tv, beta, l, all_frames, A, B, s);
      case 64: return launch_f32<64>(k, v, tk, tv, beta, l, all_frames, A, B, s);
      case 32: return launch_f32<32>(k, v, tk, tv, beta, l, all_frames, A, B, s);
      case 16: return launch_valu<float, 16>(k, v, tk, tv, beta, l, all_frames, A, B, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace vdn
