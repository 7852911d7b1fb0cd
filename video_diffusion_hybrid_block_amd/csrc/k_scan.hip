// Bidirectional VDA state scan.  Both states start from half of the text write
// S_x = B_x (I + A_x)^-1; the forward state folds the non-anchor frames in
// ascending order, the backward state in descending order, each step being the
// frame-wise joint update S <- (alpha_f S + B_f)(I + A_f)^-1 = (alpha_f S + B_f) G_f.
// The state a chunk reads is the forward state before its window and the
// backward state after it; snapshots are taken at those points and summed.
// Anchor frames are never written (and do not decay the state).
// [PaperDaily "伯克利与Impossible视频生成:14.3秒视频6.70秒去噪" §三 (two states,
//  non-overlapping far regions, text written half into each), §四 pseudocode
//  (decay, frame correlation, joint solve, both directions);
//  deepmagic blog "生成比播放還快", section 用兩條分支取代一條 (×½ text write)]
//
// gfx950 design (bf16 layouts, d in {32, 64, 128}): the rows of S are
// independent under right-multiplication, so each (batch, head, direction)
// chain is split into d/32 workgroups of 32 rows.  A workgroup has d/32 waves;
// wave w computes the 32 x 32 block of columns 32w..32w+31 of the new state
// with v_mfma_f32_32x32x16_bf16 on a three-pass bf16 split of both operands
// (X_hi G_hi + X_hi G_lo + X_lo G_hi, relative error ~2^-16).  G is symmetric,
// so its B-operand columns are contiguous rows; G_f is copied to LDS with
// coalesced direct-to-LDS loads one step ahead.  The state lives in LDS
// between steps (the MFMA result is column-owned, the next A operand
// row-owned).
#include "vdn_device.h"
#include "vdn_internal.h"

namespace vdn {

namespace {

// Next frame a chain folds after frame f (-1 when done); f = -1 asks for the
// first one.  Forward: ascending non-anchor frames below fwd_scan_end;
// backward: descending non-anchor frames above bwd_scan_begin.
__device__ __forceinline__ int next_frame(const Geo& g, int dir, int f) {
  if (dir == 0) {
    const int fend = fwd_scan_end(g);
    int n = f + 1;
    while (n < fend && is_anchor(g, n)) ++n;
    return n < fend ? n : -1;
  }
  const int fbeg = bwd_scan_begin(g);
  int n = f < 0 ? g.T - 1 : f - 1;
  while (n > fbeg && is_anchor(g, n)) --n;
  return n > fbeg ? n : -1;
}

//
// fp32 layouts (F32): the same chains, steps and snapshots with the product
// on the fp32 matrix cores (v_mfma_f32_32x32x2_f32, fp32 operands and
// accumulation, no split).  X = aS + B is formed in place in the state rows
// (padded to d + 4 floats so the row-fragment reads are conflict-free); lane
// half h takes d in [h d/2, (h + 1) d/2), so four consecutive MFMA steps read
// one 16-byte chunk of an X row and of a G row.
template <int D, bool F32 = false>
__global__ void __launch_bounds__(2 * D)
scan_mfma_kernel(const float* __restrict__ G, const float* __restrict__ Bm,
                 const float* __restrict__ alpha, float* __restrict__ Sf, float* __restrict__ Sb,
                 Geo g, int H, float* __restrict__ states) {
  constexpr int NRB = D / 32;           // row blocks per chain = waves per workgroup
  constexpr int NT = 64 * NRB;
  constexpr int LDF = F32 ? D + 4 : D;  // fp32 state row stride (floats)
  constexpr int NCH = 32 * D / 8 / NT;  // 8-value chunks of X per thread per step
  constexpr int CPR = D / 4;            // 16-byte chunks per G row
  constexpr int GBYTES = D * D * 4;
  constexpr int NGI = GBYTES / 1024 / NRB;   // DMA instructions per wave per G
  static_assert(NCH >= 1 && NCH * 8 * NT == 32 * D, "X build split");
  static_assert(NGI * 1024 * NRB == GBYTES, "G copy split");
  // G_f is staged through LDS (two buffers, the next step's copy in flight
  // during this one) with 16-byte direct-to-LDS loads, one 1 KB block per
  // instruction; chunk c of row n sits at c ^ gsw(n) so the B-operand reads
  // (sixteen consecutive rows, one chunk) are conflict-free.
  // One LDS allocation for the G buffers, the state rows S and X = aS + B as
  // bf16 hi / lo: with separate __shared__ arrays the compiler cannot tell
  // the direct-to-LDS copies of G from the other LDS accesses and waits for
  // the next step's copy before writing X.
  __shared__ __attribute__((aligned(1024))) char smem[2 * GBYTES + 32 * LDF * 4 + (F32 ? 0 : 2 * 32 * D * 2)];
  char VDN_LDS* Gl = (char VDN_LDS*)smem;
  float VDN_LDS* S = (float VDN_LDS*)(smem + 2 * GBYTES);
  char VDN_LDS* Xh = (char VDN_LDS*)(smem + 2 * GBYTES + 32 * LDF * 4);
  char VDN_LDS* Xl = Xh + 32 * D * 2;
  auto gsw = [](int row) { return CPR >= 16 ? (row & 15) : ((row >> 1) & 7); };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, half = lane >> 5;
  // Workgroup i runs on XCD i % 8.  When the grid splits evenly, each XCD
  // gets whole chains, so the NRB row blocks of a chain (which all read the
  // same G_f and B_f every step) share one L2.
  int wid = blockIdx.x;
  if (gridDim.x % (8 * NRB) == 0) wid = (wid & 7) * (gridDim.x >> 3) + (wid >> 3);
  const int rb = wid % NRB;
  const int chain = wid / NRB;
  const int dir = chain & 1;
  const int bh = chain >> 1;
  const int b = bh / H, h = bh % H;
  const int row0 = rb * 32;
  const size_t mat = (size_t)D * D;
  const float* Gbh = G + (size_t)bh * (g.T + 1) * mat;
  const float* Bbh = Bm + (size_t)bh * (g.T + 1) * mat;
  float* snap = (dir == 0 ? Sf : Sb) + (size_t)bh * (g.nc + 1) * mat;
  const float* al = alpha + (size_t)b * g.T * H + h;

  // G of `slot` into LDS buffer bi: block blk = wv*NGI + i covers slots
  // 64*blk .. +63 (row slot / CPR, physical chunk slot % CPR).
  auto copy_g = [&](int slot, int bi) {
    const float* Gs = Gbh + (size_t)slot * mat;
#pragma unroll
    for (int i = 0; i < NGI; ++i) {
      const int blk = wv * NGI + i;
      const int sl = blk * 64 + lane;
      const int row = sl / CPR;
      const int ch = (sl % CPR) ^ gsw(row);
      g2lds16(Gs + (size_t)row * D + ch * 4, Gl + bi * GBYTES + blk * 1024);
    }
  };
  // This thread's share of the B rows: X chunks q = tid + i*NT, row q / (D/8),
  // columns 8*(q % (D/8)).
  float4 bcur[2 * NCH], bnxt[2 * NCH];
  auto load_b = [&](int slot, float4* br) {
    const float* Bs = Bbh + (size_t)slot * mat + (size_t)row0 * D;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = tid + i * NT;
      const float4* bp = (const float4*)(Bs + (q / (D / 8)) * D + (q % (D / 8)) * 8);
      br[2 * i] = bp[0];
      br[2 * i + 1] = bp[1];
    }
  };
  // S <- (a S + B) G, times `post`; G from LDS buffer bi (G symmetric: its
  // B-operand columns are rows).
  auto step = [&](float a, float post, int bi) {
    if constexpr (F32) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int q = tid + i * NT;
        const int r = q / (D / 8), c = (q % (D / 8)) * 8;
        f32x4 VDN_LDS* sp = (f32x4 VDN_LDS*)((float VDN_LDS*)S + r * LDF + c);
        const float4 b0 = bcur[2 * i], b1 = bcur[2 * i + 1];
        f32x4 s0 = sp[0], s1 = sp[1];
        s0[0] = fmaf(a, s0[0], b0.x); s0[1] = fmaf(a, s0[1], b0.y);
        s0[2] = fmaf(a, s0[2], b0.z); s0[3] = fmaf(a, s0[3], b0.w);
        s1[0] = fmaf(a, s1[0], b1.x); s1[1] = fmaf(a, s1[1], b1.y);
        s1[2] = fmaf(a, s1[2], b1.z); s1[3] = fmaf(a, s1[3], b1.w);
        sp[0] = s0;
        sp[1] = s1;
      }
      lds_barrier();
      const int ml = lane & 31;
      const int n = wv * 32 + ml;
      const int x = gsw(n);
      const char VDN_LDS* grow = Gl + bi * GBYTES + n * (4 * D);
      const float VDN_LDS* xrow = (const float VDN_LDS*)S + ml * LDF + half * (D / 2);
      f32x16 acc = f32x16{};
#pragma unroll
      for (int j = 0; j < D / 8; ++j) {
        const f32x4 g4 = *(const f32x4 VDN_LDS*)(grow + (((half * (D / 8) + j) ^ x) << 4));
        const f32x4 x4 = *(const f32x4 VDN_LDS*)(xrow + 4 * j);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x4[u], g4[u], acc, 0, 0, 0);
      }
      lds_barrier();                        // every wave is done reading X
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = (j >> 2) * 8 + half * 4 + (j & 3);
        S[r * LDF + wv * 32 + ml] = acc[j] * post;
      }
      lds_barrier();
      return;
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = tid + i * NT;
      const int r = q / (D / 8), c = (q % (D / 8)) * 8;
      const f32x4 s0 = *(const f32x4 VDN_LDS*)((const float VDN_LDS*)S + r * LDF + c);
      const f32x4 s1 = *(const f32x4 VDN_LDS*)((const float VDN_LDS*)S + r * LDF + c + 4);
      const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
      const float4 b0 = bcur[2 * i], b1 = bcur[2 * i + 1];
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      bf16x8 hv, lv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16 hi, lo;
        split_bf16(fmaf(a, sv[e], bv[e]), hi, lo);
        hv[e] = hi;
        lv[e] = lo;
      }
      const int off = swz_off<D>(r, c);
      *(bf16x8 VDN_LDS*)(Xh + off) = hv;
      *(bf16x8 VDN_LDS*)(Xl + off) = lv;
    }
    lds_barrier();
    const int n = wv * 32 + (lane & 31);
    const int x = gsw(n);
    const char VDN_LDS* grow = Gl + bi * GBYTES + n * (4 * D);
    // three independent accumulation chains: X_hi G_hi, X_hi G_lo, X_lo G_hi
    f32x16 acc = f32x16{}, acc1 = f32x16{}, acc2 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int c0 = 4 * ks + 2 * half;
      const f32x4 g0 = *(const f32x4 VDN_LDS*)(grow + ((c0 ^ x) << 4));
      const f32x4 g1 = *(const f32x4 VDN_LDS*)(grow + (((c0 + 1) ^ x) << 4));
      const float gv[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
      bf16x8 gh, gl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16 a_, c_;
        split_bf16(gv[e], a_, c_);
        gh[e] = a_;
        gl[e] = c_;
      }
      const bf16x8 ah = lds_row8<D>(Xh, lane & 31, ks * 2 + half);
      const bf16x8 alo = lds_row8<D>(Xl, lane & 31, ks * 2 + half);
      acc = mfma32(ah, gh, acc);
      acc1 = mfma32(ah, gl, acc1);
      acc2 = mfma32(alo, gh, acc2);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = (j >> 2) * 8 + half * 4 + (j & 3);
      S[r * LDF + wv * 32 + (lane & 31)] = (acc[j] + (acc1[j] + acc2[j])) * post;
    }
    lds_barrier();
  };
  auto snapshot = [&](int c) {
    float* dst = snap + (size_t)c * mat + (size_t)row0 * D;
    for (int i = tid; i < 32 * D; i += NT) dst[i] = S[(i / D) * LDF + i % D];
  };
  // Backward pass only: the state after every step j of the chain (j = 0: the
  // start, half the text write), [B*H][2][T+1][d][d].
  float* st_base = states ? states + ((size_t)bh * 2 + dir) * (g.T + 1) * mat + (size_t)row0 * D
                          : nullptr;
  int nstep = 0;
  auto keep = [&]() {
    if (!st_base) return;
    float* dst = st_base + (size_t)nstep * mat;
    for (int i = tid; i < 32 * D; i += NT) dst[i] = S[(i / D) * LDF + i % D];
  };

  // Step sequence: the text write (slot T, a = 0, times 1/2) when there is
  // text, then the frames the chain folds.  Step k uses LDS buffer k & 1; the
  // copy for step k+1 is issued once every wave is done with step k-1.
  bool text = g.L > 0;
  int slot = text ? g.T : next_frame(g, dir, -1);
  if (slot >= 0) {
    copy_g(slot, 0);
    load_b(slot, bcur);
  }
  for (int i = tid; i < 32 * D; i += NT) S[(i / D) * LDF + i % D] = 0.f;
  __syncthreads();
  if (!text) {
    snapshot(g.nc);
    keep();
  }
  int c = dir == 0 ? 0 : g.nc - 1;
  int bi = 0;
  while (slot >= 0) {
    const int nslot = text ? next_frame(g, dir, -1) : next_frame(g, dir, slot);
    if (!text) {
      // chunks whose state is the one before frame `slot` (anchors in
      // between do not change the state)
      if (dir == 0) {
        while (c < g.nc && win_lo(g, c) <= slot) snapshot(c++);
      } else {
        while (c >= 0 && win_hi(g, c) >= slot) snapshot(c--);
      }
    }
    wait_vmem();                          // own copies of this step's G and B
    __syncthreads();                      // everyone's; step k-1 done with buffer bi ^ 1
    if (nslot >= 0) {
      copy_g(nslot, bi ^ 1);
      load_b(nslot, bnxt);
    }
    step(text ? 0.0f : al[(size_t)slot * H], text ? 0.5f : 1.0f, bi);
    if (text) snapshot(g.nc);
    else ++nstep;
    keep();
#pragma unroll
    for (int i = 0; i < 2 * NCH; ++i) bcur[i] = bnxt[i];
    bi ^= 1;
    text = false;
    slot = nslot;
  }
  if (dir == 0) {
    while (c < g.nc) snapshot(c++);
  } else {
    while (c >= 0) snapshot(c--);
  }
}

// The same scan for the layer's forward path, with G_f supplied as two bf16
// planes (hi, lo; hi + lo = G_f to 2^-16) by the fused statistics pass: the
// planes go straight from LDS into the MFMA B operand, so a step converts
// only X = a S + B (one 32 x d block per workgroup), not G.  The state, the
// snapshots, the step order and the three-pass products are those of
// scan_mfma_kernel.  The 64 KB copy of the next step's planes runs at the
// CU's L2 -> LDS rate (about a microsecond at d = 128) and stalls the wave
// that issues it, so a workgroup pairs each of its d/32 compute waves with a
// copy wave on the same SIMD: the copy waves issue half of the next step's
// copies while the compute waves build X and the other half during the
// products.
template <int D>
__global__ void __launch_bounds__(4 * D)
scan_split_kernel(const bf16* __restrict__ Gp, const float* __restrict__ Bm,
                  const float* __restrict__ alpha, float* __restrict__ Sf,
                  float* __restrict__ Sb, Geo g, int H) {
  constexpr int NRB = D / 32;           // row blocks per chain = compute waves per workgroup
  constexpr int NT = 64 * NRB;          // compute threads; waves NRB .. 2 NRB - 1 copy
  constexpr int LDF = D;                // fp32 state row stride (floats)
  constexpr int NCH = 32 * D / 8 / NT;  // 8-value chunks of X per thread per step
  constexpr int CPR = D / 8;            // 16-byte chunks per bf16 plane row
  constexpr int PBYTES = D * D * 2;     // one plane
  constexpr int GBYTES = 2 * PBYTES;    // hi + lo
  constexpr int PBLK = PBYTES / 1024;   // 1 KB DMA blocks per plane
  constexpr int NGI = 2 * PBLK / NRB;   // DMA blocks per copy wave per G
  constexpr int KH = D / 32;            // k steps whose fragments are read ahead at once
  static_assert(NCH >= 1 && NCH * 8 * NT == 32 * D, "X build split");
  static_assert(NGI * NRB == 2 * PBLK && NGI % 2 == 0, "G copy split");
  // One LDS allocation: two G buffers (planes with XOR-swizzled 16-byte
  // chunks, conflict-free B-operand reads), the state rows S (fp32) and
  // X = aS + B as bf16 hi / lo.
  __shared__ __attribute__((aligned(1024))) char smem[2 * GBYTES + 32 * LDF * 4 + 2 * 32 * D * 2];
  char VDN_LDS* Gl = (char VDN_LDS*)smem;
  float VDN_LDS* S = (float VDN_LDS*)(smem + 2 * GBYTES);
  char VDN_LDS* Xh = (char VDN_LDS*)(smem + 2 * GBYTES + 32 * LDF * 4);
  char VDN_LDS* Xl = Xh + 32 * D * 2;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, half = lane >> 5;
  const bool copier = wv >= NRB;
  const int cw = wv - NRB;              // copy wave index
  // Workgroup i runs on XCD i % 8; with an even split each XCD gets whole
  // chains, so the row blocks of a chain share one L2.
  int wid = blockIdx.x;
  if (gridDim.x % (8 * NRB) == 0) wid = (wid & 7) * (gridDim.x >> 3) + (wid >> 3);
  const int rb = wid % NRB;
  const int chain = wid / NRB;
  const int dir = chain & 1;
  const int bh = chain >> 1;
  const int b = bh / H, h = bh % H;
  const int row0 = rb * 32;
  const size_t mat = (size_t)D * D;
  const bf16* Gbh = Gp + (size_t)bh * (g.T + 1) * 2 * mat;
  const float* Bbh = Bm + (size_t)bh * (g.T + 1) * mat;
  float* snap = (dir == 0 ? Sf : Sb) + (size_t)bh * (g.nc + 1) * mat;
  const float* al = alpha + (size_t)b * g.T * H + h;

  // Copies i0 .. i0 + n - 1 of copy wave cw for the planes of `slot` into
  // LDS buffer bi: block blk = cw * NGI + i covers 16-byte slots 64 * (blk %
  // PBLK) .. +63 of plane blk / PBLK; slot j holds row j / CPR, logical chunk
  // (j % CPR) ^ swz(row).
  auto copy_part = [&](int slot, int bi, int i0, int n) {
    const bf16* Gs = Gbh + (size_t)slot * 2 * mat;
#pragma unroll
    for (int i = i0; i < i0 + n; ++i) {
      const int blk = cw * NGI + i;
      const int pl = blk / PBLK;
      const int j = (blk % PBLK) * 64 + lane;
      const int row = j / CPR;
      const int ch = (j % CPR) ^ swz<D>(row);
      g2lds16(Gs + pl * mat + (size_t)row * D + ch * 8, Gl + bi * GBYTES + blk * 1024);
    }
  };
  float4 bcur[2 * NCH], bnxt[2 * NCH];
  auto load_b = [&](int slot, float4* br) {
    const float* Bs = Bbh + (size_t)slot * mat + (size_t)row0 * D;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = tid + i * NT;
      const float4* bp = (const float4*)(Bs + (q / (D / 8)) * D + (q % (D / 8)) * 8);
      br[2 * i] = bp[0];
      br[2 * i + 1] = bp[1];
    }
  };
  // X = a S + B as bf16 hi / lo (compute waves)
  auto build_x = [&](float a) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = tid + i * NT;
      const int r = q / (D / 8), c = (q % (D / 8)) * 8;
      const f32x4 s0 = *(const f32x4 VDN_LDS*)((const float VDN_LDS*)S + r * LDF + c);
      const f32x4 s1 = *(const f32x4 VDN_LDS*)((const float VDN_LDS*)S + r * LDF + c + 4);
      const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
      const float4 b0 = bcur[2 * i], b1 = bcur[2 * i + 1];
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      bf16x8 hv, lv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16 hi, lo;
        split_bf16(fmaf(a, sv[e], bv[e]), hi, lo);
        hv[e] = hi;
        lv[e] = lo;
      }
      const int off = swz_off<D>(r, c);
      *(bf16x8 VDN_LDS*)(Xh + off) = hv;
      *(bf16x8 VDN_LDS*)(Xl + off) = lv;
    }
  };
  // S <- X G, times `post`, G from LDS buffer bi (symmetric: its B-operand
  // columns are plane rows); compute waves.  Fragments are read KH k steps
  // at a time ahead of their products.
  auto product = [&](float post, int bi) {
    const int n = wv * 32 + (lane & 31);
    const char VDN_LDS* gh = Gl + bi * GBYTES;
    const char VDN_LDS* gl = gh + PBYTES;
    f32x16 acc = f32x16{}, acc1 = f32x16{}, acc2 = f32x16{};
#pragma unroll
    for (int k0 = 0; k0 < D / 16; k0 += KH) {
      bf16x8 fbh[KH], fbl[KH], fah[KH], fal[KH];
#pragma unroll
      for (int u = 0; u < KH; ++u) {
        fah[u] = lds_row8<D>(Xh, lane & 31, (k0 + u) * 2 + half);
        fbh[u] = lds_row8<D>(gh, n, (k0 + u) * 2 + half);
        fbl[u] = lds_row8<D>(gl, n, (k0 + u) * 2 + half);
        fal[u] = lds_row8<D>(Xl, lane & 31, (k0 + u) * 2 + half);
      }
#pragma unroll
      for (int u = 0; u < KH; ++u) {
        acc = mfma32(fah[u], fbh[u], acc);
        acc1 = mfma32(fah[u], fbl[u], acc1);
        acc2 = mfma32(fal[u], fbh[u], acc2);
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = (j >> 2) * 8 + half * 4 + (j & 3);
      S[r * LDF + wv * 32 + (lane & 31)] = (acc[j] + (acc1[j] + acc2[j])) * post;
    }
  };
  auto snapshot = [&](int c) {
    if (copier) return;
    float* dst = snap + (size_t)c * mat + (size_t)row0 * D;
    for (int i = tid; i < 32 * D / 4; i += NT) {
      const int r = (4 * i) / D, cc = (4 * i) % D;
      *(f32x4*)(dst + 4 * i) = *(const f32x4 VDN_LDS*)((const float VDN_LDS*)S + r * LDF + cc);
    }
  };

  // frames the chain folds: (fend: forward bound, fbeg: backward bound)
  const int fend = sgpr(fwd_scan_end(g)), fbeg = sgpr(bwd_scan_begin(g));
  auto next = [&](int f) {
    if (dir == 0) {
      int m = f + 1;
      while (m < fend && is_anchor(g, m)) ++m;
      return m < fend ? m : -1;
    }
    int m = f < 0 ? g.T - 1 : f - 1;
    while (m > fbeg && is_anchor(g, m)) --m;
    return m > fbeg ? m : -1;
  };
  // Step sequence: the text write (slot T, a = 0, times 1/2) when there is
  // text, then the frames the chain folds.  Step k reads G from LDS buffer
  // k & 1; the copy waves fill the other buffer for step k+1 during step k
  // and wait for their copies before the next step's first barrier.  Every
  // wave passes three barriers per step.
  bool text = g.L > 0;
  int slot = text ? g.T : next(-1);
  // decay of the current and the next step, loaded with the step's B
  float acur = 0.f, anxt = 0.f;
  if (copier) {
    if (slot >= 0) copy_part(slot, 0, 0, NGI);
  } else {
    if (slot >= 0) {
      load_b(slot, bcur);
      acur = text ? 0.f : al[(size_t)slot * H];
    }
    for (int i = tid; i < 32 * LDF; i += NT) S[i] = 0.f;
  }
  wait_vmem();
  __syncthreads();
  if (!text) snapshot(g.nc);
  int c = dir == 0 ? 0 : g.nc - 1;
  int bi = 0;
  while (slot >= 0) {
    const int nslot = next(text ? -1 : slot);
    if (!text) {
      // chunks whose state is the one before frame `slot` (anchors in
      // between do not change the state)
      if (dir == 0) {
        while (c < g.nc && win_lo(g, c) <= slot) snapshot(c++);
      } else {
        while (c >= 0 && win_hi(g, c) >= slot) snapshot(c--);
      }
    }
    lds_barrier();                        // G of this step landed; step k-1 done with buffer bi ^ 1
    if (copier) {
      if (nslot >= 0) copy_part(nslot, bi ^ 1, 0, NGI / 2);
      lds_barrier();
      if (nslot >= 0) copy_part(nslot, bi ^ 1, NGI / 2, NGI / 2);
      lds_barrier();
      wait_vmem();                        // this wave's copies for the next step
    } else {
      if (nslot >= 0) {
        load_b(nslot, bnxt);
        anxt = al[(size_t)nslot * H];
      }
      build_x(acur);
      lds_barrier();
      product(text ? 0.5f : 1.0f, bi);
      lds_barrier();
    }
    if (text) snapshot(g.nc);
#pragma unroll
    for (int i = 0; i < 2 * NCH; ++i) bcur[i] = bnxt[i];
    acur = anxt;
    bi ^= 1;
    text = false;
    slot = nslot;
  }
  if (dir == 0) {
    while (c < g.nc) snapshot(c++);
  } else {
    while (c >= 0) snapshot(c--);
  }
}

// ---------------------------------------------------------------------------
// Backward pass of the scan.  A chain folds frames f_1, f_2, ..., f_n (fold
// order) from S_0: S_j = (alpha_j S_{j-1} + B_j) G_j.  With dS_j the gradient
// of the loss with respect to S_j (from the snapshots that read S_j and from
// step j + 1):
//   dS_{j-1} = alpha_j (dS_j G_j) + (gradients of the snapshots of S_{j-1}),
// and dS_0 also takes the anchors' read of the start state (slot nc).  Every
// dS_j is kept (dspost, [B*H][2][T+1][d][d]); the per-frame gradients of
// B_j, G_j and alpha_j follow from dS_j, G_j and S_{j-1} frame by frame.
// Same layout as the forward scan: d/32 workgroups of 32 rows per chain,
// dS_j G_j on MFMA with the three-pass bf16 split, G_j staged through LDS.
// ---------------------------------------------------------------------------

// Frame folded just before f in the chain's fold order (-1 if none); f = -1
// asks for the last frame the chain folds.
__device__ __forceinline__ int prev_frame(const Geo& g, int dir, int f) {
  if (dir == 0) {
    int n = f < 0 ? fwd_scan_end(g) - 1 : f - 1;
    while (n >= 0 && is_anchor(g, n)) --n;
    return n;
  }
  const int fbeg = bwd_scan_begin(g);
  int n = f < 0 ? fbeg + 1 : f + 1;
  while (n < g.T && is_anchor(g, n)) ++n;
  return n < g.T ? n : -1;
}

template <int D>
__global__ void __launch_bounds__(2 * D)
scan_bwd_kernel(const float* __restrict__ G, const float* __restrict__ dR,
                const float* __restrict__ alpha, float* __restrict__ dspost, Geo g, int H) {
  constexpr int NRB = D / 32;
  constexpr int NT = 64 * NRB;
  constexpr int LDF = D;
  constexpr int NCH = 32 * D / 8 / NT;
  constexpr int CPR = D / 4;
  constexpr int GBYTES = D * D * 4;
  constexpr int NGI = GBYTES / 1024 / NRB;
  // one allocation, as in the forward scan: with separate __shared__ arrays
  // the compiler waits for the next G copy before writing X
  __shared__ __attribute__((aligned(1024))) char smem[2 * GBYTES + 32 * LDF * 4 + 2 * 32 * D * 2];
  char VDN_LDS* Gl = (char VDN_LDS*)smem;
  float VDN_LDS* S = (float VDN_LDS*)(smem + 2 * GBYTES);
  char VDN_LDS* Xh = (char VDN_LDS*)(smem + 2 * GBYTES + 32 * LDF * 4);
  char VDN_LDS* Xl = Xh + 32 * D * 2;
  auto gsw = [](int row) { return CPR >= 16 ? (row & 15) : ((row >> 1) & 7); };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, half = lane >> 5;
  int wid = blockIdx.x;
  if (gridDim.x % (8 * NRB) == 0) wid = (wid & 7) * (gridDim.x >> 3) + (wid >> 3);
  const int rb = wid % NRB;
  const int chain = wid / NRB;
  const int dir = chain & 1;
  const int bh = chain >> 1;
  const int b = bh / H, h = bh % H;
  const int row0 = rb * 32;
  const size_t mat = (size_t)D * D;
  const float* Gbh = G + (size_t)bh * (g.T + 1) * mat;
  const float* dRbh = dR + (size_t)bh * (g.nc + 1) * mat + (size_t)row0 * D;
  float* post = dspost + ((size_t)bh * 2 + dir) * (g.T + 1) * mat + (size_t)row0 * D;
  const float* al = alpha + (size_t)b * g.T * H + h;

  auto copy_g = [&](int slot, int bi) {
    const float* Gs = Gbh + (size_t)slot * mat;
#pragma unroll
    for (int i = 0; i < NGI; ++i) {
      const int blk = wv * NGI + i;
      const int sl = blk * 64 + lane;
      const int row = sl / CPR;
      const int ch = (sl % CPR) ^ gsw(row);
      g2lds16(Gs + (size_t)row * D + ch * 4, Gl + bi * GBYTES + blk * 1024);
    }
  };
  // dS rows += the gradient of chunk snapshot slot c.
  auto add_slot = [&](int c) {
    const float* src = dRbh + (size_t)c * mat;
    for (int i = tid; i < 32 * D; i += NT) S[(i / D) * LDF + i % D] += src[i];
  };
  // ... for every chunk whose snapshot holds state j
  auto inject = [&](int j) {
    for (int c = 0; c < g.nc; ++c)
      if (snap_index(g, dir, c) == j) add_slot(c);
  };
  auto keep = [&](int j) {
    float* dst = post + (size_t)j * mat;
    for (int i = tid; i < 32 * D; i += NT) dst[i] = S[(i / D) * LDF + i % D];
  };
  // dS <- a * (dS G), G from LDS buffer bi.
  auto step = [&](float a, int bi) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = tid + i * NT;
      const int r = q / (D / 8), c = (q % (D / 8)) * 8;
      const f32x4 s0 = *(const f32x4 VDN_LDS*)((const float VDN_LDS*)S + r * LDF + c);
      const f32x4 s1 = *(const f32x4 VDN_LDS*)((const float VDN_LDS*)S + r * LDF + c + 4);
      const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
      bf16x8 hv, lv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16 hi, lo;
        split_bf16(sv[e], hi, lo);
        hv[e] = hi;
        lv[e] = lo;
      }
      const int off = swz_off<D>(r, c);
      *(bf16x8 VDN_LDS*)(Xh + off) = hv;
      *(bf16x8 VDN_LDS*)(Xl + off) = lv;
    }
    lds_barrier();
    const int n = wv * 32 + (lane & 31);
    const int x = gsw(n);
    const char VDN_LDS* grow = Gl + bi * GBYTES + n * (4 * D);
    f32x16 acc = f32x16{}, acc1 = f32x16{}, acc2 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int c0 = 4 * ks + 2 * half;
      const f32x4 g0 = *(const f32x4 VDN_LDS*)(grow + ((c0 ^ x) << 4));
      const f32x4 g1 = *(const f32x4 VDN_LDS*)(grow + (((c0 + 1) ^ x) << 4));
      const float gv[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
      bf16x8 gh, gl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16 a_, c_;
        split_bf16(gv[e], a_, c_);
        gh[e] = a_;
        gl[e] = c_;
      }
      const bf16x8 ah = lds_row8<D>(Xh, lane & 31, ks * 2 + half);
      const bf16x8 alo = lds_row8<D>(Xl, lane & 31, ks * 2 + half);
      acc = mfma32(ah, gh, acc);
      acc1 = mfma32(ah, gl, acc1);
      acc2 = mfma32(alo, gh, acc2);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = (j >> 2) * 8 + half * 4 + (j & 3);
      S[r * LDF + wv * 32 + (lane & 31)] = (acc[j] + (acc1[j] + acc2[j])) * a;
    }
    lds_barrier();
  };

  int f = prev_frame(g, dir, -1);
  int j = f >= 0 ? fold_index(g, dir, f) : 0;   // number of steps
  for (int i = tid; i < 32 * D; i += NT) S[(i / D) * LDF + i % D] = 0.f;
  __syncthreads();
  inject(j);
  if (f >= 0) copy_g(f, 0);
  __syncthreads();
  int bi = 0;
  while (f >= 0) {
    keep(j);
    const int pf = prev_frame(g, dir, f);
    wait_vmem();
    __syncthreads();                     // G_f landed everywhere; buffer bi^1 free
    if (pf >= 0) copy_g(pf, bi ^ 1);
    step(al[(size_t)f * H], bi);
    --j;
    inject(j);
    __syncthreads();
    bi ^= 1;
    f = pf;
  }
  add_slot(g.nc);                        // j == 0 here: the anchors' read of S_0
  keep(0);
}

// Plain fp32 path: one workgroup per (batch, head, direction), whole state.
template <int D>
__global__ void __launch_bounds__(256)
scan_valu_kernel(const float* __restrict__ G, const float* __restrict__ Bm,
                 const float* __restrict__ alpha, float* __restrict__ Sf, float* __restrict__ Sb,
                 Geo g, int H) {
  __shared__ float S[D * D];
  __shared__ float X[D * D];
  const int tid = threadIdx.x;
  const int chain = blockIdx.x;
  const int dir = chain & 1;
  const int bh = chain >> 1;
  const int b = bh / H, h = bh % H;
  const size_t mat = (size_t)D * D;
  const float* Gbh = G + (size_t)bh * (g.T + 1) * mat;
  const float* Bbh = Bm + (size_t)bh * (g.T + 1) * mat;
  float* snap = (dir == 0 ? Sf : Sb) + (size_t)bh * (g.nc + 1) * mat;
  for (int i = tid; i < D * D; i += 256) S[i] = 0.f;
  __syncthreads();
  auto step = [&](int slot, float a, float post) {
    const float* Bs = Bbh + (size_t)slot * mat;
    const float* Gs = Gbh + (size_t)slot * mat;
    for (int i = tid; i < D * D; i += 256) X[i] = fmaf(a, S[i], Bs[i]);
    __syncthreads();
    for (int i = tid; i < D * D; i += 256) {
      int r = i / D, c = i % D;
      float acc = 0.f;
      for (int kk = 0; kk < D; ++kk) acc = fmaf(X[r * D + kk], Gs[(size_t)kk * D + c], acc);
      S[i] = acc * post;
    }
    __syncthreads();
  };
  auto snapshot = [&](int c) {
    float* dst = snap + (size_t)c * mat;
    for (int i = tid; i < D * D; i += 256) dst[i] = S[i];
  };
  if (g.L > 0) step(g.T, 0.0f, 0.5f);
  snapshot(g.nc);
  const float* al = alpha + (size_t)b * g.T * H + h;
  if (dir == 0) {
    const int fend = fwd_scan_end(g);
    int c = 0;
    for (int f = 0; f < fend; ++f) {
      while (c < g.nc && win_lo(g, c) == f) snapshot(c++);
      if (is_anchor(g, f)) continue;
      step(f, al[(size_t)f * H], 1.0f);
    }
    while (c < g.nc) snapshot(c++);
  } else {
    const int fbeg = bwd_scan_begin(g);
    int c = g.nc - 1;
    for (int f = g.T - 1; f > fbeg; --f) {
      while (c >= 0 && win_hi(g, c) == f) snapshot(c--);
      if (is_anchor(g, f)) continue;
      step(f, al[(size_t)f * H], 1.0f);
    }
    while (c >= 0) snapshot(c--);
  }
}

// R = S_fwd + S_bwd for every chunk slot (slot nc: S_x/2 + S_x/2 = S_x).
__global__ void __launch_bounds__(256)
combine_kernel(const float4* __restrict__ Sf, const float4* __restrict__ Sb, float4* __restrict__ R,
               size_t n4) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    float4 a = Sf[i], c = Sb[i];
    R[i] = make_float4(a.x + c.x, a.y + c.y, a.z + c.z, a.w + c.w);
  }
}

template <int D>
hipError_t launch_d(const float* G, const float* B, const float* alpha, const vdn_layout_t& l,
                    float* Sf, float* Sb, float* R, float* states, hipStream_t s) {
  Geo g = make_geo(l);
  long chains = (long)l.batch * l.heads * 2;
  if (l.dtype == VDN_BF16 && D >= 32) {
    if constexpr (D >= 32) {
      scan_mfma_kernel<D><<<dim3((unsigned)(chains * (D / 32))), dim3(2 * D), 0, s>>>(
          G, B, alpha, Sf, Sb, g, l.heads, states);
    }
  } else if (D >= 32) {
    if (states) return hipErrorNotSupported;
    if constexpr (D >= 32) {
      scan_mfma_kernel<D, true><<<dim3((unsigned)(chains * (D / 32))), dim3(2 * D), 0, s>>>(
          G, B, alpha, Sf, Sb, g, l.heads, nullptr);
    }
  } else {
    if (states) return hipErrorNotSupported;
    scan_valu_kernel<D><<<dim3((unsigned)chains), dim3(256), 0, s>>>(G, B, alpha, Sf, Sb, g,
                                                                      l.heads);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  size_t n4 = (size_t)l.batch * l.heads * (g.nc + 1) * D * D / 4;
  unsigned blocks = (unsigned)((n4 + 255) / 256 < 4096 ? (n4 + 255) / 256 : 4096);
  combine_kernel<<<dim3(blocks), dim3(256), 0, s>>>((const float4*)Sf, (const float4*)Sb,
                                                     (float4*)R, n4);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const float* G, const float* dR, const float* alpha,
                        const vdn_layout_t& l, float* dspost, hipStream_t s) {
  if constexpr (D < 32) {
    return hipErrorNotSupported;
  } else {
    Geo g = make_geo(l);
    long chains = (long)l.batch * l.heads * 2;
    scan_bwd_kernel<D><<<dim3((unsigned)(chains * (D / 32))), dim3(2 * D), 0, s>>>(
        G, dR, alpha, dspost, g, l.heads);
    return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_scan(const float* G, const float* B, const float* alpha, const vdn_layout_t& l,
                       float* Sf, float* Sb, float* R, hipStream_t s, float* states) {
  switch (l.head_dim_k) {
    case 128: return launch_d<128>(G, B, alpha, l, Sf, Sb, R, states, s);
    case 64: return launch_d<64>(G, B, alpha, l, Sf, Sb, R, states, s);
    case 32: return launch_d<32>(G, B, alpha, l, Sf, Sb, R, states, s);
    case 16: return launch_d<16>(G, B, alpha, l, Sf, Sb, R, states, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scan_split(const void* Gp, const float* B, const float* alpha,
                             const vdn_layout_t& l, float* Sf, float* Sb, float* R, hipStream_t s) {
  if (l.dtype != VDN_BF16) return hipErrorNotSupported;
  const Geo g = make_geo(l);
  const long chains = (long)l.batch * l.heads * 2;
  const int D = l.head_dim_k;
  switch (D) {
    case 128:
      scan_split_kernel<128><<<dim3((unsigned)(chains * 4)), dim3(512), 0, s>>>(
          (const bf16*)Gp, B, alpha, Sf, Sb, g, l.heads);
      break;
    case 64:
      scan_split_kernel<64><<<dim3((unsigned)(chains * 2)), dim3(256), 0, s>>>(
          (const bf16*)Gp, B, alpha, Sf, Sb, g, l.heads);
      break;
    case 32:
      scan_split_kernel<32><<<dim3((unsigned)chains), dim3(128), 0, s>>>(
          (const bf16*)Gp, B, alpha, Sf, Sb, g, l.heads);
      break;
    default:
      return hipErrorNotSupported;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n4 = (size_t)l.batch * l.heads * (g.nc + 1) * D * D / 4;
  const unsigned blocks = (unsigned)((n4 + 255) / 256 < 4096 ? (n4 + 255) / 256 : 4096);
  combine_kernel<<<dim3(blocks), dim3(256), 0, s>>>((const float4*)Sf, (const float4*)Sb,
                                                     (float4*)R, n4);
  return hipGetLastError();
}

hipError_t launch_scan_bwd(const float* G, const float* dR, const float* alpha,
                           const vdn_layout_t& l, float* dspost, hipStream_t s) {
  switch (l.head_dim_k) {
    case 128: return launch_bwd_d<128>(G, dR, alpha, l, dspost, s);
    case 64: return launch_bwd_d<64>(G, dR, alpha, l, dspost, s);
    case 32: return launch_bwd_d<32>(G, dR, alpha, l, dspost, s);
  }
  return hipErrorNotSupported;
}

}  // namespace vdn
