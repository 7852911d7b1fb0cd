// Output projections of the two branches as one product:
//   y[m][n] = sum_k x[m][k] w[n][k],
// x = [sigmoid(l0) O_soft ; sigmoid(l1) RMSNorm(R q)] per token (2*H*d
// values, softmax branch first), w = [W_s W_l] in (out, in) order.  Each
// branch keeps its own projection; one product applies both and adds them.
// [PaperDaily "伯克利与Impossible视频生成:14.3秒视频6.70秒去噪" §三, figure 3
//  (each branch: own gate, own output projection, then added back to the
//  residual stream); arXiv listing "Video DeltaNet: A Video-Native Hybrid
//  Attention for Livestream Video Generation", abstract (separate output
//  projections and learnable gates calibrate the two branches)]
//
// gfx950 design: bf16 operands, fp32 accumulation on
// v_mfma_f32_32x32x16_bf16, bf16 output.  A workgroup of 8 waves computes a
// 256 (n) x 256 (m) block of y^T: wave (wn, wm) owns 128 n x 64 m, i.e.
// 4 x 2 MFMA blocks.  Computing y^T (A = w rows, B = x rows, both
// k-contiguous) lets each lane own one token and store four consecutive
// outputs at a time.  64-deep k steps stream through a two-stage LDS ring
// with 16-byte direct-to-LDS loads (waves 0-3 move the w tile, 4-7 the x
// tile); each wave's eight copies for the next step are spread between the
// MFMAs of the first half of the current step (issued in one burst they hold
// up the MFMA stream of every wave at once).  Rows are 128 bytes with the
// 16-byte chunk c of row r stored at c ^ ((r / 2) % 8), so sixteen lanes
// reading sixteen rows at one chunk hit distinct bank groups.  XCD-aware tile
// order (consecutive tiles on one XCD) keeps the output tiles of one token
// block on one XCD, whose L2 then serves that block's x to all of them.
#include <type_traits>

#include "vdn_device.h"
#include "vdn_internal.h"

namespace vdn {

namespace {

constexpr int PBM = 256, PBN = 256, PBK = 64;

__global__ void __launch_bounds__(512)
proj_gemm_kernel(const bf16* __restrict__ x, const bf16* __restrict__ w, bf16* __restrict__ y,
                 long M, int K, int N) {
  constexpr int ROWB = PBK * 2;                   // 128-byte rows
  constexpr int TILEB = PBM * ROWB;               // 32 KB per operand tile
  constexpr int STAGE = 2 * TILEB;                // w tile then x tile
  constexpr int NIW = TILEB / 1024 / 4;           // DMA instructions per wave per tile (8)
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  char VDN_LDS* lds = (char VDN_LDS*)smem;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int mt_n = (int)((M + PBM - 1) / PBM), nt_n = (N + PBN - 1) / PBN;
  const int ntile = mt_n * nt_n;
  // workgroup b runs on XCD b % 8: give XCD x a contiguous range of tiles
  int t = blockIdx.x;
  {
    const int q = ntile >> 3, r = ntile & 7, xc = t & 7, k = t >> 3;
    t = xc * q + (xc < r ? xc : r) + k;
  }
  const int mt = sgpr(t / nt_n), nt = sgpr(t % nt_n);
  const long m0 = (long)mt * PBM;
  const int n0 = nt * PBN;

  // DMA: waves 0-3 fill the w tile (rows n0 ..), waves 4-7 the x tile (rows
  // m0 ..); instruction i of a wave fills 1 KB block 4*i + (wv % 4), lane l
  // writing slot 64*blk + l: row slot / 8, physical chunk slot % 8, which holds
  // logical chunk (slot % 8) ^ ((row / 2) % 8).  Rows past M (N) re-read the
  // last row; their results are never stored.
  const bool xw = wv >= 4;
  const bf16* src[NIW];
#pragma unroll
  for (int i = 0; i < NIW; ++i) {
    const int sl = (i * 4 + (wv & 3)) * 64 + lane;
    const int r = sl / 8;
    const int ch = (sl % 8) ^ ((r / 2) % 8);
    const long grow = xw ? (m0 + r < M ? m0 + r : M - 1) : (long)(n0 + r < N ? n0 + r : N - 1);
    src[i] = (xw ? x : w) + grow * K + ch * 8;
  }
  // Read bases: row r, logical chunk 2j + half sits at physical
  // (2j + half) ^ ((r / 2) % 8) = 2j ^ yv, yv = half ^ ((r / 2) % 8); the 32-row
  // blocks of a wave add multiples of 4 KB (immediate offsets).
  const int wn = wv & 1, wm = wv >> 1;             // 2 (n) x 4 (m) waves
  const int rl = lane & 31;
  const int rbase = rl * ROWB + 16 * (half ^ ((rl / 2) % 8));
  const int aoff = wn * 128 * ROWB;                // w rows of this wave
  const int boff = TILEB + wm * 64 * ROWB;         // x rows of this wave

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = K / PBK;
  {
    char VDN_LDS* tb = lds + (xw ? TILEB : 0);
#pragma unroll
    for (int i = 0; i < NIW; ++i) g2lds16(src[i], tb + (i * 4 + (wv & 3)) * 1024);
  }
  // One k step: wait for this wave's copies, barrier (everyone's copies are in
  // and everyone is done with the other stage), then 4 x 8 MFMAs, with the
  // copies of the next step (when there is one) after every second MFMA of the
  // first two 16-deep slices.
  auto step = [&](int kt, auto more) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const char VDN_LDS* st = lds + (kt & 1) * STAGE;
    char VDN_LDS* tbw = lds + ((kt + 1) & 1) * STAGE + (xw ? TILEB : 0);
#pragma unroll
    for (int ks = 0; ks < PBK / 16; ++ks) {
      const int ro = rbase ^ (32 * ks);
      bf16x8 af[4], bfv[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *(const bf16x8 VDN_LDS*)(st + aoff + i * 32 * ROWB + ro);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfv[j] = *(const bf16x8 VDN_LDS*)(st + boff + j * 32 * ROWB + ro);
#pragma unroll
      for (int mi = 0; mi < 8; ++mi) {
        acc[mi >> 1][mi & 1] = mfma32(af[mi >> 1], bfv[mi & 1], acc[mi >> 1][mi & 1]);
        if constexpr (decltype(more)::value) {
          if (ks < 2 && (mi & 1)) {
            const int i = ks * 4 + (mi >> 1);
            g2lds16(src[i] + (kt + 1) * PBK, tbw + (i * 4 + (wv & 3)) * 1024);
          }
        }
      }
    }
  };
  for (int kt = 0; kt + 1 < nk; ++kt) step(kt, std::true_type{});
  step(nk - 1, std::false_type{});

  // acc[i][j][e]: y^T[n][m] with n = n0 + wn*128 + 32 i + 8 (e / 4) + 4 half +
  // e % 4 and m = m0 + wm*64 + 32 j + lane % 32: four consecutive n per group.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const long m = m0 + wm * 64 + 32 * j + rl;
    if (m >= M) continue;
    bf16* yr = y + m * N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 128 + 32 * i + 8 * g + 4 * half;
        if (n >= N) continue;
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)acc[i][j][g * 4 + e];
        *(bf16x4*)(yr + n) = v;
      }
  }
}

// ---------------------------------------------------------------------------
// FP8 projection (the pages run the linear layers after the attention in
// FP8; deepmagic blog "生成比播放還快", section 實測數據).  Format: OCP MXFP8 -
// E4M3 elements, one E8M0 power-of-two scale per 32 consecutive values along
// the contraction: for a block with largest magnitude a, X = floor(log2 a) - 8
// (448 = 1.75 * 2^8 is E4M3's largest normal; X >= -127, 0 for a zero block),
// elements = E4M3(v / 2^X), round to nearest even, clamped to +-448.
// ---------------------------------------------------------------------------

// One thread per 32-value block of a bf16 [M][K] matrix: q [M][K] E4M3 codes,
// s [M][K/32] E8M0 scales (X + 127).
__global__ void __launch_bounds__(256)
mx_quant_kernel(const bf16* __restrict__ x, uint8_t* __restrict__ qo, uint8_t* __restrict__ so,
                long nblk) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= nblk) return;
  const bf16x8* src = (const bf16x8*)(x + i * 32);
  float v[32];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const bf16x8 c = src[u];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[u * 8 + e] = (float)c[e];
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
  const int X = mx_block_exp(amax);
  uint32_t w[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) w[u] = mx_pack4(v[u * 4], v[u * 4 + 1], v[u * 4 + 2], v[u * 4 + 3], X);
  u32x4* dst = (u32x4*)(qo + i * 32);
  dst[0] = u32x4{w[0], w[1], w[2], w[3]};
  dst[1] = u32x4{w[4], w[5], w[6], w[7]};
  so[i] = (uint8_t)(X + 127);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// y[m][n] = sum_k x[m][k] w[n][k] from MXFP8 operands (codes + scales, both
// [rows][K] / [rows][K/32]); bf16 y, fp32 accumulation on
// v_mfma_scale_f32_32x32x64_f8f6f4.  Same tiling as the bf16 product: 256 x 256
// output tiles, 8 waves of 128 (n) x 64 (m), 128-byte rows (128 codes) per k
// step through a two-stage direct-to-LDS ring.  Operand layout of the scaled
// MFMA (checked on gfx950): lane (r, h) supplies for its 64-deep k block the
// 16 codes at 16h .. 16h+15 (first scale block) and 32+16h .. (second), and
// lane r + 32b the scale of block b.
__global__ void __launch_bounds__(512)
proj_mxfp8_kernel(const uint8_t* __restrict__ x, const uint8_t* __restrict__ xs,
                  const uint8_t* __restrict__ w, const uint8_t* __restrict__ wsc,
                  bf16* __restrict__ y, long M, int K, int N) {
  constexpr int BKB = 128;                        // codes (bytes) per row per k step
  constexpr int ROWB = BKB;
  constexpr int TILEB = PBM * ROWB;               // 32 KB per operand tile
  constexpr int STAGE = 2 * TILEB;
  constexpr int NIW = TILEB / 1024 / 4;           // 8
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  char VDN_LDS* lds = (char VDN_LDS*)smem;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int mt_n = (int)((M + PBM - 1) / PBM), nt_n = (N + PBN - 1) / PBN;
  const int ntile = mt_n * nt_n;
  int t = blockIdx.x;
  {
    const int q = ntile >> 3, r = ntile & 7, xc = t & 7, k = t >> 3;
    t = xc * q + (xc < r ? xc : r) + k;
  }
  const int mt = sgpr(t / nt_n), nt = sgpr(t % nt_n);
  const long m0 = (long)mt * PBM;
  const int n0 = nt * PBN;
  const int KS = K / 32;                          // scale bytes per row

  // DMA exactly as the bf16 product (128-byte rows, XOR-swizzled chunks)
  const bool xw = wv >= 4;
  const uint8_t* src[NIW];
#pragma unroll
  for (int i = 0; i < NIW; ++i) {
    const int sl = (i * 4 + (wv & 3)) * 64 + lane;
    const int r = sl / 8;
    const int ch = (sl % 8) ^ ((r / 2) % 8);
    const long grow = xw ? (m0 + r < M ? m0 + r : M - 1) : (long)(n0 + r < N ? n0 + r : N - 1);
    src[i] = (xw ? x : w) + grow * K + ch * 16;
  }
  const int wn = wv & 1, wm = wv >> 1;
  const int rl = lane & 31;
  const int sw = (rl / 2) % 8;                    // chunk swizzle of this lane's rows
  const int aoff = wn * 128 * ROWB + rl * ROWB;
  const int boff = TILEB + wm * 64 * ROWB + rl * ROWB;
  // scale rows of this lane: w rows n0 + wn*128 + 32 i + rl, x rows m0 + wm*64 + 32 j + rl
  const uint32_t* wsr[4];
  const uint32_t* xsr[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + wn * 128 + 32 * i + rl;
    wsr[i] = (const uint32_t*)(wsc + (size_t)(n < N ? n : N - 1) * KS);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const long m = m0 + wm * 64 + 32 * j + rl;
    xsr[j] = (const uint32_t*)(xs + (size_t)(m < M ? m : M - 1) * KS);
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = K / BKB;
  {
    char VDN_LDS* tb = lds + (xw ? TILEB : 0);
#pragma unroll
    for (int i = 0; i < NIW; ++i) g2lds16(src[i], tb + (i * 4 + (wv & 3)) * 1024);
  }
  uint32_t sa[4], sb[2];                          // this step's 4 scale bytes per row
#pragma unroll
  for (int i = 0; i < 4; ++i) sa[i] = wsr[i][0];
#pragma unroll
  for (int j = 0; j < 2; ++j) sb[j] = xsr[j][0];
  auto step = [&](int kt, auto more) {
    uint32_t na[4], nb[2];
    if constexpr (decltype(more)::value) {
#pragma unroll
      for (int i = 0; i < 4; ++i) na[i] = wsr[i][kt + 1];
#pragma unroll
      for (int j = 0; j < 2; ++j) nb[j] = xsr[j][kt + 1];
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const char VDN_LDS* st = lds + (kt & 1) * STAGE;
    char VDN_LDS* tbw = lds + ((kt + 1) & 1) * STAGE + (xw ? TILEB : 0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // logical chunks 4 kb + h and 4 kb + 2 + h of the row
      const int c0 = ((4 * kb + half) ^ sw) * 16, c1 = ((4 * kb + 2 + half) ^ sw) * 16;
      i32x8 af[4], bfv[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 lo = *(const u32x4 VDN_LDS*)(st + aoff + i * 32 * ROWB + c0);
        const u32x4 hi = *(const u32x4 VDN_LDS*)(st + aoff + i * 32 * ROWB + c1);
        af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 lo = *(const u32x4 VDN_LDS*)(st + boff + j * 32 * ROWB + c0);
        const u32x4 hi = *(const u32x4 VDN_LDS*)(st + boff + j * 32 * ROWB + c1);
        bfv[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
      const int sh = 8 * (2 * kb + half);
#pragma unroll
      for (int mi = 0; mi < 8; ++mi) {
        const int i = mi >> 1, j = mi & 1;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            af[i], bfv[j], acc[i][j], 0, 0, 0, (int)((sa[i] >> sh) & 0xff), 0,
            (int)((sb[j] >> sh) & 0xff));
        if constexpr (decltype(more)::value) {
          if (kb == 0) g2lds16(src[mi] + (size_t)(kt + 1) * BKB, tbw + (mi * 4 + (wv & 3)) * 1024);
        }
      }
    }
    if constexpr (decltype(more)::value) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[i] = na[i];
#pragma unroll
      for (int j = 0; j < 2; ++j) sb[j] = nb[j];
    }
  };
  for (int kt = 0; kt + 1 < nk; ++kt) step(kt, std::true_type{});
  step(nk - 1, std::false_type{});

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const long m = m0 + wm * 64 + 32 * j + rl;
    if (m >= M) continue;
    bf16* yr = y + m * N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 128 + 32 * i + 8 * g + 4 * half;
        if (n >= N) continue;
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)acc[i][j][g * 4 + e];
        *(bf16x4*)(yr + n) = v;
      }
  }
}

}  // namespace

bool proj_shape_ok(long M, int K, int N) {
  return M >= 1 && K >= PBK && K % PBK == 0 && N >= 8 && N % 8 == 0;
}

hipError_t launch_proj(const void* x, const void* w, long M, int K, int N, void* y, hipStream_t s) {
  if (!proj_shape_ok(M, K, N)) return hipErrorInvalidValue;
  const long ntile = ((M + PBM - 1) / PBM) * (long)((N + PBN - 1) / PBN);
  proj_gemm_kernel<<<dim3((unsigned)ntile), dim3(512), 0, s>>>((const bf16*)x, (const bf16*)w,
                                                                (bf16*)y, M, K, N);
  return hipGetLastError();
}

bool mx_quant_shape_ok(long M, int K) { return M >= 1 && K >= 32 && K % 32 == 0; }

hipError_t launch_mx_quant(const void* x, long M, int K, void* q, void* scales, hipStream_t s) {
  if (!mx_quant_shape_ok(M, K)) return hipErrorInvalidValue;
  const long nblk = M * (long)(K / 32);
  mx_quant_kernel<<<dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, s>>>(
      (const bf16*)x, (uint8_t*)q, (uint8_t*)scales, nblk);
  return hipGetLastError();
}

bool proj_mxfp8_shape_ok(long M, int K, int N) {
  return M >= 1 && K >= 128 && K % 128 == 0 && N >= 8 && N % 8 == 0;
}

hipError_t launch_proj_mxfp8(const void* xq, const void* xs, const void* wq, const void* ws,
                             long M, int K, int N, void* y, hipStream_t s) {
  if (!proj_mxfp8_shape_ok(M, K, N)) return hipErrorInvalidValue;
  const long ntile = ((M + PBM - 1) / PBM) * (long)((N + PBN - 1) / PBN);
  proj_mxfp8_kernel<<<dim3((unsigned)ntile), dim3(512), 0, s>>>(
      (const uint8_t*)xq, (const uint8_t*)xs, (const uint8_t*)wq, (const uint8_t*)ws, (bf16*)y,
      M, K, N);
  return hipGetLastError();
}

}  // namespace vdn
