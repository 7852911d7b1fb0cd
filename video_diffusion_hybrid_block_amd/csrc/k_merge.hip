// Read + RMSNorm + gates + merge: o = sigmoid(g0) * o_soft
//   + sigmoid(g1) * RMSNorm(R q), with R the summed forward/backward state of
// the query's chunk (the full text write for anchor frames).  The linear read
// is RMS-normalised (no weight) before its gate; each branch has its own
// content-dependent sigmoid gate and the two are added.
// [PaperDaily "伯克利与Impossible视频生成:14.3秒视频6.70秒去噪" §三 (read both
//  states and add; gates per branch; RMS normalisation of the linear branch);
//  deepmagic blog "生成比播放還快", section 用兩條分支取代一條 (sigmoid gates)]
//
// gfx950 design (bf16, d in {32, 64, 128}): one workgroup (4 waves) per
// (batch, head, frame).  R (fp32) is split once into bf16 hi + lo in LDS; the
// read is computed transposed, o^T = R q^T, on v_mfma_f32_32x32x16_bf16 (two
// passes, hi and lo), so each lane owns one token column: the RMS reduction is
// 64 local squares plus one exchange with lane l^32.  q rows are the B operand
// straight from global memory (16-byte loads).  Memory-bound: q, o_soft and
// the gate logits are read once and o is written once.
#include "vdn_device.h"
#include "vdn_internal.h"

namespace vdn {

namespace {

__device__ __forceinline__ int r_slot(const Geo& g, int t) {
  return is_anchor(g, t) ? g.nc : t / g.C;
}

template <int D>
__global__ void __launch_bounds__(256)
merge_mfma_kernel(const bf16* __restrict__ q, const bf16* o_soft, const float* __restrict__ R,
                  const float* __restrict__ gates, bf16* o, Geo g, int H, float eps) {
  constexpr int NB = D / 32;
  __shared__ __attribute__((aligned(16))) char rh[D * D * 2];
  __shared__ __attribute__((aligned(16))) char rl[D * D * 2];
  char VDN_LDS* Rh = (char VDN_LDS*)rh;
  char VDN_LDS* Rl = (char VDN_LDS*)rl;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, half = lane >> 5;
  const int N = g.T * g.P;
  const int task = blockIdx.x;
  const int t = task % g.T;
  const int bh = task / g.T;
  const int b = bh / H, h = bh % H;
  const float* Rs = R + ((size_t)bh * (g.nc + 1) + r_slot(g, t)) * D * D;
  for (int i = tid; i < D * D / 4; i += 256) {
    float4 x = ((const float4*)Rs)[i];
    int r = (i * 4) / D, c = (i * 4) % D;
    float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bf16 hi, lo;
      split_bf16(xv[e], hi, lo);
      int off = swz_off<D>(r, c + e);
      *(bf16 VDN_LDS*)(Rh + off) = hi;
      *(bf16 VDN_LDS*)(Rl + off) = lo;
    }
  }
  __syncthreads();
  const int ntiles = (g.P + 31) / 32;
  for (int tile = wv; tile < ntiles; tile += 4) {
    const int tl = tile * 32 + (lane & 31);
    const bool valid = tl < g.P;
    const int tok = t * g.P + (valid ? tl : 0);
    const size_t rowoff = ((size_t)(b * (size_t)N + tok) * H + h) * D;
    bf16x8 qv[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qv[ks] = *(const bf16x8*)(q + rowoff + ks * 16 + half * 8);
    // o_soft and the gate logits are loaded with q: one memory latency per tile
    bf16x4 os[NB][4];
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        os[bi][jj] = *(const bf16x4*)(o_soft + rowoff + bi * 32 + jj * 8 + half * 4);
    const float2 gl = *(const float2*)(gates + ((size_t)(b * (size_t)N + tok) * H + h) * 2);
    f32x16 acc[NB];
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) {
      acc[bi] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        bf16x8 ah = lds_row8<D>(Rh, bi * 32 + (lane & 31), ks * 2 + half);
        bf16x8 al = lds_row8<D>(Rl, bi * 32 + (lane & 31), ks * 2 + half);
        acc[bi] = mfma32(ah, qv[ks], acc[bi]);
        acc[bi] = mfma32(al, qv[ks], acc[bi]);
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int j = 0; j < 16; ++j) ss = fmaf(acc[bi][j], acc[bi][j], ss);
    ss = xhalf_sum(ss);
    const float inv = rsqrtf(ss * (1.0f / D) + eps);
    const float g0 = sigmoidf(gl.x), g1 = sigmoidf(gl.y) * inv;
    if (valid) {
#pragma unroll
      for (int bi = 0; bi < NB; ++bi)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d = bi * 32 + jj * 8 + half * 4;
          bf16x4 out;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            out[e] = (bf16)fmaf(g0, (float)os[bi][jj][e], g1 * acc[bi][jj * 4 + e]);
          *(bf16x4*)(o + rowoff + d) = out;
        }
    }
  }
}

// Plain fp32 path: one workgroup per (batch, head, frame), one thread per token.
template <typename T, int D>
__global__ void __launch_bounds__(256)
merge_valu_kernel(const T* __restrict__ q, const T* o_soft, const float* __restrict__ R,
                  const float* __restrict__ gates, T* o, Geo g, int H, float eps) {
  __shared__ float Rsh[D * D];
  const int tid = threadIdx.x;
  const int N = g.T * g.P;
  const int task = blockIdx.x;
  const int t = task % g.T;
  const int bh = task / g.T;
  const int b = bh / H, h = bh % H;
  const float* Rs = R + ((size_t)bh * (g.nc + 1) + r_slot(g, t)) * D * D;
  for (int i = tid; i < D * D; i += 256) Rsh[i] = Rs[i];
  __syncthreads();
  for (int tl = tid; tl < g.P; tl += 256) {
    const int tok = t * g.P + tl;
    const size_t rowoff = ((size_t)(b * (size_t)N + tok) * H + h) * D;
    float qv[D], ov[D];
    for (int d = 0; d < D; ++d) qv[d] = Elem<T>::to_f(q[rowoff + d]);
    float ss = 0.f;
    for (int r = 0; r < D; ++r) {
      float acc = 0.f;
      for (int c = 0; c < D; ++c) acc = fmaf(Rsh[r * D + c], qv[c], acc);
      ov[r] = acc;
      ss = fmaf(acc, acc, ss);
    }
    const float inv = rsqrtf(ss / D + eps);
    const size_t goff = ((size_t)(b * (size_t)N + tok) * H + h) * 2;
    const float g0 = sigmoidf(gates[goff]), g1 = sigmoidf(gates[goff + 1]) * inv;
    for (int d = 0; d < D; ++d)
      o[rowoff + d] = Elem<T>::from_f(fmaf(g0, Elem<T>::to_f(o_soft[rowoff + d]), g1 * ov[d]));
  }
}

template <int D>
hipError_t launch_mfma(const void* q, const void* o_soft, const float* R, const float* gates,
                       const vdn_layout_t& l, float eps, void* o, hipStream_t s) {
  Geo g = make_geo(l);
  long grid = (long)l.batch * l.heads * g.T;
  merge_mfma_kernel<D><<<dim3((unsigned)grid), dim3(256), 0, s>>>(
      (const bf16*)q, (const bf16*)o_soft, R, gates, (bf16*)o, g, l.heads, eps);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_valu(const void* q, const void* o_soft, const float* R, const float* gates,
                       const vdn_layout_t& l, float eps, void* o, hipStream_t s) {
  Geo g = make_geo(l);
  long grid = (long)l.batch * l.heads * g.T;
  merge_valu_kernel<T, D><<<dim3((unsigned)grid), dim3(256), 0, s>>>(
      (const T*)q, (const T*)o_soft, R, gates, (T*)o, g, l.heads, eps);
  return hipGetLastError();
}

// Merge backward from saved residuals.  With s0, s1 the gate sigmoids, O_s
// the softmax branch and n = RMSNorm(o_lin) = o_lin / r of one token-head:
// dl0 = (dO . O_s) s0 (1 - s0), dl1 = (dO . n) s1 (1 - s1), dO_s = s0 dO
// (bf16, the softmax backward's operand), -D (D = dO_s . O_s), and through the
// normalisation do_lin = (s1 dO - n (s1 dO . n) / d) / r.  32 lanes per
// token-head (d/32 consecutive values each, 16-byte loads for d = 128),
// 8 token-heads per workgroup; HBM-bound.
template <int D>
__global__ void __launch_bounds__(256)
merge_bwd_saved_kernel(const bf16* __restrict__ dO, const float* __restrict__ gates,
                       const float* __restrict__ o_soft, const float* __restrict__ o_lin,
                       const float* __restrict__ rinv, float* __restrict__ dgates,
                       bf16* __restrict__ dos, float* __restrict__ dlin,
                       float* __restrict__ dvec, long rows, int N, int H) {
  constexpr int NE = D / 32;
  using fv = float __attribute__((ext_vector_type(NE)));
  using bv = bf16 __attribute__((ext_vector_type(NE)));
  const long r = (long)blockIdx.x * 8 + (threadIdx.x >> 5);   // (b N + token) H + h
  const int l32 = threadIdx.x & 31;
  if (r >= rows) return;                 // whole 32-lane groups leave together
  const size_t off = (size_t)r * D + l32 * NE;
  const bv dov = *(const bv*)(dO + off);
  const fv os = *(const fv*)(o_soft + off);
  const fv n = *(const fv*)(o_lin + off);
  const float2 gl = *(const float2*)(gates + r * 2);
  const long bt = r / H;
  const int h = (int)(r - bt * H);
  const long b = bt / N;
  const size_t ri = ((size_t)b * H + h) * N + (size_t)(bt - b * N);
  const float ir = rinv[ri];
  const float s0 = sigmoidf(gl.x), s1 = sigmoidf(gl.y);
  float dot0 = 0.f, dot1 = 0.f, dsum = 0.f;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const float dv = (float)dov[e];
    dot0 = fmaf(dv, os[e], dot0);
    dot1 = fmaf(dv, n[e], dot1);
    dsum = fmaf((float)(bf16)(s0 * dv), os[e], dsum);
  }
#pragma unroll
  for (int m = 16; m > 0; m >>= 1) {
    dot0 += __shfl_xor(dot0, m, 32);
    dot1 += __shfl_xor(dot1, m, 32);
    dsum += __shfl_xor(dsum, m, 32);
  }
  const float kn = s1 * dot1 * (1.0f / D);
  bv vs;
  fv vl;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const float dv = (float)dov[e];
    vs[e] = (bf16)(s0 * dv);
    vl[e] = ir * fmaf(-n[e], kn, s1 * dv);
  }
  *(bv*)(dos + off) = vs;
  *(fv*)(dlin + off) = vl;
  if (l32 == 0) {
    *(float2*)(dgates + r * 2) = make_float2(dot0 * s0 * (1.0f - s0), dot1 * s1 * (1.0f - s1));
    dvec[ri] = -dsum;                       // -D: the backward's products start from it
  }
}

template <int D>
hipError_t launch_bwd_saved(const void* dO, const float* gates, const float* o_soft,
                            const float* o_lin, const float* rinv, const vdn_layout_t& l,
                            float* dgates, void* dos, float* dlin, float* dvec, hipStream_t s) {
  const int N = l.frames * l.tokens_per_frame;
  const long rows = (long)l.batch * N * l.heads;
  const long grid = (rows + 7) / 8;
  if (grid >= (1L << 31)) return hipErrorInvalidValue;
  merge_bwd_saved_kernel<D><<<dim3((unsigned)grid), dim3(256), 0, s>>>(
      (const bf16*)dO, gates, o_soft, o_lin, rinv, dgates, (bf16*)dos, dlin, dvec, rows, N,
      l.heads);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge_bwd_saved(const void* dO, const float* gates, const float* o_soft,
                                  const float* o_lin, const float* rinv, const vdn_layout_t& l,
                                  float* dgates, void* dos, float* dlin, float* dvec,
                                  hipStream_t s) {
  if (l.dtype != VDN_BF16) return hipErrorNotSupported;
  switch (l.head_dim_k) {
    case 128: return launch_bwd_saved<128>(dO, gates, o_soft, o_lin, rinv, l, dgates, dos, dlin, dvec, s);
    case 64: return launch_bwd_saved<64>(dO, gates, o_soft, o_lin, rinv, l, dgates, dos, dlin, dvec, s);
    case 32: return launch_bwd_saved<32>(dO, gates, o_soft, o_lin, rinv, l, dgates, dos, dlin, dvec, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const void* q, const void* o_soft, const float* R, const float* gates,
                        const vdn_layout_t& l, float eps, void* o, hipStream_t s) {
  const int d = l.head_dim_k;
  if (l.dtype == VDN_BF16) {
    switch (d) {
      case 128: return launch_mfma<128>(q, o_soft, R, gates, l, eps, o, s);
      case 64: return launch_mfma<64>(q, o_soft, R, gates, l, eps, o, s);
      case 32: return launch_mfma<32>(q, o_soft, R, gates, l, eps, o, s);
      case 16: return launch_valu<bf16, 16>(q, o_soft, R, gates, l, eps, o, s);
    }
  } else {
    switch (d) {
      case 128: return launch_valu<float, 128>(q, o_soft, R, gates, l, eps, o, s);
      case 64: return launch_valu<float, 64>(q, o_soft, R, gates, l, eps, o, s);
      case 32: return launch_valu<float, 32>(q, o_soft, R, gates, l, eps, o, s);
      case 16: return launch_valu<float, 16>(q, o_soft, R, gates, l, eps, o, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace vdn
