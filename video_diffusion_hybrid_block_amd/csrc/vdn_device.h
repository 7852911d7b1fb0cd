// Device helpers for the gfx950 (CDNA4) kernels: vector types, MFMA wrappers,
// LDS swizzles and transposed LDS reads.
//
// MFMA operand layouts used throughout (checked on gfx950 hardware):
//   v_mfma_f32_32x32x16_bf16: lane l supplies A[m = l%32][k = 8*(l/32) + e] and
//     B[k = 8*(l/32) + e][n = l%32], e = 0..7; result register j of lane l is
//     C[8*(j/4) + 4*(l/32) + j%4][l%32].
//   ds_read_b64_tr_b16: inside each group of 16 lanes, lane j receives element
//     j%4 of the 8-byte words addressed by lanes j/4 + 4*i, i = 0..3.  With lane
//     s addressing row s/4, columns 4*(s%4)..+3 of a 16-wide block, lane j gets
//     column j of the four rows: a 4x16 -> 16x4 transpose.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define VDN_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Element type traits: loads of 8 / 4 consecutive values as float.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float to_f(float x) { return x; }
  static __device__ __forceinline__ float from_f(float x) { return x; }
};
template <> struct Elem<bf16> {
  static __device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
  static __device__ __forceinline__ bf16 from_f(float x) { return (bf16)x; }
};

// Split a float into bf16 hi + bf16 lo with hi + lo == x up to 2^-16 relative.
__device__ __forceinline__ void split_bf16(float x, bf16& hi, bf16& lo) {
  hi = (bf16)x;
  lo = (bf16)(x - (float)hi);
}

// Exchange with lane l^32: returns max / sum of the value and its partner's.
// v_max3_f32 / v_max_f32 without the NaN-quieting copies the compiler adds
// to fmaxf on MFMA results (scores are finite or -inf).
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float xhalf_max_raw(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ int sgpr(int x) { return __builtin_amdgcn_readfirstlane(x); }
// A wave-uniform pointer, pinned to SGPRs (lets loads use scalar base +
// 32-bit vector offset addressing).
__device__ __forceinline__ const char* sgpr_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float xhalf_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// MXFP8 (OCP microscaling, E4M3 elements): the shared exponent X of a block
// whose largest magnitude is amax is floor(log2 amax) - 8 (8 = exponent of
// E4M3's largest normal, 448 = 1.75 * 2^8), at least -127 (E8M0 range); an
// all-zero block gets X = 0.  The scale byte is X + 127.
__device__ __forceinline__ int mx_block_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int ex;
  frexpf(amax, &ex);                 // amax = f 2^ex, f in [0.5, 1)
  const int X = ex - 1 - 8;
  return X < -127 ? -127 : X;
}
// Four values v / 2^X as E4M3 codes (round to nearest even; magnitudes past
// 448 clamp to 448), byte e of the result holding value e.
__device__ __forceinline__ uint32_t mx_pack4(float a, float b, float c, float d, int X) {
  const float a2 = fminf(fmaxf(ldexpf(a, -X), -448.f), 448.f);
  const float b2 = fminf(fmaxf(ldexpf(b, -X), -448.f), 448.f);
  const float c2 = fminf(fmaxf(ldexpf(c, -X), -448.f), 448.f);
  const float d2 = fminf(fmaxf(ldexpf(d, -X), -448.f), 448.f);
  int acc = __builtin_amdgcn_cvt_pk_fp8_f32(a2, b2, 0, false);   // bytes 0, 1
  acc = __builtin_amdgcn_cvt_pk_fp8_f32(c2, d2, acc, true);      // bytes 2, 3
  return (uint32_t)acc;
}

// XOR swizzle of the 16-byte chunk index inside an LDS row of D bf16 values.
// It makes (a) 16 consecutive rows read at one logical chunk by ds_read_b128
// and (b) 4 consecutive rows x 64 bytes read by ds_read_b64_tr_b16 fall on
// distinct banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else if constexpr (D == 64) {
    int u = (r >> 1) & 7;
    return u ^ ((u & 1) << 2);
  } else {
    static_assert(D == 32, "head size");
    return (r >> 2) & 3;
  }
}

// Byte offset of (row r, element col) in a swizzled [rows][D] bf16 LDS tile.
template <int D>
__device__ __forceinline__ int swz_off(int r, int col) {
  int ch = (col >> 3) ^ swz<D>(r);
  return r * (D * 2) + ch * 16 + (col & 7) * 2;
}

// 16-byte read of logical chunk `ch` of row r.
template <int D>
__device__ __forceinline__ bf16x8 lds_row8(const char VDN_LDS* base, int r, int ch) {
  const char VDN_LDS* p = base + r * (D * 2) + ((ch ^ swz<D>(r)) << 4);
  return *(const bf16x8 VDN_LDS*)p;
}

// MFMA operand with 8 consecutive *rows* of one column from a swizzled
// [rows][D] bf16 tile, using two transposed reads: lane l gets
// tile[row0 + 8*(l/32) + e][col0 + l%32], e = 0..7.
template <int D>
__device__ __forceinline__ bf16x8 lds_col8(const char VDN_LDS* base, int row0, int col0, int lane) {
  int g = lane >> 4, s = lane & 15;
  int col = col0 + ((g & 1) << 4) + ((s & 3) << 2);
  int r = row0 + ((g >> 1) << 3) + (s >> 2);
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (i16x4 VDN_LDS*)(base + swz_off<D>(r, col)));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (i16x4 VDN_LDS*)(base + swz_off<D>(r + 4, col)));
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Asynchronous 16-byte global -> LDS copy: this lane's 16 bytes land at
// lds_wave_base + 16 * lane.
__device__ __forceinline__ void g2lds16(const void* gptr, char VDN_LDS* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gptr, (void VDN_LDS*)lds_wave_base, 16, 0, 0);
}

// The same copies written as asm, from a wave-uniform base plus a 32-bit
// byte offset per lane (dma16s, dma4s) or from a 64-bit address per lane
// (dma16v).  The compiler then does not order LDS reads after them: it cannot
// tell which LDS bytes a copy writes, and before a transposed LDS read it
// waits for every copy in flight, the ones prefetched for later tiles
// included.  Completion is the kernel's own vmcnt wait plus a barrier.
// The compiler's hazard checks do not look inside the asm, so each copy
// starts with five wait states: enough after an SGPR written by a VALU
// instruction (v_readfirstlane of the base) and after the M0 write.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, char VDN_LDS* lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase),
                  "{m0}"(__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds))
               : "memory");
}
__device__ __forceinline__ void dma4s(const void* sbase, uint32_t voff, float VDN_LDS* lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(sbase),
                  "{m0}"(__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds))
               : "memory");
}
__device__ __forceinline__ void dma16v(const void* gptr, char VDN_LDS* lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gptr),
                  "{m0}"(__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds))
               : "memory");
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier that orders LDS only: each wave waits for its own LDS
// operations, not for its global loads, stores or direct-to-LDS copies in
// flight.  __syncthreads() also makes the wave's global stores visible, i.e.
// waits for every outstanding vector memory operation, including copies
// prefetched for the next step.  The empty asm statements keep the compiler
// from moving memory accesses across the barrier.
// s_waitcnt vmcnt(n) for a wave-uniform count known only at run time
// (n in 1 .. 15; any other value waits for every operation in flight).
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
    case 15: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float sigmoidf(float x) { return 1.0f / (1.0f + __expf(-x)); }

}  // namespace vdn
