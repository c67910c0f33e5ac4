// Device helpers for float32 contractions on the fp16 matrix cores
// (v_mfma_f32_16x16x32_f16): a float32 operand v is split as hi = fp16(v),
// lo = fp16(v - hi), and a product is accumulated as hi.hi + hi.lo + lo.hi in
// float32 (each fp16 x fp16 product is exact in float32), ~22 significant bits
// per operand.  Before the split a group of values is scaled by an exact power
// of two that brings its largest magnitude into [2^14, 2^15): the hi parts
// stay below the fp16 maximum and the lo parts clear of the fp16 subnormals.
#pragma once

#include <hip/hip_runtime.h>

namespace dssm {
namespace mx {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double2 zmul(double2 a, double2 b) {
  return make_double2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

// float32 value v split into fp16 (hi, lo) with hi + lo = v to ~22 bits.
__device__ __forceinline__ void split16(float v, _Float16& hi, _Float16& lo) {
  hi = (_Float16)v;
  lo = (_Float16)(v - (float)hi);
}

// Eight values scaled by 2^sc (exact) and split into an MFMA fragment pair.
__device__ __forceinline__ void split8(const float* v, half8& hi, half8& lo, int sc = 0) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    _Float16 a, b;
    split16(__builtin_amdgcn_ldexpf(v[e], sc), a, b);
    hi[e] = a;
    lo[e] = b;
  }
}

// 8 consecutive floats of LDS starting at a 16-byte aligned address.
__device__ __forceinline__ void lds_read8(const float* p, f4& a, f4& b) {
  a = *reinterpret_cast<const f4*>(p);
  b = *reinterpret_cast<const f4*>(p + 4);
}

// Raw buffer resource over `bytes` bytes at `base`: loads at or beyond
// `bytes` (voffset + instruction offset) return zero, such stores are dropped.
typedef __amdgpu_buffer_rsrc_t BufRes;
__device__ __forceinline__ BufRes buf_res(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Raw buffer over `bytes` bytes at a base the caller knows to be the same in
// every lane: the fields are taken from the first lane, so the descriptor
// lives in scalar registers (no per-lane loop around the access).
__device__ __forceinline__ BufRes buf_res_uniform(const void* base, unsigned bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  const void* p = reinterpret_cast<const void*>(((unsigned long long)hi << 32) | lo);
  return buf_res(p, __builtin_amdgcn_readfirstlane(bytes));
}

// The value of x, hidden from the optimiser: values derived from it are formed
// where they are used, not hoisted out of an enclosing loop and kept live.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// A float32 value the optimiser may not trace back to a wider source: a split
// of (float)d for a double d then converts float32 to fp16 in hardware rather
// than fusing both roundings into a software double-to-fp16 conversion.
__device__ __forceinline__ float opaquef(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Largest x >= 0 over the 16 lanes of a DPP row (non-negative floats order as
// their bit patterns).  Every lane of the wave must be active.
__device__ __forceinline__ float row_max16(float x) {
  int v = __float_as_int(x);
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false));  // row_mirror
  return __int_as_float(v);
}

// Largest x >= 0 over the wave (uniform result).  Every lane must be active.
__device__ __forceinline__ float wave_max(float x) {
  const int v = __float_as_int(row_max16(x));
  const int a = max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16));
  const int b = max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48));
  return __int_as_float(max(a, b));
}

// Power-of-two exponent s that brings a group of values with largest
// magnitude m into [2^14, 2^15) (s = 15 for m = 0).
__device__ __forceinline__ int scale_exp(float m) { return 15 - __builtin_amdgcn_frexp_expf(m); }

__device__ __forceinline__ float amax4(const float* v) {
  return fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
}

}  // namespace mx
}  // namespace dssm
