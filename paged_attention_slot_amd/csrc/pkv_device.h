// Device helpers for the gfx950 (CDNA4) kernels of libpkv: bf16 packing,
// cross-lane reductions with DPP and the gfx950 permlane swaps, exp2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// float -> bfloat16 bits, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// a.lo*b.lo + a.hi*b.hi + c, bf16 pairs in, fp32 accumulate (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A 16-byte load of data read once per pass (the K/V history): marked
// non-temporal, so the stream does not displace reused lines from the L2 and
// last-level caches (measured 8-9 % faster on the decode kernels than plain
// loads).  Coherence across kernels is unchanged.
typedef unsigned u32x4_native_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const u32x4_native_t x = __builtin_nontemporal_load(static_cast<const u32x4_native_t*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// Two OCP e4m3 codes (bytes 0-1 of w, or 2-3 with hi) -> two bf16 in one word,
// the first code in the low half: gfx950's packed conversion with a unit
// scale.  Exact (every finite e4m3 value is a bf16 value); checked bit for bit
// against the fp8 -> f32 conversion for all code pairs without a NaN.
typedef __bf16 bf16x2_native_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
  return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}

// DPP controls (GCN/CDNA encoding).
enum : int {
  kDppQuadXor1 = 0xB1,      // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,      // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141,
  kDppRowRor8 = 0x128,      // row_ror:8 == lane ^ 8 inside a 16-lane row
};

template <int Ctrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), Ctrl, 0xF, 0xF, true));
}

// Sum over each aligned group of 8 lanes; every lane of the group gets it.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  return x;
}

__device__ __forceinline__ float max8(float x) {
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  return x;
}

// Reductions across the 8 lanes that share (lane & 7): lane ^ 8, ^ 16, ^ 32.
__device__ __forceinline__ float sum_across_groups8(float x) {
  x += dpp<kDppRowRor8>(x);
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float max_across_groups8(float x) {
  x = fmaxf(x, dpp<kDppRowRor8>(x));
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Reductions across the 4 lanes that share (lane & 15): lane ^ 16, ^ 32.
__device__ __forceinline__ float sum_across_rows16(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float max_across_rows16(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Whole-wave reductions (every lane of the wave must be active).
__device__ __forceinline__ float wave_sum(float x) { return sum_across_groups8(sum8(x)); }
__device__ __forceinline__ float wave_max(float x) { return max_across_groups8(max8(x)); }

}  // namespace pkv
