// Device helpers shared by the gfx950 kernels of libdc.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dc {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

// A bf16 value is the top half of the fp32 with the same bits, so widening
// is a shift or a mask.  Two bf16 share a 32-bit word, element 0 in the low
// half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 pair -> packed bf16 pair, round to nearest even (one
// v_cvt_pk_bf16_f32 on gfx950; fp32 subnormals are kept by the kernel's
// float mode).
__device__ __forceinline__ uint32_t bf16_pack_rne(float a, float b) {
  f32x2 x = {a, b};
  bf16x2 y = __builtin_convertvector(x, bf16x2);
  return __builtin_bit_cast(uint32_t, y);
}

// Same, with every NaN written as the quiet NaN 0x7FC0 carrying its sign.
__device__ __forceinline__ uint32_t bf16_pack_out(float a, float b) {
  uint32_t w = bf16_pack_rne(a, b);
  if (__builtin_isnan(a)) w = (w & 0xFFFF0000u) | ((__float_as_uint(a) >> 16) & 0x8000u) | 0x7FC0u;
  if (__builtin_isnan(b)) w = (w & 0x0000FFFFu) | (__float_as_uint(b) & 0x80000000u) | 0x7FC00000u;
  return w;
}

__device__ __forceinline__ uint16_t bf16_out(float a) {
  return (uint16_t)(bf16_pack_out(a, 0.0f) & 0xFFFFu);
}

// Round a pair to bf16 and widen it back (exact): the dtype rounding of a
// pre-divided contribution.
__device__ __forceinline__ void bf16_round_pair(float& a, float& b) {
  uint32_t w = bf16_pack_rne(a, b);
  a = bf16_lo(w);
  b = bf16_hi(w);
}

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT>
__device__ __forceinline__ void store16(u32x4* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

}  // namespace dc
