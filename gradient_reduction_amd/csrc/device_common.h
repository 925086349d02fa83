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

// Buffer resource word 3 for raw (untyped) buffer accesses on gfx9-class
// GPUs: 32-bit data format, everything else zero.
constexpr int32_t kBufferFlags = 0x00020000;

// One 16-byte store through a buffer resource over `bytes` bytes from
// `row_base`, with cache-policy bits AUX (gfx950: bit 0 sc0, bit 1 nt, bit 4
// sc1).  Offsets at or past `bytes` are dropped by the hardware.
template <int AUX>
__device__ __forceinline__ void store_buf(u32x4* row_base, int32_t bytes, int32_t off, u32x4 v) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(row_base, (short)0, bytes, kBufferFlags);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, AUX);
}

// Cache policies of the planned flush's streams (and of the access-mix
// reference that runs at the same shapes), from an interleaved sweep on the
// 402.8M-element W = 8 flush: stores of tiles that write every row ran 3-4%
// faster with sc0 sc1 nt than with nt alone; one-row tiles 0.5% with nt sc1.
constexpr int kStoreOneRow = 18;   // nt sc1
constexpr int kStoreAllRows = 19;  // sc0 sc1 nt

// ---------------------------------------------------------------------------
// Folding helpers shared by the streaming kernels.  A contribution is
// pre-divided by the communicator size c when PRE is set: a multiply by the
// exact reciprocal inv when c is a power of two (bit-identical to the
// division), a true division otherwise (inv == 0), then rounded to the dtype.
// ---------------------------------------------------------------------------

// The three ways a contribution is pre-divided, as a compile-time mode.
enum : int { kPreNone = 0, kPreMul = 1, kPreDiv = 2 };

template <bool BF16, int MODE>
__device__ __forceinline__ void fold16m(float* acc, u32x4 x, bool first, float inv, float c) {
  if constexpr (BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float a = bf16_lo(x[q]), b = bf16_hi(x[q]);
      if constexpr (MODE == kPreMul) { a *= inv; b *= inv; }
      if constexpr (MODE == kPreDiv) { a = a / c; b = b / c; }
      if constexpr (MODE != kPreNone) bf16_round_pair(a, b);
      acc[2 * q] = first ? a : acc[2 * q] + a;
      acc[2 * q + 1] = first ? b : acc[2 * q + 1] + b;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float a = __uint_as_float(x[q]);
      if constexpr (MODE == kPreMul) a *= inv;
      if constexpr (MODE == kPreDiv) a = a / c;
      acc[q] = first ? a : acc[q] + a;
    }
  }
}

// The mode taken per contribution from the arguments (inv == 0: divide).
template <bool BF16, bool PRE>
__device__ __forceinline__ void fold16(float* acc, u32x4 x, bool first, float inv, float c) {
  if constexpr (!PRE) fold16m<BF16, kPreNone>(acc, x, first, inv, c);
  else if (inv != 0.0f) fold16m<BF16, kPreMul>(acc, x, first, inv, c);
  else fold16m<BF16, kPreDiv>(acc, x, first, inv, c);
}

template <int M>
struct PreMode {
  static constexpr int value = M;
};

// Calls f(PreMode<MODE>{}) once, with the mode that PRE and inv select.
// inv is the same for the whole launch, so this is one uniform branch
// around a whole fold instead of one per contribution (with one per
// contribution, a bf16 fold of 8 rows carried 64 branches and ran 4-9%
// slower).
template <bool PRE, class F>
__device__ __forceinline__ auto with_pre_mode(float inv, F&& f) {
  if constexpr (!PRE) {
    return f(PreMode<kPreNone>{});
  } else {
    if (inv != 0.0f) return f(PreMode<kPreMul>{});
    return f(PreMode<kPreDiv>{});
  }
}

template <bool BF16>
__device__ __forceinline__ u32x4 pack16(const float* acc) {
  u32x4 y;
  if constexpr (BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) y[q] = bf16_pack_out(acc[2 * q], acc[2 * q + 1]);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) y[q] = __float_as_uint(acc[q]);
  }
  return y;
}

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* base, int64_t idx) {
  if constexpr (BF16) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[idx] << 16);
  else return reinterpret_cast<const float*>(base)[idx];
}

template <bool BF16>
__device__ __forceinline__ void store_elem(void* base, int64_t idx, float v) {
  if constexpr (BF16) reinterpret_cast<uint16_t*>(base)[idx] = bf16_out(v);
  else reinterpret_cast<float*>(base)[idx] = v;
}

template <bool BF16>
__device__ __forceinline__ float pre_elem(float x, bool pre, float inv, float c) {
  if (!pre) return x;
  float v = inv != 0.0f ? x * inv : x / c;
  if constexpr (BF16) v = bf16_lo(bf16_pack_rne(v, 0.0f));
  return v;
}

// Block-wide k-ary search over n sorted keys: r1 = #{i : key(i) <= x1},
// r2 = #{i : key(i) < x2}.  Each round the TPB threads of the block probe TPB
// evenly spaced keys of both ranges and keep the bracket the counts point to,
// so n keys take ceil(log_TPB n) rounds.  Every bound is block-uniform and the
// interval shrinks every round, so the loop ends for any key contents.  Every
// thread of the block must call it (it synchronizes).
template <int TPB, class Key>
__device__ void kary_bounds(int32_t n, Key key, int64_t x1, int64_t x2, int32_t& r1, int32_t& r2) {
  int32_t lo1 = 0, hi1 = n, lo2 = 0, hi2 = n;
  while (lo1 < hi1 || lo2 < hi2) {
    const int32_t st1 = (hi1 - lo1 + TPB - 1) / TPB;
    const int32_t st2 = (hi2 - lo2 + TPB - 1) / TPB;
    const int32_t q1 = lo1 + (int32_t)threadIdx.x * st1;
    const int32_t q2 = lo2 + (int32_t)threadIdx.x * st2;
    const bool p1 = lo1 < hi1 && q1 < hi1 && key(q1) <= x1;
    const bool p2 = lo2 < hi2 && q2 < hi2 && key(q2) < x2;
    const int32_t n1 = __syncthreads_count(p1);
    const int32_t n2 = __syncthreads_count(p2);
    if (lo1 < hi1) {
      const int32_t k1 = (hi1 - lo1 + st1 - 1) / st1;
      const int32_t nlo = n1 >= 1 ? lo1 + (n1 - 1) * st1 + 1 : lo1;
      const int32_t nhi = n1 < k1 ? lo1 + n1 * st1 : hi1;
      lo1 = nlo;
      hi1 = nhi;
    }
    if (lo2 < hi2) {
      const int32_t k2 = (hi2 - lo2 + st2 - 1) / st2;
      const int32_t nlo = n2 >= 1 ? lo2 + (n2 - 1) * st2 + 1 : lo2;
      const int32_t nhi = n2 < k2 ? lo2 + n2 * st2 : hi2;
      lo2 = nlo;
      hi2 = nhi;
    }
  }
  r1 = lo1;
  r2 = lo2;
}

// Index of the last of cnt sorted keys (in LDS) that is <= x, or 0.
__device__ __forceinline__ int32_t last_le(const int64_t* key, int32_t cnt, int64_t x) {
  int32_t lo = 0, hi = cnt;
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (key[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace dc
