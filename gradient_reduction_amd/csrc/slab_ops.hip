// Reduce-scatter, all-gather, replica-local accumulation and the deferred
// reduce for gfx950, plus the bf16 rounding self-check and a plain
// streaming copy used as the achievable-bandwidth reference.
//
// All are streaming kernels over 16-byte column vectors of [rows, ld] slabs:
// every element is read once and written once per destination, nothing is
// reused, so they are HBM bound.  Sizes whose shard boundaries are not
// vector aligned run an element-wise variant.
#include "device_common.h"
#include "internal.h"

namespace dc {
namespace {

// Vectors (or elements) per thread per launch tile, per kernel.
#ifndef DC_RS_U
#define DC_RS_U 1
#endif
#ifndef DC_AG_U
#define DC_AG_U 2
#endif
#ifndef DC_ACC_U
#define DC_ACC_U 1
#endif
#ifndef DC_DEF_U
#define DC_DEF_U 1
#endif
#ifndef DC_COPY_U
#define DC_COPY_U 1
#endif
#ifndef DC_SLAB_NT
#define DC_SLAB_NT 1      // nontemporal loads (every input is read once)
#endif
#ifndef DC_SLAB_NTS
#define DC_SLAB_NTS 1     // nontemporal stores (reduce-scatter, accumulate, reduce, copy)
#endif
#ifndef DC_AG_NTS
#define DC_AG_NTS 0       // nontemporal stores in the all-gather
#endif
#ifndef DC_SLAB_TPB
#define DC_SLAB_TPB 64    // threads per workgroup: one wave; small tiles measured
                          // 2-6% faster than 256-thread ones on every kernel here
#endif
constexpr int kST = DC_SLAB_TPB;
constexpr bool kNT = DC_SLAB_NT != 0;
constexpr bool kNTS = DC_SLAB_NTS != 0;
constexpr bool kAgNTS = DC_AG_NTS != 0;

// Cache policy of the result stores (gfx950 bits: 0 sc0, 1 nt, 4 sc1; < 0:
// nontemporal global stores), from an interleaved sweep at the bench shapes:
// the reduce-scatters (one row written per vector folded) ran the same with
// every policy tried and keep nontemporal stores; the accumulate ran about
// 1% faster with nt sc1, and the kernels that write several rows (the
// deferred reduce, 6.64 against 6.41-6.55 TB/s, and the fused
// accumulate-reduce, 6.14-6.36 against 6.00-6.25) with nt sc1 as well.
#ifndef DC_SLAB_SP1
#define DC_SLAB_SP1 -1
#endif
#ifndef DC_SLAB_SPACC
#define DC_SLAB_SPACC 18
#endif
#ifndef DC_SLAB_SPN
#define DC_SLAB_SPN 18
#endif

// Store vector k of a row whose workgroup covers the run of vectors
// [t0, t0 + n) (t0 and n the same for the whole workgroup): through a buffer
// resource over the run with cache bits SP, or a nontemporal global store.
template <int SP>
__device__ __forceinline__ void store_run(u32x4* row, int64_t t0, int64_t n, int64_t k, u32x4 v) {
  if constexpr (SP < 0) {
    store16<kNTS>(row + k, v);
  } else {
    store_buf<SP>(row + t0, (int32_t)(n * 16), (int32_t)((k - t0) * 16), v);
  }
}

// Fold the W rows of vector column `v` (rows `ldv` vectors apart).  With W
// known at compile time every row load is issued before the first add.
template <bool BF16, int WT, int MODE>
__device__ __forceinline__ u32x4 fold_rows_m(const u32x4* in, int64_t ldv, int64_t v, int32_t W,
                                             float inv, float c) {
  constexpr int E = BF16 ? 8 : 4;
  float acc[E];
  if constexpr (WT > 0) {
    u32x4 x[WT];
#pragma unroll
    for (int r = 0; r < WT; ++r) x[r] = load16<kNT>(in + r * ldv + v);
#pragma unroll
    for (int r = 0; r < WT; ++r) fold16m<BF16, MODE>(acc, x[r], r == 0, inv, c);
  } else {
#pragma unroll 4
    for (int32_t r = 0; r < W; ++r) fold16m<BF16, MODE>(acc, load16<kNT>(in + r * ldv + v), r == 0, inv, c);
  }
  return pack16<BF16>(acc);
}

template <bool BF16, int WT, bool PRE>
__device__ __forceinline__ u32x4 fold_rows(const u32x4* in, int64_t ldv, int64_t v, int32_t W,
                                           float inv, float c) {
  return with_pre_mode<PRE>(inv, [&](auto m) {
    return fold_rows_m<BF16, WT, decltype(m)::value>(in, ldv, v, W, inv, c);
  });
}

// ---------------------------------------------------------------------------
// Reduce-scatter: out[s][k] = fold_r pre(in[r][s*L + k])
// ---------------------------------------------------------------------------

// Vector path (L a multiple of the vector width): blockIdx.y = shard.
template <bool BF16, int WT, bool PRE>
__global__ __launch_bounds__(kST) void k_rs_vec(int32_t W, const u32x4* __restrict__ in,
                                                     int64_t ldv_in, u32x4* __restrict__ out,
                                                     int64_t ldv_out, int64_t Lv, float inv,
                                                     float c) {
  const int64_t s = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * (kST * DC_RS_U);
  const int64_t n = min((int64_t)(kST * DC_RS_U), Lv - t0);
#pragma unroll
  for (int u = 0; u < DC_RS_U; ++u) {
    const int64_t k = t0 + threadIdx.x + (int64_t)u * kST;
    if (k < Lv)
      store_run<DC_SLAB_SP1>(out + s * ldv_out, t0, n, k,
                             fold_rows<BF16, WT, PRE>(in, ldv_in, s * Lv + k, W, inv, c));
  }
}

template <bool BF16>
__global__ __launch_bounds__(kST) void k_rs_elem(int32_t W, const void* __restrict__ in,
                                                      int64_t ld_in, void* __restrict__ out,
                                                      int64_t ld_out, int64_t L, int32_t pre,
                                                      float inv, float c) {
  const int64_t s = blockIdx.y;
  const int64_t k0 = (int64_t)blockIdx.x * (kST * DC_RS_U) + threadIdx.x;
  for (int u = 0; u < DC_RS_U; ++u) {
    const int64_t k = k0 + (int64_t)u * kST;
    if (k >= L) continue;
    float acc = 0.0f;
    for (int32_t r = 0; r < W; ++r) {
      const float v = pre_elem<BF16>(load_elem<BF16>(in, r * ld_in + s * L + k), pre != 0, inv, c);
      acc = r == 0 ? v : acc + v;
    }
    store_elem<BF16>(out, s * ld_out + k, acc);
  }
}

// Reduce-scatter with variable shards (after a relayout): shard q is
// columns [seg[q], seg[q+1]) of the input; out[q][k] = fold_r pre(in[r][seg[q]+k]).
// Shards start wherever the relayout's packed segments do, so a shard's
// input is usually not vector aligned while its output row is: each full
// output vector is cut out of the two aligned input vectors around it
// (funnel16, with the block-uniform offset of the shard), folded and stored
// aligned.  The partial last vector of a shard goes element by element.
struct SegArgs {
  int64_t seg[DC_MAX_W + 1];
  int64_t bpre[DC_MAX_W + 1];   // first workgroup of each shard (prefix of its workgroup counts)
};

// A shard's workgroups start kRsvAlign-aligned in absolute input vectors:
// lanes in front of the shard idle, and every wave reads whole cache lines.
constexpr int64_t kRsvAlign = 64;

// The 16 bytes that start `wo` words + `bs` bytes (wo in 0..3, bs in {0, 2})
// into the 32 bytes a:b; wo and bs are the same for the whole block.
__device__ __forceinline__ u32x4 funnel16(u32x4 a, u32x4 b, int wo, int bs) {
  const uint32_t c[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  uint32_t w[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const uint32_t x01 = (wo & 1) ? c[j + 1] : c[j];
    const uint32_t x23 = (wo & 1) ? c[j + 3] : c[j + 2];
    w[j] = (wo & 2) ? x23 : x01;
  }
  u32x4 y;
#pragma unroll
  for (int j = 0; j < 4; ++j) y[j] = __builtin_amdgcn_alignbyte(w[j + 1], w[j], bs);
  return y;
}

template <bool BF16, int WT, bool PRE>
__global__ __launch_bounds__(kST) void k_rs_v(int32_t W, const void* __restrict__ in,
                                                   int64_t ld_in, void* __restrict__ out,
                                                   int64_t ld_out, SegArgs sa, float inv, float c) {
  constexpr int E = BF16 ? 8 : 4;
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int QMAX = WT > 0 ? WT : DC_MAX_W;
  // the shard of this workgroup: the grid covers exactly the shards' vectors,
  // shard after shard (compile-time indices into the argument arrays)
  const int64_t blk = blockIdx.x;
  int32_t q = 0;
  int64_t s0 = sa.seg[0], s1 = sa.seg[1], b0 = 0;
#pragma unroll
  for (int i = 1; i < QMAX; ++i) {
    if (i < W && blk >= sa.bpre[i]) {
      q = i;
      s0 = sa.seg[i];
      s1 = sa.seg[i + 1];
      b0 = sa.bpre[i];
    }
  }
  const int64_t len = s1 - s0;
  const int64_t k = (blk - b0) * kST + threadIdx.x - (s0 / E) % kRsvAlign;
  if (k < 0 || k * E >= len) return;
  const int64_t ldv = ld_in / E;
  const int32_t o = (int32_t)(s0 % E);
  if ((k + 1) * E <= len) {
    u32x4 y;
    if (o == 0) {
      y = fold_rows<BF16, WT, PRE>(reinterpret_cast<const u32x4*>(in), ldv, s0 / E + k, W, inv, c);
    } else {
      // input vectors v and v+1 hold the window; v+1 ends inside the row
      // because the window does and rows are whole vectors long
      const u32x4* in4 = reinterpret_cast<const u32x4*>(in);
      const int64_t v = s0 / E + k;
      const int wo = (o * EB) >> 2, bs = (o * EB) & 3;
      float acc[E];
      if constexpr (WT > 0) {
        u32x4 a[WT], b[WT];
#pragma unroll
        for (int r = 0; r < WT; ++r) {
          a[r] = load16<kNT>(in4 + r * ldv + v);
          b[r] = load16<kNT>(in4 + r * ldv + v + 1);
        }
        with_pre_mode<PRE>(inv, [&](auto m) {
#pragma unroll
          for (int r = 0; r < WT; ++r)
            fold16m<BF16, decltype(m)::value>(acc, funnel16(a[r], b[r], wo, bs), r == 0, inv, c);
        });
      } else {
        for (int32_t r = 0; r < W; ++r)
          fold16<BF16, PRE>(acc, funnel16(load16<kNT>(in4 + r * ldv + v), load16<kNT>(in4 + r * ldv + v + 1), wo, bs),
                            r == 0, inv, c);
      }
      y = pack16<BF16>(acc);
    }
    store16<kNTS>(reinterpret_cast<u32x4*>(out) + q * (ld_out / E) + k, y);
  } else {
    const int64_t e1 = min((k + 1) * E, len);
    for (int64_t e = k * E; e < e1; ++e) {
      float acc = 0.0f;
      for (int32_t r = 0; r < W; ++r) {
        const float v = pre_elem<BF16>(load_elem<BF16>(in, r * ld_in + s0 + e), PRE, inv, c);
        acc = r == 0 ? v : acc + v;
      }
      store_elem<BF16>(out, q * ld_out + e, acc);
    }
  }
}

// Ring-order reduce-scatter: shard s folded in rank order s, s+1, ..., s-1
// (mod W), the order in which a ring passes the partial sums along.  The
// rows are loaded in that order, so the register array is indexed
// statically.
template <bool BF16, int WT, bool PRE>
__global__ __launch_bounds__(kST) void k_rs_ring(int32_t W, const u32x4* __restrict__ in,
                                                      int64_t ldv_in, u32x4* __restrict__ out,
                                                      int64_t ldv_out, int64_t Lv, float inv,
                                                      float c) {
  constexpr int E = BF16 ? 8 : 4;
  const int32_t s = blockIdx.y;
  const int64_t k = (int64_t)blockIdx.x * kST + threadIdx.x;
  if (k >= Lv) return;
  const int64_t v = (int64_t)s * Lv + k;
  float acc[E];
  if constexpr (WT > 0) {
    u32x4 x[WT];
#pragma unroll
    for (int j = 0; j < WT; ++j) x[j] = load16<kNT>(in + (int64_t)((s + j) % WT) * ldv_in + v);
    with_pre_mode<PRE>(inv, [&](auto m) {
#pragma unroll
      for (int j = 0; j < WT; ++j) fold16m<BF16, decltype(m)::value>(acc, x[j], j == 0, inv, c);
    });
  } else {
    for (int32_t j = 0; j < W; ++j)
      fold16<BF16, PRE>(acc, load16<kNT>(in + (int64_t)((s + j) % W) * ldv_in + v), j == 0, inv, c);
  }
  const int64_t t0 = (int64_t)blockIdx.x * kST;
  store_run<DC_SLAB_SP1>(out + (int64_t)s * ldv_out, t0, min((int64_t)kST, Lv - t0), k,
                         pack16<BF16>(acc));
}

template <bool BF16>
__global__ __launch_bounds__(kST) void k_rs_ring_elem(int32_t W, const void* __restrict__ in,
                                                           int64_t ld_in, void* __restrict__ out,
                                                           int64_t ld_out, int64_t L, int32_t pre,
                                                           float inv, float c) {
  const int32_t s = blockIdx.y;
  const int64_t k = (int64_t)blockIdx.x * kST + threadIdx.x;
  if (k >= L) return;
  float acc = 0.0f;
  for (int32_t j = 0; j < W; ++j) {
    const float v = pre_elem<BF16>(load_elem<BF16>(in, (int64_t)((s + j) % W) * ld_in + (int64_t)s * L + k),
                                   pre != 0, inv, c);
    acc = j == 0 ? v : acc + v;
  }
  store_elem<BF16>(out, (int64_t)s * ld_out + k, acc);
}

// ---------------------------------------------------------------------------
// All-gather
// ---------------------------------------------------------------------------

// One step of an all-gather schedule on the [W, W*L] buffer, every chunk at
// its own index.  Transfer t of node i at step `step`:
//   step 0: node i places its own shard (from `in`);
//   ring: chunk (i - step) mod W from node i-1;
//   bidirectional ring: t = 0 chunk (i - step) mod W from node i-1, t = 1
//     chunk (i + step) mod W from node i+1 (not when the two coincide);
//   recursive doubling: the 2^(step-1) chunks of node i XOR 2^(step-1).
// Every chunk a step reads was placed by an earlier step, and every chunk it
// writes is new, so one launch per step is race free.
__device__ __forceinline__ bool ag_transfer(int32_t W, int32_t algo, int32_t step, int32_t i,
                                            int32_t t, int32_t* src, int32_t* chunk) {
  if (step == 0) {
    *src = -1;
    *chunk = i;
    return t == 0;
  }
  if (algo == 0) {
    *src = (i - 1 + W) % W;
    *chunk = ((i - step) % W + W) % W;
    return t == 0;
  }
  if (algo == 1) {
    if (t == 0) {
      *src = (i - 1 + W) % W;
      *chunk = ((i - step) % W + W) % W;
      return true;
    }
    *src = (i + 1) % W;
    *chunk = (i + step) % W;
    return t == 1 && (2 * step) % W != 0;
  }
  const int32_t d = 1 << (step - 1);
  *src = i ^ d;
  *chunk = (*src & ~(d - 1)) + t;
  return t < d;
}

template <int EB>
__global__ __launch_bounds__(kST) void k_ag_step(int32_t W, const char* __restrict__ in,
                                                      int64_t ld_in, char* out, int64_t ld_out,
                                                      int64_t L, int32_t algo, int32_t step) {
  constexpr int E = 16 / EB;
  const int32_t i = blockIdx.y, t = blockIdx.z;
  int32_t src, chunk;
  if (!ag_transfer(W, algo, step, i, t, &src, &chunk)) return;
  const int64_t k = (int64_t)blockIdx.x * kST + threadIdx.x;
  const char* from = src < 0 ? in + (int64_t)i * ld_in * EB
                             : out + ((int64_t)src * ld_out + (int64_t)chunk * L) * EB;
  char* to = out + ((int64_t)i * ld_out + (int64_t)chunk * L) * EB;
  if (L % E == 0) {
    if (k < L / E)
      store16<kAgNTS>(reinterpret_cast<u32x4*>(to) + k, load16<kNT>(reinterpret_cast<const u32x4*>(from) + k));
  } else {
    for (int64_t e = k * E; e < min((k + 1) * E, L); ++e) {
      if constexpr (EB == 2)
        reinterpret_cast<uint16_t*>(to)[e] = reinterpret_cast<const uint16_t*>(from)[e];
      else
        reinterpret_cast<uint32_t*>(to)[e] = reinterpret_cast<const uint32_t*>(from)[e];
    }
  }
}

// Thread (s, k) reads chunk s's vector k once and writes it wherever node i
// keeps chunk s: position s (rank order) or (i - s) mod W (ring order).  In
// step mode only chunk `step` (rank) or position `step` (ring) is written.
// Each workgroup covers U runs of 64 vectors of one chunk; a full one stores
// through buffer resources with cache-policy bits SP (SP < 0: plain stores),
// a partial one with plain stores.
template <int U, int SP>
__global__ __launch_bounds__(kST) void k_ag_vec(int32_t W, const u32x4* __restrict__ in,
                                                int64_t ldv_in, u32x4* __restrict__ out,
                                                int64_t ldv_out, int64_t Lv, int32_t order,
                                                int32_t step) {
  const int32_t s = blockIdx.y;
  if (order == DC_ORDER_RANK && step >= 0 && s != step) return;
  const int64_t t0 = (int64_t)blockIdx.x * (kST * U);
  const bool full = t0 + kST * U <= Lv;
  u32x4 x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t k = t0 + threadIdx.x + (int64_t)u * kST;
    if (k < Lv) x[u] = load16<kNT>(in + (int64_t)s * ldv_in + k);
  }
  for (int32_t i = 0; i < W; ++i) {
    const int32_t p = order == DC_ORDER_RANK ? s : (i - s + W) % W;
    if (order == DC_ORDER_RING && step >= 0 && p != step) continue;
    u32x4* base = out + (int64_t)i * ldv_out + (int64_t)p * Lv + t0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t j = (int32_t)threadIdx.x + u * kST;
      if (SP >= 0 && full) {
        store_buf<(SP >= 0 ? SP : 0)>(base, kST * U * 16, j * 16, x[u]);
      } else if (t0 + j < Lv) {
        store16<kAgNTS>(base + j, x[u]);
      }
    }
  }
}

template <typename E>
__global__ __launch_bounds__(kST) void k_ag_elem(int32_t W, const E* __restrict__ in,
                                                      int64_t ld_in, E* __restrict__ out,
                                                      int64_t ld_out, int64_t L, int32_t order,
                                                      int32_t step) {
  const int32_t s = blockIdx.y;
  if (order == DC_ORDER_RANK && step >= 0 && s != step) return;
  const int64_t k0 = (int64_t)blockIdx.x * (kST * DC_AG_U) + threadIdx.x;
  for (int u = 0; u < DC_AG_U; ++u) {
    const int64_t k = k0 + (int64_t)u * kST;
    if (k >= L) continue;
    const E x = in[(int64_t)s * ld_in + k];
    for (int32_t i = 0; i < W; ++i) {
      const int32_t p = order == DC_ORDER_RANK ? s : (i - s + W) % W;
      if (order == DC_ORDER_RING && step >= 0 && p != step) continue;
      out[(int64_t)i * ld_out + (int64_t)p * L + k] = x;
    }
  }
}

// ---------------------------------------------------------------------------
// Accumulate: acc = acc + x   (init: acc = +0 + x)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kST) void k_accumulate(const float* __restrict__ x,
                                                         int64_t ld_x, float* acc,
                                                         int64_t ld_acc, int64_t M, int32_t init) {
  const int64_t r = blockIdx.y;
  const int64_t nvec = M / 4;
  const int64_t k0 = (int64_t)blockIdx.x * (kST * DC_ACC_U) + threadIdx.x;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x + r * ld_x);
  u32x4* av = reinterpret_cast<u32x4*>(acc + r * ld_acc);
#pragma unroll
  for (int u = 0; u < DC_ACC_U; ++u) {
    const int64_t k = k0 + (int64_t)u * kST;
    if (k < nvec) {
      const u32x4 xx = load16<kNT>(xv + k);
      u32x4 aa;
      if (init) {
        aa = u32x4{0u, 0u, 0u, 0u};
      } else {
        aa = load16<kNT>(av + k);
      }
      u32x4 y;
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = __float_as_uint(__uint_as_float(aa[q]) + __uint_as_float(xx[q]));
      const int64_t t0 = (int64_t)blockIdx.x * (kST * DC_ACC_U);
      store_run<DC_SLAB_SPACC>(av, t0, min((int64_t)(kST * DC_ACC_U), nvec - t0), k, y);
    } else if (k == nvec) {
      for (int64_t j = nvec * 4; j < M; ++j) {
        const float a = init ? 0.0f : acc[r * ld_acc + j];
        acc[r * ld_acc + j] = a + x[r * ld_x + j];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Deferred reduce: out[i][j] = fold_r acc[r][j], i < out_rows
// ---------------------------------------------------------------------------
template <int WT>
__global__ __launch_bounds__(kST) void k_deferred(int32_t W, const float* acc, int64_t ld_acc,
                                                       float* out, int64_t ld_out, int64_t M,
                                                       int32_t out_rows) {
  const int64_t nvec = M / 4;
  const int64_t k0 = (int64_t)blockIdx.x * (kST * DC_DEF_U) + threadIdx.x;
  const u32x4* in = reinterpret_cast<const u32x4*>(acc);
  u32x4* ov = reinterpret_cast<u32x4*>(out);
#pragma unroll
  for (int u = 0; u < DC_DEF_U; ++u) {
    const int64_t k = k0 + (int64_t)u * kST;
    if (k < nvec) {
      const u32x4 y = fold_rows<false, WT, false>(in, ld_acc / 4, k, W, 0.0f, 1.0f);
      const int64_t t0 = (int64_t)blockIdx.x * (kST * DC_DEF_U);
      const int64_t n = min((int64_t)(kST * DC_DEF_U), nvec - t0);
      for (int32_t i = 0; i < out_rows; ++i) store_run<DC_SLAB_SPN>(ov + i * (ld_out / 4), t0, n, k, y);
    } else if (k == nvec) {
      for (int64_t j = nvec * 4; j < M; ++j) {
        float sum = 0.0f;
        for (int32_t r = 0; r < W; ++r) sum = r == 0 ? acc[r * ld_acc + j] : sum + acc[r * ld_acc + j];
        for (int32_t i = 0; i < out_rows; ++i) out[i * ld_out + j] = sum;
      }
    }
  }
}

// Accumulate and deferred reduce fused: a_r = acc_r + x_r (or +0 + x_r), optionally kept, then
// folded in rank order.  W known at compile time loads every row first.
template <int WT>
__global__ __launch_bounds__(kST) void k_accum_reduce(int32_t W, const float* x, int64_t ld_x,
                                                           float* acc, int64_t ld_acc, int32_t init,
                                                           int32_t keep, float* out, int64_t ld_out,
                                                           int32_t out_rows, int64_t M) {
  const int64_t nvec = M / 4;
  const int64_t k = (int64_t)blockIdx.x * kST + threadIdx.x;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  u32x4* av = reinterpret_cast<u32x4*>(acc);
  u32x4* ov = reinterpret_cast<u32x4*>(out);
  const int64_t lx = ld_x / 4, la = ld_acc / 4, lo = ld_out / 4;
  const int64_t t0 = (int64_t)blockIdx.x * kST, n = min((int64_t)kST, nvec - t0);
  if (k < nvec) {
    float sum[4];
    constexpr int RB = WT > 0 ? WT : 4;  // rows per batch of loads
    for (int32_t r0 = 0; r0 < W; r0 += RB) {
      u32x4 xx[RB], aa[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        if (WT == 0 && r0 + i >= W) break;
        xx[i] = load16<kNT>(xv + (r0 + i) * lx + k);
        aa[i] = init ? u32x4{0u, 0u, 0u, 0u} : load16<kNT>(av + (r0 + i) * la + k);
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        if (WT == 0 && r0 + i >= W) break;
        u32x4 a;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v = __uint_as_float(aa[i][q]) + __uint_as_float(xx[i][q]);
          a[q] = __float_as_uint(v);
          sum[q] = (r0 + i) == 0 ? v : sum[q] + v;
        }
        if (keep) store_run<DC_SLAB_SPN>(av + (r0 + i) * la, t0, n, k, a);
      }
    }
    const u32x4 y = u32x4{__float_as_uint(sum[0]), __float_as_uint(sum[1]), __float_as_uint(sum[2]),
                          __float_as_uint(sum[3])};
    for (int32_t i = 0; i < out_rows; ++i) store_run<DC_SLAB_SPN>(ov + i * lo, t0, n, k, y);
  } else if (k == nvec) {
    for (int64_t j = nvec * 4; j < M; ++j) {
      float s = 0.0f;
      for (int32_t r = 0; r < W; ++r) {
        const float a = (init ? 0.0f : acc[r * ld_acc + j]) + x[r * ld_x + j];
        if (keep) acc[r * ld_acc + j] = a;
        s = r == 0 ? a : s + a;
      }
      for (int32_t i = 0; i < out_rows; ++i) out[i * ld_out + j] = s;
    }
  }
}

__global__ __launch_bounds__(kST) void k_round_bf16(const float* __restrict__ in,
                                                         uint16_t* __restrict__ out, int64_t n) {
  const int64_t step = (int64_t)gridDim.x * kST;
  for (int64_t i = (int64_t)blockIdx.x * kST + threadIdx.x; i < n; i += step) out[i] = bf16_out(in[i]);
}

__global__ __launch_bounds__(kST) void k_copy(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t nvec) {
  const int64_t k0 = (int64_t)blockIdx.x * (kST * DC_COPY_U) + threadIdx.x;
#pragma unroll
  for (int u = 0; u < DC_COPY_U; ++u) {
    const int64_t k = k0 + (int64_t)u * kST;
    if (k < nvec) store16<kNTS>(dst + k, load16<kNT>(src + k));
  }
}

// Access-mix reference: R rows read, NW rows written, xor only.
template <int R, int NW>
__global__ __launch_bounds__(kST) void k_stream_rows(const u32x4* __restrict__ src,
                                                          int64_t sld, u32x4* __restrict__ dst,
                                                          int64_t dld, int64_t nvec) {
  const int64_t k = (int64_t)blockIdx.x * kST + threadIdx.x;
  if (k >= nvec) return;
  u32x4 x[R];
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = load16<kNT>(src + r * sld + k);
  u32x4 y = x[0];
#pragma unroll
  for (int r = 1; r < R; ++r) y ^= x[r];
#pragma unroll
  for (int r = 0; r < NW; ++r) store16<kNTS>(dst + r * dld + k, y);
}

// The same mix at a launch shape of the planned kernels: each one-wave
// workgroup takes G runs of 64 vectors; with one row written the G results
// are stored together after the last load, with several rows written each
// vector's rows are stored as soon as it is folded (R = 1 is the
// all-gather's one-row-to-every-row mix); stores use the planned flush's
// cache policies.  A workgroup short of G full runs (the tail) goes vector
// by vector.
template <int R, int NW, int G>
__global__ __launch_bounds__(kST) void k_stream_rows_g(const u32x4* __restrict__ src,
                                                       int64_t sld, u32x4* __restrict__ dst,
                                                       int64_t dld, int64_t nvec) {
  static_assert(kST == 64, "runs of one vector per thread of a wave");
  const int64_t v0 = (int64_t)blockIdx.x * (kST * G);
  if (v0 + kST * G <= nvec) {
    constexpr int32_t bytes = G * kST * 16;
    if constexpr (NW == 1) {
      u32x4 y[G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int64_t k = v0 + j * kST + threadIdx.x;
        u32x4 x[R];
#pragma unroll
        for (int r = 0; r < R; ++r) x[r] = load16<kNT>(src + r * sld + k);
        y[j] = x[0];
#pragma unroll
        for (int r = 1; r < R; ++r) y[j] ^= x[r];
      }
#pragma unroll
      for (int j = 0; j < G; ++j) store_buf<kStoreOneRow>(dst + v0, bytes, (j * kST + threadIdx.x) * 16, y[j]);
    } else {
#pragma unroll 1
      for (int j = 0; j < G; ++j) {
        const int64_t k = v0 + j * kST + threadIdx.x;
        u32x4 x[R];
#pragma unroll
        for (int r = 0; r < R; ++r) x[r] = load16<kNT>(src + r * sld + k);
        u32x4 y = x[0];
#pragma unroll
        for (int r = 1; r < R; ++r) y ^= x[r];
#pragma unroll
        for (int r = 0; r < NW; ++r)
          store_buf<kStoreAllRows>(dst + r * dld + v0, bytes, (j * kST + threadIdx.x) * 16, y);
      }
    }
    return;
  }
#pragma unroll 1
  for (int j = 0; j < G; ++j) {
    const int64_t k = v0 + j * kST + threadIdx.x;
    if (k >= nvec) break;
    u32x4 x[R];
#pragma unroll
    for (int r = 0; r < R; ++r) x[r] = load16<kNT>(src + r * sld + k);
    u32x4 y = x[0];
#pragma unroll
    for (int r = 1; r < R; ++r) y ^= x[r];
#pragma unroll
    for (int r = 0; r < NW; ++r) store16<kNTS>(dst + r * dld + k, y);
  }
}

// Row accesses in flight per compute unit (KB) at which each kernel below
// measured fastest, 5-10% over a full compute unit, in interleaved sweeps
// on the 7B-layer reduce-scatter / all-gather (W = 8), the relaid buckets of
// the 402.8M-element gradient and the W = 4 deferred reduce.  The
// reduce-scatters in rank and ring order run at 9 workgroups per compute
// unit at W = 8 (ring order 6.93 TB/s, against 6.71 at 10 and 6.31 at 16;
// rank order 6.64 against 6.57 at 10 and 6.43 at 12); the variable-shard
// one at 10 (6.62, against 6.53 at 8 or 9 and 6.34 uncapped).  Other W keep
// the same budget.
#ifndef DC_KB_RS
#define DC_KB_RS 84
#endif
#ifndef DC_KB_RS_RING
#define DC_KB_RS_RING 84
#endif
#ifndef DC_KB_RSV
#define DC_KB_RSV 96
#endif
#ifndef DC_KB_DEFERRED
#define DC_KB_DEFERRED 96
#endif
#ifndef DC_KB_ACCRED
#define DC_KB_ACCRED 120
#endif
constexpr int kKbRs = DC_KB_RS, kKbRsRing = DC_KB_RS_RING, kKbRsv = DC_KB_RSV,
              kKbDeferred = DC_KB_DEFERRED, kKbAccRed = DC_KB_ACCRED;

// All-gather launch shapes (vectors per thread, store policy; workgroups per
// compute unit), from interleaved sweeps on the 7B-layer all-gather (W = 8
// bf16, 25.3M-element shards): one vector per thread with sc0 sc1 nt stores
// ran at 6.07 TB/s in rank order at 12 workgroups per compute unit and 6.20
// in ring order at 12 (6.12 at 16), against 5.62-5.69 for two vectors per
// thread with plain stores at 8.
#ifndef DC_AG_RANK_SHAPE
#define DC_AG_RANK_SHAPE 1, 19
#endif
#ifndef DC_AG_RANK_CAP
#define DC_AG_RANK_CAP 12
#endif
#ifndef DC_AG_RING_SHAPE
#define DC_AG_RING_SHAPE 1, 19
#endif
#ifndef DC_AG_RING_CAP
#define DC_AG_RING_CAP 12
#endif


// The dynamic LDS that caps a launch of `kern` at `cap` workgroups per compute unit.
template <typename K>
size_t pad_for(K* kern, int cap) {
  return occupancy_pad(reinterpret_cast<const void*>(kern), cap);
}

inline unsigned blocks_for(int64_t n, int u) {
  return (unsigned)((n + kST * u - 1) / (kST * u));
}
template <int U, int SP>
void launch_ag_vec(int32_t W, const u32x4* in, int64_t ldv_in, u32x4* out, int64_t ldv_out,
                   int64_t Lv, int32_t order, int32_t step, int cap, hipStream_t stream) {
  hipLaunchKernelGGL((k_ag_vec<U, SP>), dim3(blocks_for(Lv, U), (unsigned)W), dim3(kST),
                     pad_for(k_ag_vec<U, SP>, cap), stream, W, in, ldv_in, out, ldv_out, Lv, order,
                     step);
}


inline void reciprocal(int32_t c, float* inv, float* cf) {
  *cf = (float)c;
  *inv = (c & (c - 1)) == 0 ? 1.0f / (float)c : 0.0f;  // exact for powers of two
}

template <bool BF16, bool PRE>
hipError_t rs_vec_w(int32_t W, const void* in, int64_t ld_in, void* out, int64_t ld_out, int64_t L,
                    float inv, float c, hipStream_t stream) {
  constexpr int E = BF16 ? 8 : 4;
  const int64_t Lv = L / E;
  const dim3 grid(blocks_for(Lv, DC_RS_U), (unsigned)W);
  const int cap = stream_cap(W + 1, DC_RS_U, kKbRs);
  const u32x4* i4 = reinterpret_cast<const u32x4*>(in);
  u32x4* o4 = reinterpret_cast<u32x4*>(out);
  switch (W) {
#define DC_RS_W(w)                                                                           \
  case w:                                                                                    \
    hipLaunchKernelGGL((k_rs_vec<BF16, w, PRE>), grid, dim3(kST),                            \
                       pad_for(k_rs_vec<BF16, w, PRE>, cap), stream, W, i4,                  \
                       ld_in / E, o4, ld_out / E, Lv, inv, c);                               \
    break;
    DC_RS_W(1)
    DC_RS_W(2)
    DC_RS_W(4)
    DC_RS_W(8)
    DC_RS_W(16)
#undef DC_RS_W
    default:
      hipLaunchKernelGGL((k_rs_vec<BF16, 0, PRE>), grid, dim3(kST),
                         pad_for(k_rs_vec<BF16, 0, PRE>, cap), stream, W, i4,
                         ld_in / E, o4, ld_out / E, Lv, inv, c);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce_scatter(int32_t W, int32_t dtype, const void* in, int64_t ld_in,
                                 void* out, int64_t ld_out, int64_t M, int32_t pre_div,
                                 hipStream_t stream) {
  const int64_t L = M / W;
  if (L == 0) return hipSuccess;
  float inv, c;
  reciprocal(W, &inv, &c);
  const bool bf = dtype == DC_BF16;
  const int E = bf ? 8 : 4;
  if (L % E == 0) {
    if (bf) return pre_div ? rs_vec_w<true, true>(W, in, ld_in, out, ld_out, L, inv, c, stream)
                           : rs_vec_w<true, false>(W, in, ld_in, out, ld_out, L, inv, c, stream);
    return pre_div ? rs_vec_w<false, true>(W, in, ld_in, out, ld_out, L, inv, c, stream)
                   : rs_vec_w<false, false>(W, in, ld_in, out, ld_out, L, inv, c, stream);
  }
  const dim3 grid(blocks_for(L, DC_RS_U), (unsigned)W);
  if (bf)
    hipLaunchKernelGGL(k_rs_elem<true>, grid, dim3(kST), 0, stream, W, in, ld_in, out, ld_out,
                       L, pre_div, inv, c);
  else
    hipLaunchKernelGGL(k_rs_elem<false>, grid, dim3(kST), 0, stream, W, in, ld_in, out,
                       ld_out, L, pre_div, inv, c);
  return hipGetLastError();
}

template <bool BF16, bool PRE>
hipError_t rs_v_w(int32_t W, const void* in, int64_t ld_in, void* out, int64_t ld_out,
                  const SegArgs& sa, int64_t maxlen, float inv, float c, hipStream_t stream) {
  const dim3 grid((unsigned)sa.bpre[W]);
  (void)maxlen;
  const int cap = stream_cap(W + 1, 1, kKbRsv);
  switch (W) {
#define DC_RSV_W(w)                                                                          \
  case w:                                                                                    \
    hipLaunchKernelGGL((k_rs_v<BF16, w, PRE>), grid, dim3(kST),                              \
                       pad_for(k_rs_v<BF16, w, PRE>, cap), stream, W, in, ld_in, out, ld_out, \
                       sa, inv, c);                                                          \
    break;
    DC_RSV_W(1)
    DC_RSV_W(2)
    DC_RSV_W(4)
    DC_RSV_W(8)
    DC_RSV_W(16)
#undef DC_RSV_W
    default:
      hipLaunchKernelGGL((k_rs_v<BF16, 0, PRE>), grid, dim3(kST), pad_for(k_rs_v<BF16, 0, PRE>, cap),
                         stream, W, in, ld_in, out, ld_out, sa, inv, c);
  }
  return hipGetLastError();
}

hipError_t launch_reduce_scatter_v(int32_t W, int32_t dtype, const void* in, int64_t ld_in,
                                   void* out, int64_t ld_out, const int64_t* seg_start,
                                   int32_t pre_div, hipStream_t stream) {
  SegArgs sa{};
  int64_t maxlen = 0;
  const int64_t E = dtype == DC_BF16 ? 8 : 4;
  for (int q = 0; q <= W; ++q) sa.seg[q] = seg_start[q];
  sa.bpre[0] = 0;
  for (int q = 0; q < W; ++q) {
    const int64_t len = seg_start[q + 1] - seg_start[q];
    maxlen = max(maxlen, len);
    const int64_t lead = (seg_start[q] / E) % kRsvAlign;
    sa.bpre[q + 1] = sa.bpre[q] + (lead + (len + E - 1) / E + kST - 1) / kST;
  }
  for (int q = W + 1; q <= DC_MAX_W; ++q) sa.bpre[q] = sa.bpre[W];
  if (maxlen == 0) return hipSuccess;
  float inv, c;
  reciprocal(W, &inv, &c);
  if (dtype == DC_BF16)
    return pre_div ? rs_v_w<true, true>(W, in, ld_in, out, ld_out, sa, maxlen, inv, c, stream)
                   : rs_v_w<true, false>(W, in, ld_in, out, ld_out, sa, maxlen, inv, c, stream);
  return pre_div ? rs_v_w<false, true>(W, in, ld_in, out, ld_out, sa, maxlen, inv, c, stream)
                 : rs_v_w<false, false>(W, in, ld_in, out, ld_out, sa, maxlen, inv, c, stream);
}

template <bool BF16, bool PRE>
hipError_t rs_ring_w(int32_t W, const void* in, int64_t ld_in, void* out, int64_t ld_out, int64_t L,
                     float inv, float c, hipStream_t stream) {
  constexpr int E = BF16 ? 8 : 4;
  const int64_t Lv = L / E;
  const dim3 grid(blocks_for(Lv, 1), (unsigned)W);
  const int cap = stream_cap(W + 1, 1, kKbRsRing);
  const u32x4* i4 = reinterpret_cast<const u32x4*>(in);
  u32x4* o4 = reinterpret_cast<u32x4*>(out);
  switch (W) {
#define DC_RR_W(w)                                                                                \
  case w:                                                                                         \
    hipLaunchKernelGGL((k_rs_ring<BF16, w, PRE>), grid, dim3(kST),                                \
                       pad_for(k_rs_ring<BF16, w, PRE>, cap), stream, W, i4, ld_in / E,           \
                       o4, ld_out / E, Lv, inv, c);                                               \
    break;
    DC_RR_W(1)
    DC_RR_W(2)
    DC_RR_W(4)
    DC_RR_W(8)
    DC_RR_W(16)
#undef DC_RR_W
    default:
      hipLaunchKernelGGL((k_rs_ring<BF16, 0, PRE>), grid, dim3(kST),
                         pad_for(k_rs_ring<BF16, 0, PRE>, cap), stream, W, i4,
                         ld_in / E, o4, ld_out / E, Lv, inv, c);
  }
  return hipGetLastError();
}

hipError_t launch_reduce_scatter_ring(int32_t W, int32_t dtype, const void* in, int64_t ld_in,
                                      void* out, int64_t ld_out, int64_t M, int32_t pre_div,
                                      hipStream_t stream) {
  const int64_t L = M / W;
  if (L == 0) return hipSuccess;
  float inv, c;
  reciprocal(W, &inv, &c);
  const bool bf = dtype == DC_BF16;
  const int E = bf ? 8 : 4;
  if (L % E == 0) {
    if (bf) return pre_div ? rs_ring_w<true, true>(W, in, ld_in, out, ld_out, L, inv, c, stream)
                           : rs_ring_w<true, false>(W, in, ld_in, out, ld_out, L, inv, c, stream);
    return pre_div ? rs_ring_w<false, true>(W, in, ld_in, out, ld_out, L, inv, c, stream)
                   : rs_ring_w<false, false>(W, in, ld_in, out, ld_out, L, inv, c, stream);
  }
  const dim3 grid(blocks_for(L, 1), (unsigned)W);
  if (bf)
    hipLaunchKernelGGL(k_rs_ring_elem<true>, grid, dim3(kST), 0, stream, W, in, ld_in, out,
                       ld_out, L, pre_div, inv, c);
  else
    hipLaunchKernelGGL(k_rs_ring_elem<false>, grid, dim3(kST), 0, stream, W, in, ld_in, out,
                       ld_out, L, pre_div, inv, c);
  return hipGetLastError();
}

hipError_t launch_all_gather_step(int32_t W, int32_t dtype, const void* in, int64_t ld_in,
                                  void* out, int64_t ld_out, int64_t L, int32_t algo,
                                  int32_t step, hipStream_t stream) {
  if (L == 0) return hipSuccess;
  const int E = dtype == DC_BF16 ? 8 : 4;
  const int32_t tmax = step == 0 ? 1 : algo == 0 ? 1 : algo == 1 ? 2 : 1 << (step - 1);
  const dim3 grid(blocks_for((L + E - 1) / E, 1), (unsigned)W, (unsigned)tmax);
  if (dtype == DC_BF16)
    hipLaunchKernelGGL(k_ag_step<2>, grid, dim3(kST), 0, stream, W,
                       reinterpret_cast<const char*>(in), ld_in, reinterpret_cast<char*>(out), ld_out,
                       L, algo, step);
  else
    hipLaunchKernelGGL(k_ag_step<4>, grid, dim3(kST), 0, stream, W,
                       reinterpret_cast<const char*>(in), ld_in, reinterpret_cast<char*>(out), ld_out,
                       L, algo, step);
  return hipGetLastError();
}

hipError_t launch_all_gather(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                             int64_t ld_out, int64_t L, int32_t order, int32_t step,
                             hipStream_t stream) {
  if (L == 0) return hipSuccess;
  const bool bf = dtype == DC_BF16;
  const int E = bf ? 8 : 4;
  if (L % E == 0) {
    const int64_t Lv = L / E;
    const u32x4* i4 = reinterpret_cast<const u32x4*>(in);
    u32x4* o4 = reinterpret_cast<u32x4*>(out);
    if (order == DC_ORDER_RANK)
      launch_ag_vec<DC_AG_RANK_SHAPE>(W, i4, ld_in / E, o4, ld_out / E, Lv, order, step,
                                      DC_AG_RANK_CAP, stream);
    else
      launch_ag_vec<DC_AG_RING_SHAPE>(W, i4, ld_in / E, o4, ld_out / E, Lv, order, step,
                                      DC_AG_RING_CAP, stream);
  } else if (bf) {
    hipLaunchKernelGGL(k_ag_elem<uint16_t>, dim3(blocks_for(L, DC_AG_U), (unsigned)W), dim3(kST), 0,
                       stream, W, reinterpret_cast<const uint16_t*>(in), ld_in,
                       reinterpret_cast<uint16_t*>(out), ld_out, L, order, step);
  } else {
    hipLaunchKernelGGL(k_ag_elem<uint32_t>, dim3(blocks_for(L, DC_AG_U), (unsigned)W), dim3(kST), 0,
                       stream, W, reinterpret_cast<const uint32_t*>(in), ld_in,
                       reinterpret_cast<uint32_t*>(out), ld_out, L, order, step);
  }
  return hipGetLastError();
}

hipError_t launch_accumulate(int32_t rows, const float* x, int64_t ld_x, float* acc,
                             int64_t ld_acc, int64_t M, int32_t init, hipStream_t stream) {
  if (M == 0 || rows == 0) return hipSuccess;
  const int64_t nvec = M / 4;
  hipLaunchKernelGGL(k_accumulate, dim3(blocks_for(nvec + 1, DC_ACC_U), (unsigned)rows), dim3(kST), 0,
                     stream, x, ld_x, acc, ld_acc, M, init);
  return hipGetLastError();
}

hipError_t launch_deferred_reduce(int32_t W, const float* acc, int64_t ld_acc, float* out,
                                  int64_t ld_out, int64_t M, int32_t out_rows,
                                  hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const dim3 grid(blocks_for(M / 4 + 1, DC_DEF_U));
  const int cap = stream_cap(W + out_rows, DC_DEF_U, kKbDeferred);
  switch (W) {
#define DC_DR_W(w)                                                                            \
  case w:                                                                                     \
    hipLaunchKernelGGL(k_deferred<w>, grid, dim3(kST),                                        \
                       pad_for(k_deferred<w>, cap), stream, W, acc, ld_acc, out,              \
                       ld_out, M, out_rows);                                                  \
    break;
    DC_DR_W(1)
    DC_DR_W(2)
    DC_DR_W(4)
    DC_DR_W(8)
    DC_DR_W(16)
#undef DC_DR_W
    default:
      hipLaunchKernelGGL(k_deferred<0>, grid, dim3(kST),
                         pad_for(k_deferred<0>, cap), stream, W, acc, ld_acc, out,
                         ld_out, M, out_rows);
  }
  return hipGetLastError();
}

hipError_t launch_accumulate_reduce(int32_t W, const float* x, int64_t ld_x, float* acc,
                                    int64_t ld_acc, int32_t init, int32_t keep_acc, float* out,
                                    int64_t ld_out, int32_t out_rows, int64_t M,
                                    hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const dim3 grid(blocks_for(M / 4 + 1, 1));
  const int cap = stream_cap(W + (init ? 0 : W) + (keep_acc ? W : 0) + out_rows, 1, kKbAccRed);
  switch (W) {
#define DC_AR_W(w)                                                                            \
  case w:                                                                                     \
    hipLaunchKernelGGL(k_accum_reduce<w>, grid, dim3(kST),                                    \
                       pad_for(k_accum_reduce<w>, cap), stream, W, x, ld_x, acc,              \
                       ld_acc, init, keep_acc, out, ld_out, out_rows, M);                     \
    break;
    DC_AR_W(1)
    DC_AR_W(2)
    DC_AR_W(4)
    DC_AR_W(8)
    DC_AR_W(16)
#undef DC_AR_W
    default:
      hipLaunchKernelGGL(k_accum_reduce<0>, grid, dim3(kST),
                         pad_for(k_accum_reduce<0>, cap), stream, W, x, ld_x, acc,
                         ld_acc, init, keep_acc, out, ld_out, out_rows, M);
  }
  return hipGetLastError();
}

hipError_t launch_round_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + kST - 1) / kST;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_round_bf16, dim3((unsigned)blocks), dim3(kST), 0, stream, in, out, n);
  return hipGetLastError();
}

hipError_t launch_stream_rows(const void* src, int64_t src_ld_vec, int32_t rows_read, void* dst,
                              int64_t dst_ld_vec, int32_t rows_written, int64_t nvec,
                              hipStream_t stream) {
  if (nvec == 0) return hipSuccess;
  const dim3 grid(blocks_for(nvec, 1));
  const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
  u32x4* d4 = reinterpret_cast<u32x4*>(dst);
#define DC_SR(R, NW)                                                                          \
  if (rows_read == R && rows_written == NW) {                                                 \
    hipLaunchKernelGGL((k_stream_rows<R, NW>), grid, dim3(kST), 0, stream, s4, src_ld_vec, \
                       d4, dst_ld_vec, nvec);                                                 \
    return hipGetLastError();                                                                 \
  }
  DC_SR(4, 1) DC_SR(4, 4) DC_SR(8, 1) DC_SR(8, 8) DC_SR(16, 1) DC_SR(16, 16)
#undef DC_SR
  return hipErrorInvalidValue;
}

hipError_t launch_stream_rows_shaped(const void* src, int64_t src_ld_vec, int32_t rows_read,
                                     void* dst, int64_t dst_ld_vec, int32_t rows_written,
                                     int64_t nvec, int32_t group, int32_t cap, hipStream_t stream) {
  if (nvec == 0) return hipSuccess;
  const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
  u32x4* d4 = reinterpret_cast<u32x4*>(dst);
#define DC_SRG(R, NW, G)                                                                       \
  if (rows_read == R && rows_written == NW && group == G) {                                    \
    auto kern = k_stream_rows_g<R, NW, G>;                                                     \
    hipLaunchKernelGGL(kern, dim3(blocks_for(nvec, G)), dim3(kST), pad_for(kern, cap), stream, \
                       s4, src_ld_vec, d4, dst_ld_vec, nvec);                                  \
    return hipGetLastError();                                                                  \
  }
#define DC_SRG3(R, NW) DC_SRG(R, NW, 1) DC_SRG(R, NW, 2) DC_SRG(R, NW, 4)
  DC_SRG3(4, 1) DC_SRG3(4, 4) DC_SRG3(8, 1) DC_SRG3(8, 8) DC_SRG3(16, 1) DC_SRG3(16, 16)
  DC_SRG3(1, 4) DC_SRG3(1, 8) DC_SRG3(1, 16) DC_SRG3(8, 4)
#undef DC_SRG3
#undef DC_SRG
  return hipErrorInvalidValue;
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  const int64_t nvec = bytes / 16;
  if (nvec == 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy, dim3(blocks_for(nvec, DC_COPY_U)), dim3(kST), 0, stream,
                     reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), nvec);
  return hipGetLastError();
}

}  // namespace dc
