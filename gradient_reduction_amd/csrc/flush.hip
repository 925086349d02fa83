// Bucket flush for gfx950.
//
// DeepSpeed issue "[REQUEST] DeepCompile ZeRO-1: reduce-to-owner instead of
// AllReduce", problem statement and "Describe the solution": every bucket
// task is summed over the ranks of its communicator (optionally pre-divided
// by the communicator size) and the sum goes either to the single rank that
// owns the parameter (reduce-to-owner) or to every rank (AllReduce).
//
// Layout: W rank rows of a slab, each a run of 16-byte column vectors
// (8 bf16 or 4 fp32).  Vectors sit on absolute slab columns, so a task's
// offset never breaks alignment; a vector can still straddle a task or
// bucket boundary, and those vectors take an element-wise path.
//
// Searched flush: a workgroup of one wave (64 threads) owns a tile of 64*U
// consecutive vectors; tiles of about 128 vectors measured 2-4% faster than
// 512 on every flush path (more, smaller tiles spread each bucket more
// evenly).  It finds the tasks overlapping its tile with a block-wide k-ary
// search over the sorted task table, stages them in LDS with their roots
// resolved through the owner map before any row is read (the issue's design
// points resolve a bucket's roots ahead of its reduction), then streams its
// vectors: W 16-byte row loads, an fp32 fold in rank order, one 16-byte
// store to the owner row or W stores (AllReduce).
//
// Planned flush: a plan built once per bucket layout on the host gives every
// tile of 64 vectors its task range and, for a tile inside one task, its
// root.  A one-wave workgroup takes one plan tile; a tile inside one task
// streams with no search and no staging.
//
// This is a streaming reduction with no reuse: no MFMA, HBM bound.

#include "device_common.h"
#include "internal.h"

namespace dc {
namespace {

#ifndef DC_FLUSH_TPB
#define DC_FLUSH_TPB 64   // threads per workgroup (one wave)
#endif
constexpr int kFT = DC_FLUSH_TPB;
constexpr int kStage = kFT;  // tasks staged in LDS per pass over a tile (one per thread)

#ifndef DC_FLUSH_U
#define DC_FLUSH_U 2      // vectors per thread per tile
#endif
#ifndef DC_FLUSH_NT
#define DC_FLUSH_NT 1     // nontemporal row loads (each input is read once)
#endif
#ifndef DC_FLUSH_NTS
#define DC_FLUSH_NTS 1    // nontemporal result stores
#endif


struct FlushParams {
  const void* in;
  void* out;
  int64_t ld_in;   // row strides in elements
  int64_t ld_out;
  int64_t c0;      // bucket columns [c0, c1)
  int64_t c1;
  int64_t v0;      // first vector the bucket touches (absolute)
  int64_t nv;      // vectors the bucket touches
  const dc_task* tasks;
  int32_t ntasks;
  const int32_t* owner;
  const int64_t* flat;   // ZeRO-2: flat offset of each param in its group
  const int64_t* psize;  // ZeRO-2: partition size of each param's group (0: AllReduce)
  int32_t nparams;
  int32_t W;
  int32_t ncomms;
  int32_t pre_div;
  int32_t csize[DC_MAX_COMMS];
  int32_t cstride[DC_MAX_COMMS];
  float cinv[DC_MAX_COMMS];  // 1/c when c is a power of two, else 0
  const dc_tile* tiles;      // planned flush: one record per plan tile, else NULL
  int64_t root_tiles;        // planned: tiles that write one row (host side: the residency cap)
};

// A contribution pre-divided in mode kPreNone, kPreMul (an exact power-of-two
// reciprocal: the same correctly rounded result as dividing) or kPreDiv.
__device__ __forceinline__ float pre_scale(float x, int mode, float inv, float c) {
  if (mode == kPreMul) return x * inv;
  if (mode == kPreDiv) return x / c;
  return x;
}

// Shape of communicator `comm`, selected with compile-time indices: a
// run-time index into the kernel-argument arrays would make the compiler
// copy them to per-lane private memory.
__device__ __forceinline__ void comm_shape(const FlushParams& p, int32_t comm, int32_t& c,
                                           int32_t& s, float& inv) {
  c = p.csize[0];
  s = p.cstride[0];
  inv = p.cinv[0];
#pragma unroll
  for (int k = 1; k < DC_MAX_COMMS; ++k) {
    if (comm == k) {
      c = p.csize[k];
      s = p.cstride[k];
      inv = p.cinv[k];
    }
  }
}

__device__ __forceinline__ int32_t member(int32_t b, int32_t i, int32_t c, int32_t s) {
  return (s == 1 ? b * c : b) + i * s;
}

// ---------------------------------------------------------------------------
// Vector paths: every column of the 16-byte vector belongs to one task.
// ---------------------------------------------------------------------------

// Fold one row's vector into acc (8 bf16 or 4 fp32 columns).
template <bool BF16, int PRE>
__device__ __forceinline__ void fold_vec(float* acc, u32x4 x, bool first, float inv, float c) {
  if constexpr (BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float a = bf16_lo(x[q]);
      float b = bf16_hi(x[q]);
      if constexpr (PRE != kPreNone) {
        a = pre_scale(a, PRE, inv, c);
        b = pre_scale(b, PRE, inv, c);
        bf16_round_pair(a, b);
      }
      acc[2 * q] = first ? a : acc[2 * q] + a;
      acc[2 * q + 1] = first ? b : acc[2 * q + 1] + b;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float a = __uint_as_float(x[q]);
      if constexpr (PRE != kPreNone) a = pre_scale(a, PRE, inv, c);
      acc[q] = first ? a : acc[q] + a;
    }
  }
}

template <bool BF16>
__device__ __forceinline__ u32x4 pack_vec(const float* acc) {
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

// W known at compile time: the W row vectors of column vector `av`.
template <bool BF16, int WT, bool NT>
__device__ __forceinline__ void load_rows(const FlushParams& p, int64_t av, u32x4 (&x)[WT]) {
  constexpr int E = BF16 ? 8 : 4;
  const u32x4* in = reinterpret_cast<const u32x4*>(p.in) + av;
  const int64_t ldi = p.ld_in / E;
#pragma unroll
  for (int r = 0; r < WT; ++r) x[r] = load16<NT>(in + r * ldi);
}

// Fold the blocks of a communicator of C members with stride S (C = WT:
// the data-parallel comm, one block) from the loaded rows, members in
// order, then store: the owner row when there is one, else every member.
// The pre-division reciprocal 1/C is a compile-time power of two.
template <bool BF16, int WT, int C, int S, int PRE>
__device__ __forceinline__ void fold_store(const FlushParams& p, const u32x4 (&x)[WT], int64_t av,
                                           int32_t root) {
  constexpr int E = BF16 ? 8 : 4;
  constexpr float inv = 1.0f / (float)C;
  u32x4* out = reinterpret_cast<u32x4*>(p.out) + av;
  const int64_t ldo = p.ld_out / E;
#pragma unroll
  for (int b = 0; b < WT / C; ++b) {
    constexpr int step = S;
    const int base = S == 1 ? b * C : b;
    float acc[E];
#pragma unroll
    for (int i = 0; i < C; ++i) fold_vec<BF16, PRE>(acc, x[base + i * step], i == 0, inv, (float)C);
    const u32x4 y = pack_vec<BF16>(acc);
    if (C == WT && root >= 0) {
      store16<DC_FLUSH_NTS>(out + root * ldo, y);
    } else {
#pragma unroll
      for (int i = 0; i < C; ++i) store16<DC_FLUSH_NTS>(out + (base + i * step) * ldo, y);
    }
  }
}

// The fast kernel's two communicator shapes: the data-parallel comm (size
// WT) or the one sub-communicator shape (C2, S2) the launch was made for.
template <bool BF16, int WT, int C2, int S2, int PRE>
__device__ __forceinline__ void fold_store_shape(const FlushParams& p, const u32x4 (&x)[WT],
                                                 int64_t av, int32_t root, int32_t c) {
  if constexpr (C2 > 0) {
    if (c != WT) {
      fold_store<BF16, WT, C2, S2, PRE>(p, x, av, -1);
      return;
    }
  }
  fold_store<BF16, WT, WT, 1, PRE>(p, x, av, root);
}

// Any W and communicator, sizes known at run time: per block, load-and-fold
// its members in order, then write the block (or the owner row).
template <bool BF16, bool NT>
__device__ __forceinline__ void vec_generic(const FlushParams& p, int64_t av, int32_t root,
                                            int32_t c, int32_t s, float inv) {
  constexpr int E = BF16 ? 8 : 4;
  const u32x4* in = reinterpret_cast<const u32x4*>(p.in);
  u32x4* out = reinterpret_cast<u32x4*>(p.out);
  const int64_t ldi = p.ld_in / E, ldo = p.ld_out / E;
  const int mode = !p.pre_div ? kPreNone : (inv != 0.0f ? kPreMul : kPreDiv);
  const float cf = (float)c;
  for (int32_t b = 0; b < p.W / c; ++b) {
    float acc[E];
    for (int32_t i = 0; i < c; ++i) {
      const u32x4 x = load16<NT>(in + (int64_t)member(b, i, c, s) * ldi + av);
      if (mode == kPreNone) fold_vec<BF16, kPreNone>(acc, x, i == 0, inv, cf);
      else if (mode == kPreMul) fold_vec<BF16, kPreMul>(acc, x, i == 0, inv, cf);
      else fold_vec<BF16, kPreDiv>(acc, x, i == 0, inv, cf);
    }
    const u32x4 y = pack_vec<BF16>(acc);
    if (root >= 0) {
      store16<false>(out + (int64_t)root * ldo + av, y);
    } else {
      for (int32_t i = 0; i < c; ++i) store16<false>(out + (int64_t)member(b, i, c, s) * ldo + av, y);
    }
  }
}

// ---------------------------------------------------------------------------
// Element path: a column of a vector that straddles a task or bucket edge.
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ void elem_flush(const FlushParams& p, int64_t col, int32_t root,
                                           int32_t c, int32_t s, float inv) {
  const int mode = !p.pre_div ? kPreNone : (inv != 0.0f ? kPreMul : kPreDiv);
  const float cf = (float)c;
  for (int32_t b = 0; b < p.W / c; ++b) {
    float acc = 0.0f;
    for (int32_t i = 0; i < c; ++i) {
      const int64_t r = member(b, i, c, s);
      float v;
      if constexpr (BF16) {
        v = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p.in)[r * p.ld_in + col] << 16);
        if (mode != kPreNone) {
          v = pre_scale(v, mode, inv, cf);
          v = bf16_lo(bf16_pack_rne(v, 0.0f));
        }
      } else {
        v = reinterpret_cast<const float*>(p.in)[r * p.ld_in + col];
        v = pre_scale(v, mode, inv, cf);
      }
      acc = i == 0 ? v : acc + v;
    }
    if constexpr (BF16) {
      const uint16_t y = bf16_out(acc);
      uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
      if (root >= 0) out[(int64_t)root * p.ld_out + col] = y;
      else for (int32_t i = 0; i < c; ++i) out[(int64_t)member(b, i, c, s) * p.ld_out + col] = y;
    } else {
      float* out = reinterpret_cast<float*>(p.out);
      if (root >= 0) out[(int64_t)root * p.ld_out + col] = acc;
      else for (int32_t i = 0; i < c; ++i) out[(int64_t)member(b, i, c, s) * p.ld_out + col] = acc;
    }
  }
}


// The vectors [t0, t1) of the bucket's grid (relative to v0, at most kFT*U
// of them, thread i taking t0 + i + u*kFT) whose tasks are first..last of the
// task table: staged in LDS in chunks of kStage, roots resolved; vectors
// inside one task stream, vectors cut by an edge go element by element.
// Every thread of the workgroup must call it (it synchronizes).
template <bool BF16, int WT, int C2, int S2, int PRE, int U, bool NT, bool Z2>
__device__ void flush_staged(const FlushParams& p, int64_t t0, int64_t t1, int32_t first,
                             int32_t last) {
  static_assert(U <= 32, "slow-vector mask is 32 bits");
  constexpr int E = BF16 ? 8 : 4;
  __shared__ int64_t s_off[kStage];
  __shared__ int64_t s_end[kStage];
  __shared__ int32_t s_root[kStage];
  __shared__ int32_t s_csz[kStage];
  __shared__ int32_t s_cst[kStage];
  __shared__ float s_cinv[kStage];
  // ZeRO-2: flat offset of the task's first element and its partition size
  __shared__ int64_t s_za[Z2 ? kStage : 1];
  __shared__ int64_t s_zs[Z2 ? kStage : 1];

  // the range's columns, relative to the bucket
  const int64_t lo = max((p.v0 + t0) * E, p.c0) - p.c0;
  const int64_t hi = min((p.v0 + t1) * E, p.c1) - p.c0;

  for (int32_t base = first; base <= last; base += kStage) {
    const int32_t cnt = min(kStage, last - base + 1);
    __syncthreads();
    if ((int32_t)threadIdx.x < cnt) {
      const dc_task t = p.tasks[base + threadIdx.x];
      int32_t comm = (t.comm >= 0 && t.comm < p.ncomms) ? t.comm : 0;
      int32_t root = -1;
      if (comm == 0 && p.owner != nullptr && t.param >= 0 && t.param < p.nparams) {
        root = p.owner[t.param];
        if (root >= p.W) root = -1;
      }
      s_off[threadIdx.x] = t.offset;
      s_end[threadIdx.x] = t.offset + (t.numel > 0 ? t.numel : 0);
      s_root[threadIdx.x] = root < 0 ? -1 : root;
      int32_t c, st;
      float inv;
      comm_shape(p, comm, c, st, inv);
      s_csz[threadIdx.x] = c;
      s_cst[threadIdx.x] = st;
      s_cinv[threadIdx.x] = inv;
      if constexpr (Z2) {
        int64_t a = 0, S = 0;
        if (comm == 0 && t.param >= 0 && t.param < p.nparams) {
          S = p.psize[t.param];
          a = p.flat[t.param];
        }
        s_za[threadIdx.x] = a;
        s_zs[threadIdx.x] = S > 0 ? S : 0;
      }
    }
    __syncthreads();
    const int64_t clo = max(lo, s_off[0]);
    const int64_t chi = min(hi, s_end[cnt - 1]);
    if (clo >= chi) continue;

    // phase 1: vectors inside one task; phase 2: vectors cut by an edge.
    uint32_t slow = 0;
#pragma unroll 1
    for (int u = 0; u < U; ++u) {
      const int64_t tv = t0 + threadIdx.x + (int64_t)u * kFT;
      if (tv >= t1) break;
      const int64_t av = p.v0 + tv;
      const int64_t rc = av * E - p.c0;  // the vector's first column, relative
      const int64_t e_lo = max(rc, clo), e_hi = min(rc + E, chi);
      if (e_lo >= e_hi) continue;
      const int32_t k = last_le(s_off, cnt, e_lo);
      bool whole = e_lo == rc && e_hi == rc + E && s_off[k] <= rc && s_end[k] >= rc + E;
      int32_t vroot = s_root[k];
      if constexpr (Z2) {
        // every element goes to the rank of its partition; a vector cut by
        // a partition boundary takes the element path
        if (whole && s_zs[k] > 0) {
          const int64_t pos = s_za[k] + (rc - s_off[k]);
          const int64_t q0 = pos / s_zs[k], q1 = (pos + E - 1) / s_zs[k];
          if (q0 == q1 && q0 < (WT > 0 ? WT : p.W)) vroot = (int32_t)q0;
          else whole = false;
        }
      }
      if (whole) {
        if constexpr (WT > 0) {
          u32x4 x[WT];
          load_rows<BF16, WT, NT>(p, av, x);
          fold_store_shape<BF16, WT, C2, S2, PRE>(p, x, av, vroot, s_csz[k]);
        } else {
          vec_generic<BF16, NT>(p, av, vroot, s_csz[k], s_cst[k], s_cinv[k]);
        }
      } else {
        slow |= 1u << u;
      }
    }
#pragma unroll 1
    for (int u = 0; u < U; ++u) {
      if (!((slow >> u) & 1u)) continue;
      const int64_t av = p.v0 + t0 + threadIdx.x + (int64_t)u * kFT;
      const int64_t rc = av * E - p.c0;
      const int64_t e_lo = max(rc, clo), e_hi = min(rc + E, chi);
      for (int64_t x = e_lo; x < e_hi; ++x) {
        const int32_t kk = last_le(s_off, cnt, x);
        if (s_off[kk] <= x && x < s_end[kk]) {
          int32_t eroot = s_root[kk];
          if constexpr (Z2) {
            if (s_zs[kk] > 0) {
              const int64_t q = (s_za[kk] + (x - s_off[kk])) / s_zs[kk];
              eroot = q < p.W ? (int32_t)q : -1;
            }
          }
          elem_flush<BF16>(p, p.c0 + x, eroot, s_csz[kk], s_cst[kk], s_cinv[kk]);
        }
      }
    }
  }
}

// The task range of vectors [t0, t1) by a block-wide k-ary search of the
// sorted task table: the task holding the first column through the last
// task starting before the range's end.  Every thread must call it.
template <int E>
__device__ __forceinline__ void search_range(const FlushParams& p, int64_t t0, int64_t t1,
                                             int32_t& first, int32_t& last) {
  const int64_t lo = max((p.v0 + t0) * E, p.c0) - p.c0;
  const int64_t hi = min((p.v0 + t1) * E, p.c1) - p.c0;
  kary_bounds<kFT>(p.ntasks, [&](int32_t i) { return p.tasks[i].offset; }, lo, hi, first, last);
  first = max(first - 1, 0);  // the task holding column lo
  last = last - 1;            // the last task starting before hi
}

// Searched flush.  WT > 0: W known at compile time, every communicator of
// the launch is the data-parallel one or the single shape (C2, S2) (C2 = 0:
// none).  WT = 0: any W and any communicators, all at run time.
template <bool BF16, int WT, int C2, int S2, int PRE, int U, bool NT, bool Z2>
__global__ __launch_bounds__(kFT) void k_flush(FlushParams p) {
  constexpr int E = BF16 ? 8 : 4;
  const int64_t t0 = (int64_t)blockIdx.x * (kFT * U);
  const int64_t t1 = min(t0 + (int64_t)(kFT * U), p.nv);
  int32_t first, last;
  search_range<E>(p, t0, t1, first, last);
  flush_staged<BF16, WT, C2, S2, PRE, U, NT, Z2>(p, t0, t1, first, last);
}

// Planned flush: workgroup b takes plan tile b, kPlanTile vectors (thread i:
// vector i).  With PF, a full tile issues its W row loads together with the
// load of its plan record (the row addresses do not depend on the plan), so
// the record arrives under the rows' latency.  A tile the record marks
// whole (inside one task and the bucket) folds and stores straight away, to
// its root row or to every member; any other tile takes the staged path over
// the record's task range.
template <bool BF16, int WT, int C2, int S2, int PRE, bool NT, bool Z2, bool PF>
__global__ __launch_bounds__(kFT) void k_flush_planned(FlushParams p) {
  constexpr int E = BF16 ? 8 : 4;
  const int64_t tile = blockIdx.x;
  const int64_t t0 = tile * kPlanTile, t1 = min(t0 + kPlanTile, p.nv);
  const int64_t slot = tile_slot(tile, (int64_t)gridDim.x);
  if constexpr (WT > 0) {
    if (t1 - t0 == kPlanTile) {
      const int64_t av = p.v0 + t0 + threadIdx.x;
      u32x4 x[WT];
      if constexpr (PF) load_rows<BF16, WT, NT>(p, av, x);
      const dc_tile rec = p.tiles[slot];
      if (rec.flags & 1) {
        int32_t comm = (rec.flags >> 8) & 0xFF;
        comm = comm < p.ncomms ? comm : 0;
        const int32_t root = (comm == 0 && rec.root >= 0 && rec.root < p.W) ? rec.root : -1;
        int32_t fc, fs;
        float finv;
        comm_shape(p, comm, fc, fs, finv);
        if constexpr (!PF) load_rows<BF16, WT, NT>(p, av, x);
        if (C2 == 0 || fc == WT) {
          constexpr float inv = 1.0f / (float)WT;
          float acc[E];
#pragma unroll
          for (int i = 0; i < WT; ++i) fold_vec<BF16, PRE>(acc, x[i], i == 0, inv, (float)WT);
          const u32x4 y = pack_vec<BF16>(acc);
          u32x4* out = reinterpret_cast<u32x4*>(p.out) + (p.v0 + t0);
          const int64_t ldo = p.ld_out / E;
          constexpr int32_t bytes = kPlanTile * 16;
          if (root >= 0) {
            store_buf<kStoreOneRow>(out + root * ldo, bytes, threadIdx.x * 16, y);
          } else {
#pragma unroll
            for (int r = 0; r < WT; ++r) store_buf<kStoreAllRows>(out + r * ldo, bytes, threadIdx.x * 16, y);
          }
        } else {
          // the launch's one sub-communicator shape: block by block
          fold_store_shape<BF16, WT, C2, S2, PRE>(p, x, av, root, fc);
        }
        return;
      }
      if constexpr (PF) {
        // the rows are used on this path too, so the compiler keeps their
        // loads ahead of the record test (here it only waits for them)
#pragma unroll
        for (int i = 0; i < WT; ++i) asm volatile("" ::"v"(x[i]));
      }
    }
  }
  const dc_tile rec = p.tiles[slot];
  if (WT == 0 && (rec.flags & 1) && t1 - t0 == kPlanTile) {
    int32_t comm = (rec.flags >> 8) & 0xFF;
    comm = comm < p.ncomms ? comm : 0;
    const int32_t root = (comm == 0 && rec.root >= 0 && rec.root < p.W) ? rec.root : -1;
    int32_t fc, fs;
    float finv;
    comm_shape(p, comm, fc, fs, finv);
    vec_generic<BF16, NT>(p, p.v0 + t0 + threadIdx.x, root, fc, fs, finv);
    return;
  }
  const int32_t first = max(rec.first, 0), last = min(rec.last, p.ntasks - 1);
  flush_staged<BF16, WT, C2, S2, PRE, 1, NT, Z2>(p, t0, t1, first, last);
}

// Planned launch shapes (one-wave workgroups, one plan tile each, LDS
// reserved to cap residency), from interleaved sweeps on the 402.8M-element
// W = 8 bf16 and the 1.2B-element W = 16 fp32 flushes: W = 8 buckets whose
// tiles mostly write one row ran fastest at 8 workgroups per compute unit
// (6.40 TB/s, against 6.35 at 10, 6.24 at 7 and 5.88 at 6), buckets whose
// tiles write every row at 6 (6.48-6.55, against 6.34-6.36 at 4, 5 and 7);
// W = 16 at 6 and 3.  W = 4 keeps
// the caps measured there with two-vector tiles.  Other W take the caps of
// the nearest measured W below them.  A searched launch keeps full
// occupancy: its per-tile search needs the other resident workgroups to
// hide it.
#ifndef DC_PLAN_CAP_W8
#define DC_PLAN_CAP_W8 8, 6     // W = 8: one-row buckets, every-row buckets
#endif
#ifndef DC_PLAN_CAP_W16
#define DC_PLAN_CAP_W16 6, 3
#endif
#ifndef DC_PLAN_CAP_W4
#define DC_PLAN_CAP_W4 12, 8
#endif
// Whether a planned workgroup loads its tile's rows together with its plan
// record (before it knows the tile's root): faster at W = 8 (6.49 against
// 6.27 TB/s on the 402.8M-element flush), much slower at W = 16 fp32 (4.8
// against 6.0 TB/s per bucket).
#ifndef DC_PLAN_PF_W8
#define DC_PLAN_PF_W8 1
#endif
#ifndef DC_PLAN_PF_W16
#define DC_PLAN_PF_W16 0
#endif
#ifndef DC_PLAN_PF_W4
#define DC_PLAN_PF_W4 1
#endif
constexpr bool plan_prefetch(int WT) {
  return WT == 8 ? DC_PLAN_PF_W8 != 0 : WT == 16 ? DC_PLAN_PF_W16 != 0 : WT == 4 ? DC_PLAN_PF_W4 != 0 : false;
}

int cap_pick(int one, int all, bool one_row) { return one_row ? one : all; }

int plan_cap(int32_t W, bool one_row) {
  if (W >= 16) return cap_pick(DC_PLAN_CAP_W16, one_row);
  if (W >= 8) return cap_pick(DC_PLAN_CAP_W8, one_row);
  if (W >= 4) return cap_pick(DC_PLAN_CAP_W4, one_row);
  return 0;
}

// Dynamic LDS a launch of one kernel reserves, unused, so that at most `cap`
// of its workgroups fit in one compute unit's LDS.
template <typename K>
size_t kernel_pad(K* kern, int cap) {
  return occupancy_pad(reinterpret_cast<const void*>(kern), cap);
}

template <bool BF16, int WT, int C2, int S2, int PRE, bool Z2>
hipError_t launch_planned(const FlushParams& p, hipStream_t stream) {
  const FlushTiles g = plan_tiles(BF16 ? DC_BF16 : DC_F32, p.c0, p.c1);
  if (g.count == 0) return hipSuccess;
  FlushParams q = p;
  q.v0 = g.v0;
  q.nv = g.nv;
  const int cap = plan_cap(p.W, 2 * p.root_tiles >= g.count);
  auto kern = k_flush_planned<BF16, WT, C2, S2, PRE, DC_FLUSH_NT != 0, Z2, plan_prefetch(WT)>;
  hipLaunchKernelGGL(kern, dim3((unsigned)g.count), dim3(kFT), kernel_pad(kern, cap), stream, q);
  return hipGetLastError();
}

template <bool BF16, int WT, int C2, int S2, int PRE>
hipError_t launch_kernel(const FlushParams& p, hipStream_t stream) {
  if (p.tiles != nullptr) {
    return p.flat != nullptr ? launch_planned<BF16, WT, C2, S2, PRE, true>(p, stream)
                             : launch_planned<BF16, WT, C2, S2, PRE, false>(p, stream);
  }
  constexpr int U = DC_FLUSH_U;
  // Tiles sit on absolute multiples of the tile size, not at the bucket's
  // first vector: a bucket that starts inside a cache line would otherwise
  // have every wave's 1 KB straddle lines, sharing partial lines between
  // neighbouring tiles (measured 15% slower on such buckets).  Vectors in
  // front of the bucket fall outside its columns and are skipped.
  const FlushTiles g = flush_tiles(BF16 ? DC_BF16 : DC_F32, p.c0, p.c1);
  if (g.count == 0) return hipSuccess;
  FlushParams q = p;
  q.v0 = g.v0;
  q.nv = g.nv;
  if (q.flat != nullptr) {
    hipLaunchKernelGGL((k_flush<BF16, WT, C2, S2, PRE, U, DC_FLUSH_NT != 0, true>),
                       dim3((unsigned)g.count), dim3(kFT), 0, stream, q);
  } else {
    hipLaunchKernelGGL((k_flush<BF16, WT, C2, S2, PRE, U, DC_FLUSH_NT != 0, false>),
                       dim3((unsigned)g.count), dim3(kFT), 0, stream, q);
  }
  return hipGetLastError();
}

template <bool BF16, int WT, int C2, int S2>
hipError_t launch_pre(const FlushParams& p, hipStream_t stream) {
  return p.pre_div ? launch_kernel<BF16, WT, C2, S2, kPreMul>(p, stream)
                   : launch_kernel<BF16, WT, C2, S2, kPreNone>(p, stream);
}

// The one sub-communicator shape of a comm table, canonicalised (size 1 has
// stride 1); 0 when there is none, -1 when there are several.
int sub_shape(const FlushParams& p, int32_t* c2, int32_t* s2) {
  *c2 = 0;
  *s2 = 1;
  for (int k = 1; k < p.ncomms; ++k) {
    const int32_t c = p.csize[k], s = c == 1 ? 1 : p.cstride[k];
    if (c == p.W) continue;
    if (*c2 == 0) {
      *c2 = c;
      *s2 = s;
    } else if (*c2 != c || *s2 != s) {
      return -1;
    }
  }
  return *c2 ? 1 : 0;
}

template <bool BF16, int WT>
hipError_t launch_w(const FlushParams& p, int32_t c2, int32_t s2, hipStream_t stream) {
  // every (C2, S2) a power-of-two W allows: C2 = WT/2, WT/4, ... with stride
  // 1 (contiguous blocks) or WT/C2 (strided); size 1 has one shape
  if (c2 == 0) return launch_pre<BF16, WT, 0, 1>(p, stream);
#define DC_SUB(C)                                                                   \
  if constexpr (WT > C && WT % C == 0) {                                            \
    if (c2 == C) return s2 == 1 ? launch_pre<BF16, WT, C, 1>(p, stream)             \
                                : launch_pre<BF16, WT, C, (C > 0 ? WT / C : 1)>(p, stream); \
  }
  DC_SUB(1)
  DC_SUB(2)
  DC_SUB(4)
  DC_SUB(8)
#undef DC_SUB
  return launch_kernel<BF16, 0, 0, 1, kPreNone>(p, stream);
}

template <bool BF16>
hipError_t launch_dtype(const FlushParams& p, hipStream_t stream) {
  int32_t c2, s2;
  if (sub_shape(p, &c2, &s2) >= 0) {
    switch (p.W) {
      case 1: return launch_w<BF16, 1>(p, c2, s2, stream);
      case 2: return launch_w<BF16, 2>(p, c2, s2, stream);
      case 4: return launch_w<BF16, 4>(p, c2, s2, stream);
      case 8: return launch_w<BF16, 8>(p, c2, s2, stream);
      case 16: return launch_w<BF16, 16>(p, c2, s2, stream);
      default: break;
    }
  }
  return launch_kernel<BF16, 0, 0, 1, kPreNone>(p, stream);
}

}  // namespace

hipError_t launch_flush(const FlushLaunch& a, hipStream_t stream) {
  FlushParams p;
  const int E = a.dtype == DC_BF16 ? 8 : 4;
  p.in = a.in;
  p.out = a.out;
  p.ld_in = a.ld_in;
  p.ld_out = a.ld_out;
  p.c0 = a.c0;
  p.c1 = a.c1;
  p.v0 = a.c0 / E;
  p.nv = a.c1 > a.c0 ? (a.c1 + E - 1) / E - p.v0 : 0;
  p.tasks = a.tasks;
  p.ntasks = a.ntasks;
  p.owner = a.owner;
  p.flat = a.flat;
  p.psize = a.psize;
  p.nparams = a.nparams;
  p.W = a.W;
  p.ncomms = a.ncomms;
  p.pre_div = a.pre_div;
  for (int k = 0; k < DC_MAX_COMMS; ++k) {
    const int32_t c = k < a.ncomms ? a.comms[k].size : 1;
    p.csize[k] = c;
    p.cstride[k] = k < a.ncomms ? a.comms[k].stride : 1;
    p.cinv[k] = (c & (c - 1)) == 0 ? 1.0f / (float)c : 0.0f;  // exact for powers of two
  }
  p.tiles = a.tiles;
  p.root_tiles = a.root_tiles;
  if (p.nv == 0 || a.ntasks == 0) return hipSuccess;
  return a.dtype == DC_BF16 ? launch_dtype<true>(p, stream) : launch_dtype<false>(p, stream);
}

namespace {
FlushTiles tiles_of(int32_t dtype, int64_t c0, int64_t c1, int64_t tile) {
  const int64_t E = dtype == DC_BF16 ? 8 : 4;
  FlushTiles g;
  g.tile = tile;
  const int64_t first = c0 / E;
  const int64_t shift = first % g.tile;
  g.v0 = first - shift;
  g.nv = c1 > c0 ? (c1 + E - 1) / E - first + shift : 0;
  g.count = (g.nv + g.tile - 1) / g.tile;
  return g;
}
}  // namespace

FlushTiles flush_tiles(int32_t dtype, int64_t c0, int64_t c1) {
  return tiles_of(dtype, c0, c1, (int64_t)kFT * DC_FLUSH_U);
}

FlushTiles plan_tiles(int32_t dtype, int64_t c0, int64_t c1) {
  static_assert(kPlanTile == kFT, "a plan tile is one vector per thread of a workgroup");
  return tiles_of(dtype, c0, c1, kPlanTile);
}


}  // namespace dc
