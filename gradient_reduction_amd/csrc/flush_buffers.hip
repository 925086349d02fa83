// Bucket flush with copy-in and copy-out fused in (DeepSpeed issue
// "[REQUEST] DeepCompile ZeRO-1: reduce-to-owner instead of AllReduce",
// problem statement: gradients reach the bucket from each rank, and after the
// reduction a copy-out loop moves the result into the rank's gradient buffer,
// skipping every rank whose buffer is empty).  Here each rank's gradient is
// read from its own buffer and the sum goes straight into the grad buffers
// that exist, through per-task pointer tables: no bucket staging in HBM, and
// nothing written for a rank that keeps no buffer.
//
// Task offsets are a coordinate system only: vector slot v covers columns
// [v*E, v*E + E) of it (E elements per 16 bytes).  A slot that lies inside
// one task whose offset is a multiple of E and whose pointers are all 16-byte
// aligned moves as 16-byte vectors; any other slot goes element by element.
// HBM bound: W*n*b read + (buffers kept)*n*b written per task of n elements.
#include "device_common.h"
#include "internal.h"

namespace dc {
namespace {

#ifndef DC_BUF_TPB
#define DC_BUF_TPB 64               // threads per workgroup (one wave)
#endif
constexpr int kBT = DC_BUF_TPB;
// Vector slots per thread of a tile: planned launches take the plan's tiles;
// a searched launch takes two per thread (1-7% faster than one or four,
// where each tile searches and stages its tasks).
constexpr int kBufU = (int)(kBufTile / kBT);
#ifndef DC_BUF_US
#define DC_BUF_US 2
#endif
constexpr int kBufUSearched = DC_BUF_US;
static_assert(kBufU * kBT == kBufTile, "a tile is whole slots per thread");
#ifndef DC_BUF_PTRS
#define DC_BUF_PTRS 256             // staged pointers per table (LDS): small enough
                                    // that one-wave workgroups are not LDS bound
#endif
constexpr int kPtrStage = DC_BUF_PTRS;
// Result stores of whole planned tiles at W <= 8 and at W = 16: nontemporal
// global stores (-1), or buffer stores over the tile's run with these
// cache-policy bits.  Interleaved A/B: sc0 sc1 nt and nt sc1 +0.9% at W = 8
// bf16 (6.33 against 6.27 TB/s); at W = 16 fp32 1.2% slower in the faster of
// the runs' two placement modes, equal in the other.
#ifndef DC_BUF_SP8
#define DC_BUF_SP8 19
#endif
#ifndef DC_BUF_SP16
#define DC_BUF_SP16 -1
#endif

struct BufParams {
  const dc_task* tasks;
  const void* const* in_ptrs;
  void* const* out_ptrs;
  int64_t nslots;
  int64_t bucket_numel;
  int32_t ntasks;
  int32_t W;
  int32_t num_comms;
  int32_t csize[DC_MAX_COMMS];
  int32_t cstride[DC_MAX_COMMS];
  const dc_tile* tiles;  // planned: one record per tile (XCD-major), else NULL
};

__device__ __forceinline__ int32_t member_of(int32_t b, int32_t i, int32_t c, int32_t s) {
  return (s == 1 ? b * c : b) + i * s;
}

__device__ __forceinline__ void comm_recip(int32_t c, float* inv, float* cf) {
  *cf = (float)c;
  *inv = (c & (c - 1)) == 0 ? 1.0f / (float)c : 0.0f;  // exact for powers of two
}

// U: vector slots per thread of the launch's tiles (kBufU when planned).
template <bool BF16, int WT, bool PRE, int U>
__global__ __launch_bounds__(kBT) void k_flush_buffers(BufParams p) {
  constexpr int E = BF16 ? 8 : 4;
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int WS = WT > 0 ? WT : DC_MAX_W;                    // pointer stride per task
  constexpr int S = kPtrStage / WS < 256 ? kPtrStage / WS : 256;  // staged tasks per round
  __shared__ const char* s_in[S * WS];
  __shared__ char* s_out[S * WS];
  __shared__ int64_t s_off[S];
  __shared__ int64_t s_end[S];
  __shared__ int32_t s_comm[S];
  __shared__ int32_t s_vec[S];
  __shared__ int32_t s_cs[DC_MAX_COMMS];
  __shared__ int32_t s_cst[DC_MAX_COMMS];
  const int32_t W = WT > 0 ? WT : p.W;
#pragma unroll
  for (int q = 0; q < DC_MAX_COMMS; ++q) {
    if ((int)threadIdx.x == q) {
      s_cs[q] = p.csize[q];
      s_cst[q] = p.cstride[q];
    }
  }
  const int64_t t0 = (int64_t)blockIdx.x * (kBT * U);
  const int64_t t1 = min(t0 + (int64_t)(kBT * U), p.nslots);
  const int64_t lo = t0 * E, hi = min(t1 * E, p.bucket_numel);
  int32_t first, last;
  if (p.tiles != nullptr) {
    // planned: the record names the tile's tasks.  A tile whose slots all lie
    // in one vector-aligned data-parallel task with 16-byte aligned pointers
    // streams straight from the task's pointer row; the kernel checks that
    // itself, so a stale record can only send the tile down the staged path.
    const dc_tile rec = p.tiles[tile_slot((int64_t)blockIdx.x, (int64_t)gridDim.x)];
    first = min(max(rec.first, 0), p.ntasks - 1);
    last = min(rec.last, p.ntasks - 1);
    if constexpr (WT > 0) {
      if (rec.flags & 1) {
        const dc_task t = p.tasks[first];
        bool fast = t.comm == 0 && t.offset % E == 0 && t.offset <= lo && t1 * E <= t.offset + t.numel;
        const char* in[WT];
        char* out[WT];
        uintptr_t bits = 0;
#pragma unroll
        for (int r = 0; r < WT; ++r) {
          in[r] = reinterpret_cast<const char*>(p.in_ptrs[(int64_t)first * WT + r]);
          out[r] = reinterpret_cast<char*>(p.out_ptrs[(int64_t)first * WT + r]);
          bits |= reinterpret_cast<uintptr_t>(in[r]) | reinterpret_cast<uintptr_t>(out[r]);
        }
        if (fast && (bits & 15) == 0) {
          float inv, cf;
          comm_recip(WT, &inv, &cf);
#pragma unroll 1
          for (int u = 0; u < U; ++u) {
            const int64_t v = t0 + threadIdx.x + (int64_t)u * kBT;
            if (v >= t1) break;
            const int64_t byte = (v * E - t.offset) * EB;
            u32x4 x[WT];
#pragma unroll
            for (int r = 0; r < WT; ++r) x[r] = load16<true>(reinterpret_cast<const u32x4*>(in[r] + byte));
            float acc[E];
#pragma unroll
            for (int r = 0; r < WT; ++r) fold16<BF16, PRE>(acc, x[r], r == 0, inv, cf);
            const u32x4 y = pack16<BF16>(acc);
            constexpr int SP = WT <= 8 ? DC_BUF_SP8 : DC_BUF_SP16;
            if constexpr (SP >= 0) {
              // the tile's run of each output buffer, from the tile's first slot
              const int64_t tb = (t0 * E - t.offset) * EB;
              const int32_t rb = (int32_t)((t1 - t0) * 16), off = (int32_t)(byte - tb);
#pragma unroll
              for (int r = 0; r < WT; ++r)
                if (out[r] != nullptr)
                  store_buf<(SP >= 0 ? SP : 0)>(reinterpret_cast<u32x4*>(out[r] + tb), rb, off, y);
            } else {
#pragma unroll
              for (int r = 0; r < WT; ++r)
                if (out[r] != nullptr) store16<true>(reinterpret_cast<u32x4*>(out[r] + byte), y);
            }
          }
          return;
        }
      }
    }
  } else {
    kary_bounds<kBT>(p.ntasks, [&](int32_t i) { return p.tasks[i].offset; }, lo, hi, first, last);
    first = max(first - 1, 0);
    last = last - 1;
  }
  for (int32_t base = first; base <= last; base += S) {
    const int32_t cnt = min(S, last - base + 1);
    __syncthreads();
    for (int32_t x = threadIdx.x; x < cnt; x += kBT) {
      const dc_task t = p.tasks[base + x];
      s_off[x] = t.offset;
      s_end[x] = t.offset + (t.numel > 0 ? t.numel : 0);
      s_comm[x] = (t.comm >= 0 && t.comm < p.num_comms) ? t.comm : 0;
    }
    for (int32_t x = threadIdx.x; x < cnt * W; x += kBT) {
      const int32_t k = x / W, r = x - k * W;
      const int64_t g = (int64_t)(base + k) * W + r;
      s_in[k * WS + r] = reinterpret_cast<const char*>(p.in_ptrs[g]);
      s_out[k * WS + r] = reinterpret_cast<char*>(p.out_ptrs[g]);
    }
    __syncthreads();
    for (int32_t x = threadIdx.x; x < cnt; x += kBT) s_vec[x] = s_off[x] % E == 0;
    __syncthreads();
    for (int32_t x = threadIdx.x; x < cnt * W; x += kBT) {
      const int32_t k = x / W, r = x - k * W;
      if (((reinterpret_cast<uintptr_t>(s_in[k * WS + r]) | reinterpret_cast<uintptr_t>(s_out[k * WS + r])) & 15) != 0)
        s_vec[k] = 0;
    }
    __syncthreads();
#pragma unroll 1
    for (int u = 0; u < U; ++u) {
      const int64_t v = t0 + threadIdx.x + (int64_t)u * kBT;
      if (v >= t1) break;
      const int64_t d0 = v * E;
      const int32_t k = last_le(s_off, cnt, d0);
      if (s_vec[k] && s_off[k] <= d0 && d0 + E <= s_end[k]) {
        const int64_t byte = (d0 - s_off[k]) * EB;
        const int32_t comm = s_comm[k];
        const int32_t c = s_cs[comm], st = s_cst[comm];
        float inv, cf;
        comm_recip(c, &inv, &cf);
        const char* const* in = s_in + k * WS;
        char* const* out = s_out + k * WS;
        if (comm == 0 && WT > 0) {
          // the data-parallel group: one block, every rank, rank order
          constexpr int WR = WT > 0 ? WT : 1;
          u32x4 x[WR];
#pragma unroll
          for (int r = 0; r < WR; ++r) x[r] = load16<true>(reinterpret_cast<const u32x4*>(in[r] + byte));
          float acc[E];
#pragma unroll
          for (int r = 0; r < WR; ++r) fold16<BF16, PRE>(acc, x[r], r == 0, inv, cf);
          const u32x4 y = pack16<BF16>(acc);
#pragma unroll
          for (int r = 0; r < WR; ++r)
            if (out[r] != nullptr) store16<true>(reinterpret_cast<u32x4*>(out[r] + byte), y);
        } else {
          const int32_t nb = W / c;
          for (int32_t b = 0; b < nb; ++b) {
            float acc[E];
            for (int32_t i = 0; i < c; ++i) {
              const int32_t r = member_of(b, i, c, st);
              fold16<BF16, PRE>(acc, load16<true>(reinterpret_cast<const u32x4*>(in[r] + byte)), i == 0,
                                inv, cf);
            }
            const u32x4 y = pack16<BF16>(acc);
            for (int32_t i = 0; i < c; ++i) {
              const int32_t r = member_of(b, i, c, st);
              if (out[r] != nullptr) store16<true>(reinterpret_cast<u32x4*>(out[r] + byte), y);
            }
          }
        }
      } else {
        const int64_t d1 = min(d0 + E, p.bucket_numel);
        for (int64_t d = d0; d < d1; ++d) {
          const int32_t kk = last_le(s_off, cnt, d);
          if (!(s_off[kk] <= d && d < s_end[kk])) continue;
          const int64_t e = d - s_off[kk];
          const int32_t comm = s_comm[kk];
          const int32_t c = s_cs[comm], st = s_cst[comm];
          float inv, cf;
          comm_recip(c, &inv, &cf);
          const int32_t nb = W / c;
          for (int32_t b = 0; b < nb; ++b) {
            float sum = 0.0f;
            for (int32_t i = 0; i < c; ++i) {
              const int32_t r = member_of(b, i, c, st);
              const float val = pre_elem<BF16>(load_elem<BF16>(s_in[kk * WS + r], e), PRE, inv, cf);
              sum = i == 0 ? val : sum + val;
            }
            for (int32_t i = 0; i < c; ++i) {
              const int32_t r = member_of(b, i, c, st);
              if (s_out[kk * WS + r] != nullptr) store_elem<BF16>(s_out[kk * WS + r], e, sum);
            }
          }
        }
      }
    }
  }
}

// Workgroups per compute unit for a planned launch at W <= 8, from
// interleaved sweeps with one-slot-per-thread tiles at W = 8 bf16: 12 (6.28
// TB/s) against 6.25 at 14, 6.16 at 16, 5.94 at 10 and 5.78 at 8; at W = 16
// fp32 caps of 8 and 12 were 8-20% slower than none.
#ifndef DC_BUF_CAP8
#define DC_BUF_CAP8 12
#endif
#ifndef DC_BUF_CAP16
#define DC_BUF_CAP16 0
#endif
constexpr int kBufPlannedCap = DC_BUF_CAP8;

template <bool BF16, bool PRE, int U>
hipError_t launch_wu(const BufParams& p, int cap, hipStream_t stream) {
  const dim3 grid((unsigned)((p.nslots + kBT * U - 1) / (kBT * U)));
  switch (p.W) {
#define DC_FB_W(w)                                                                              \
  case w:                                                                                       \
    hipLaunchKernelGGL((k_flush_buffers<BF16, w, PRE, U>), grid, dim3(kBT),                     \
                       occupancy_pad(reinterpret_cast<const void*>(&k_flush_buffers<BF16, w, PRE, U>), cap), \
                       stream, p);                                                              \
    break;
    DC_FB_W(2)
    DC_FB_W(4)
    DC_FB_W(8)
    DC_FB_W(16)
#undef DC_FB_W
    default:
      hipLaunchKernelGGL((k_flush_buffers<BF16, 0, PRE, U>), grid, dim3(kBT), 0, stream, p);
  }
  return hipGetLastError();
}

template <bool BF16, bool PRE>
hipError_t launch_w(const BufParams& p, hipStream_t stream) {
  if (p.tiles == nullptr) return launch_wu<BF16, PRE, kBufUSearched>(p, 0, stream);
  return launch_wu<BF16, PRE, kBufU>(p, p.W <= 8 ? kBufPlannedCap : DC_BUF_CAP16, stream);
}

}  // namespace

hipError_t launch_flush_buffers(int32_t W, int32_t dtype, int64_t bucket_numel, const dc_task* tasks,
                                int32_t num_tasks, const void* const* in_ptrs, void* const* out_ptrs,
                                const dc_comm* comms, int32_t num_comms, int32_t pre_div,
                                hipStream_t stream, const dc_tile* tiles) {
  if (bucket_numel == 0 || num_tasks == 0) return hipSuccess;
  const int E = dtype == DC_BF16 ? 8 : 4;
  BufParams p{};
  p.tasks = tasks;
  p.in_ptrs = in_ptrs;
  p.out_ptrs = out_ptrs;
  p.nslots = (bucket_numel + E - 1) / E;
  p.bucket_numel = bucket_numel;
  p.ntasks = num_tasks;
  p.W = W;
  p.num_comms = num_comms;
  p.tiles = tiles;
  for (int q = 0; q < DC_MAX_COMMS; ++q) {
    p.csize[q] = q < num_comms ? comms[q].size : W;
    p.cstride[q] = q < num_comms ? comms[q].stride : 1;
  }
  if (dtype == DC_BF16)
    return pre_div ? launch_w<true, true>(p, stream) : launch_w<true, false>(p, stream);
  return pre_div ? launch_w<false, true>(p, stream) : launch_w<false, false>(p, stream);
}

}  // namespace dc
