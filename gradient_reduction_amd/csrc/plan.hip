// Device-side planners: the tile records of the host planners
// (dc_plan_flush, dc_plan_flush_buffers, dc_plan_relayout_tiles), bit for
// bit, written on the stream from tables that live on the device.
// DeepSpeed issue "[REQUEST] DeepCompile ZeRO-1: reduce-to-owner instead of
// AllReduce", Design points: the destinations of a bucket's reductions are
// settled for the whole bucket ahead of the reduction itself; here that is
// done per plan tile, one thread per tile.  A thread finds its tile's task
// (or relayout piece) range by binary search and, for a tile that lies
// inside one task and the bucket, the row its sums go to (or the source run
// it copies).  Integer work: about log2(tasks) reads of the table and one
// record per tile.
#include "internal.h"
#include "plan.h"

namespace dc {
namespace {

constexpr int kPlanThreads = 256;

struct PlanParams {
  const dc_task* tasks;
  const int32_t* owner;
  const int64_t* flat;
  const int64_t* psize;
  dc_tile* tiles;
  int64_t* root_tiles;
  int64_t c0;     // first slab column of the bucket
  int64_t numel;  // bucket columns
  int64_t E;      // elements per 16-byte vector
  int64_t v0;     // first vector of tile 0
  int64_t nv;     // vectors from v0 to the bucket's last one
  int64_t tile;   // vectors per tile
  int64_t count;  // tiles
  int32_t ntasks;
  int32_t nparams;
  int32_t ncomms;
  int32_t W;
};

// How many entries start at or before x (strict: before x), by binary search
// of start(i), which a valid table holds in ascending order; any table keeps
// the reads inside [0, n).
template <typename F>
__device__ __forceinline__ int32_t starting_by(int32_t n, int64_t x, bool strict, F start) {
  int32_t lo = 0, hi = n;
  while (lo < hi) {
    const int32_t mid = lo + (hi - lo) / 2;
    const int64_t o = start(mid);
    if (strict ? o < x : o <= x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int32_t tasks_starting_by(const dc_task* t, int32_t n, int64_t x,
                                                     bool strict) {
  return starting_by(n, x, strict, [&](int32_t i) { return t[i].offset; });
}

// Thread b writes the record of tile b at its XCD-major slot.  The record:
// first = the last task starting at or before the tile's first bucket
// column, last = the last task starting before its end (-1 when none does);
// a tile inside one task and the bucket is whole (flags bit 0, the task's
// communicator in bits 8-15) with its root: the owner in owner-map mode, the
// partition holding every element of the tile in ZeRO-2 mode (a tile cut by
// a partition boundary is not whole), -1 for every member row.  A task whose
// param or communicator lies outside its table gives a tile that is not
// whole, so no table is read out of range.
__global__ __launch_bounds__(kPlanThreads) void k_plan_flush(PlanParams p) {
  const int64_t b = (int64_t)blockIdx.x * kPlanThreads + threadIdx.x;
  bool rooted = false;
  if (b < p.count) {
    dc_tile rec{0, -1, -1, 0};
    if (p.ntasks > 0) {
      const int64_t t0 = b * p.tile, t1 = min(t0 + p.tile, p.nv);
      const int64_t f_lo = (p.v0 + t0) * p.E - p.c0, f_hi = (p.v0 + t1) * p.E - p.c0;
      const int64_t lo = max(f_lo, (int64_t)0), hi = min(f_hi, p.numel);
      const int32_t first = max(tasks_starting_by(p.tasks, p.ntasks, lo, false) - 1, 0);
      int32_t last = max(tasks_starting_by(p.tasks, p.ntasks, hi, true) - 1, first);
      if (p.tasks[0].offset >= hi) last = -1;
      rec.first = first;
      rec.last = last;
      const dc_task t = p.tasks[first];
      if (last == first && f_lo >= 0 && f_hi <= p.numel && t.offset <= f_lo &&
          f_hi <= t.offset + t.numel && t.param >= 0 && t.param < p.nparams && t.comm >= 0 &&
          t.comm < p.ncomms) {
        int32_t root = -1;
        bool whole = true;
        if (t.comm == 0) {
          if (p.flat != nullptr) {
            const int64_t S = p.psize[t.param];
            if (S > 0) {
              const int64_t a = p.flat[t.param];
              const int64_t q0 = (a + (f_lo - t.offset)) / S;
              const int64_t q1 = (a + (f_hi - 1 - t.offset)) / S;
              if (q0 == q1 && q0 >= 0 && q0 < p.W) root = (int32_t)q0;
              else whole = false;
            }
          } else if (p.owner != nullptr) {
            const int32_t o = p.owner[t.param];
            if (o >= 0 && o < p.W) root = o;
          }
        }
        if (whole) {
          rec.root = root;
          rec.flags = 1 | (t.comm << 8);
          rooted = root >= 0;
        }
      }
    }
    p.tiles[tile_slot(b, p.count)] = rec;
  }
  if (p.root_tiles != nullptr) {
    // the workgroup's count of tiles with a root: wave counts summed in LDS,
    // then one device atomic per workgroup (one per wave doubled the
    // planner's time on a 131K-tile bucket, 20 against 10 us)
    __shared__ unsigned int s_roots;
    if (threadIdx.x == 0) s_roots = 0;
    __syncthreads();
    const uint64_t m = __ballot(rooted);
    if ((threadIdx.x & 63) == 0 && m != 0) atomicAdd(&s_roots, (unsigned int)__popcll(m));
    __syncthreads();
    if (threadIdx.x == 0 && s_roots != 0)
      atomicAdd(reinterpret_cast<unsigned long long*>(p.root_tiles), (unsigned long long)s_roots);
  }
}

// The fused flush's tiles: kBufTile slots of E columns each over the
// bucket's buffer coordinates.  A tile is whole (flags 1) when it lies
// inside one task on the data-parallel communicator whose offset is a whole
// number of slots; the root is always -1 (the pointer tables say which
// buffers exist).
__global__ __launch_bounds__(kPlanThreads) void k_plan_flush_buffers(const dc_task* __restrict__ tasks,
                                                                     int32_t ntasks, int64_t numel,
                                                                     int64_t E, int64_t count,
                                                                     dc_tile* __restrict__ tiles) {
  const int64_t b = (int64_t)blockIdx.x * kPlanThreads + threadIdx.x;
  if (b >= count) return;
  const int64_t nslots = (numel + E - 1) / E;
  const int64_t s0 = b * kBufTile, s1 = min(s0 + kBufTile, nslots);
  const int64_t lo = s0 * E, hi = min(s1 * E, numel);
  const int32_t first = max(tasks_starting_by(tasks, ntasks, lo, false) - 1, 0);
  int32_t last = max(tasks_starting_by(tasks, ntasks, hi, true) - 1, first);
  if (tasks[0].offset >= hi) last = -1;
  const dc_task t = tasks[first];
  const bool whole = last == first && t.comm == 0 && t.offset % E == 0 && t.offset <= lo &&
                     s1 * E <= t.offset + t.numel;
  tiles[tile_slot(b, count)] = dc_tile{first, last, -1, whole ? 1 : 0};
}

// The relayout's destination tiles of kRelayoutTile vectors: a tile whose
// columns all belong to one piece (the last piece starting at or before
// each column; no later piece starts inside the tile) copies straight from
// that piece when its source run starts on a vector and stays in the bucket:
// the record is the run's first absolute source vector, else -1.
__global__ __launch_bounds__(kPlanThreads) void k_plan_relayout_tiles(
    const dc_piece* __restrict__ pieces, int32_t npieces, int64_t bucket_col, int64_t bucket_numel,
    int64_t out_numel, int64_t E, int64_t count, int64_t* __restrict__ tiles) {
  const int64_t t = (int64_t)blockIdx.x * kPlanThreads + threadIdx.x;
  if (t >= count) return;
  const int64_t span = kRelayoutTile * E;
  const int64_t d0 = t * span, d1 = d0 + span;
  int64_t rec = -1;
  if (npieces > 0 && d1 <= out_numel) {
    const auto dst = [&](int32_t i) { return pieces[i].dst; };
    const int32_t k = max(starting_by(npieces, d0, false, dst) - 1, 0);
    const dc_piece pc = pieces[k];
    if (pc.dst <= d0 && d1 <= pc.dst + pc.len && (k + 1 == npieces || pieces[k + 1].dst >= d1)) {
      const int64_t src0 = pc.src + (d0 - pc.dst);
      if (src0 >= 0 && src0 + span <= bucket_numel && (bucket_col + src0) % E == 0)
        rec = (bucket_col + src0) / E;
    }
  }
  tiles[tile_slot(t, count)] = rec;
}

// Clears the root count before the planner adds to it (a kernel, so that a
// captured graph holds no memset node).
__global__ void k_clear_count(int64_t* n) {
  if (threadIdx.x == 0) *n = 0;
}

}  // namespace

hipError_t launch_plan_flush(const PlanLaunch& a, hipStream_t stream) {
  const FlushTiles g = plan_tiles(a.dtype, a.c0, a.c0 + a.numel);
  if (a.root_tiles != nullptr) {
    hipLaunchKernelGGL(k_clear_count, dim3(1), dim3(64), 0, stream, a.root_tiles);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (g.count == 0) return hipSuccess;
  PlanParams p{};
  p.tasks = a.tasks;
  p.owner = a.owner;
  p.flat = a.flat;
  p.psize = a.psize;
  p.tiles = a.tiles;
  p.root_tiles = a.root_tiles;
  p.c0 = a.c0;
  p.numel = a.numel;
  p.E = a.dtype == DC_BF16 ? 8 : 4;
  p.v0 = g.v0;
  p.nv = g.nv;
  p.tile = g.tile;
  p.count = g.count;
  p.ntasks = a.ntasks;
  p.nparams = a.nparams;
  p.ncomms = a.ncomms;
  p.W = a.W;
  const int64_t blocks = (g.count + kPlanThreads - 1) / kPlanThreads;
  hipLaunchKernelGGL(k_plan_flush, dim3((unsigned)blocks), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_plan_flush_buffers(int32_t dtype, int64_t numel, const dc_task* tasks,
                                     int32_t ntasks, dc_tile* tiles, int64_t count,
                                     hipStream_t stream) {
  if (count == 0 || ntasks == 0) return hipSuccess;
  const int64_t blocks = (count + kPlanThreads - 1) / kPlanThreads;
  hipLaunchKernelGGL(k_plan_flush_buffers, dim3((unsigned)blocks), dim3(kPlanThreads), 0, stream,
                     tasks, ntasks, numel, (int64_t)(dtype == DC_BF16 ? 8 : 4), count, tiles);
  return hipGetLastError();
}

hipError_t launch_plan_relayout_tiles(int32_t dtype, int64_t bucket_col, int64_t bucket_numel,
                                      const dc_piece* pieces, int32_t npieces, int64_t out_numel,
                                      int64_t* tiles, int64_t count, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  const int64_t blocks = (count + kPlanThreads - 1) / kPlanThreads;
  hipLaunchKernelGGL(k_plan_relayout_tiles, dim3((unsigned)blocks), dim3(kPlanThreads), 0, stream,
                     pieces, npieces, bucket_col, bucket_numel, out_numel,
                     (int64_t)(dtype == DC_BF16 ? 8 : 4), count, tiles);
  return hipGetLastError();
}

}  // namespace dc
