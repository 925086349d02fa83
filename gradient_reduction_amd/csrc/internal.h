// Launchers of libdc's kernels.  Called by api.cpp after its host-side
// argument checks; each returns the launch's hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dc.h"

namespace dc {

struct CommSpec {
  int32_t size;
  int32_t stride;
};

struct FlushLaunch {
  int32_t W;
  int32_t dtype;
  int32_t pre_div;
  const void* in;
  void* out;
  int64_t ld_in;
  int64_t ld_out;
  int64_t c0;  // first slab column of the bucket
  int64_t c1;  // one past its last column
  const dc_task* tasks;
  int32_t ntasks;
  const int32_t* owner;
  const int64_t* flat;   // ZeRO-2 mode when non-null (with psize)
  const int64_t* psize;
  int32_t nparams;
  int32_t ncomms;
  CommSpec comms[DC_MAX_COMMS];
  const dc_tile* tiles;  // planned flush when non-null (ntiles records)
  int64_t ntiles;
  int64_t root_tiles;    // planned: tiles that write one row (picks the residency cap)
};

hipError_t launch_flush(const FlushLaunch& a, hipStream_t stream);

// Dynamic LDS a launch of `kernel` reserves, unused, so that at most `cap` of
// its workgroups fit in one compute unit (0 when cap <= 0 or unreachable).
size_t occupancy_pad(const void* kernel, int cap);

// Workgroup cap for a 64-thread streaming launch whose threads each keep
// `rows` row accesses of `u` 16-byte vectors in flight, so that about `kb`
// KB of row accesses are in flight per compute unit (0 = no cap).
int stream_cap(int rows, int u, int kb);

// A tile grid over bucket columns [c0, c1) of a dtype: tile b covers
// vectors [v0 + b*tile, v0 + min((b+1)*tile, nv)) in absolute 16-byte column
// vectors.  `count` is the tile count (0 for an empty bucket).
struct FlushTiles {
  int64_t v0;    // first vector of tile 0 (a multiple of the tile size)
  int64_t nv;    // vectors from v0 to the bucket's last one
  int64_t tile;  // vectors per tile
  int64_t count;
};
// The searched flush's grid: tiles of 128 vectors (2 per thread of a wave).
FlushTiles flush_tiles(int32_t dtype, int64_t c0, int64_t c1);

// The planned flush's grid: plan tiles of kPlanTile vectors (one per thread
// of a wave, one tile per workgroup).
constexpr int64_t kPlanTile = 64;
FlushTiles plan_tiles(int32_t dtype, int64_t c0, int64_t c1);

// Where tile b's record sits among n records: XCD-major.  The hardware deals
// workgroups to the 8 XCDs in turn, so workgroup b runs on XCD b mod 8;
// keeping each XCD's records together lets one 128-byte line serve eight of
// its workgroups from that XCD's L2, where tile order would have every XCD
// fetch every line for one record in eight.
__host__ __device__ inline int64_t tile_slot(int64_t b, int64_t n) {
  const int64_t r = b % 8, q = n / 8, rem = n % 8;
  return r * q + (r < rem ? r : rem) + b / 8;
}

struct GroupTable {
  int32_t num_groups;
  int32_t begin[DC_MAX_GROUPS + 1];
  int32_t parts[DC_MAX_GROUPS];
  int32_t eligible[DC_MAX_GROUPS];
};

hipError_t launch_partition_ids(int32_t num_params, const int64_t* numel, const GroupTable& g,
                                int64_t* flat_offset, int64_t* part_size, int32_t* pid_offsets,
                                int32_t* pids, int64_t pids_capacity, hipStream_t stream);

hipError_t launch_param_part_size(int32_t num_params, const GroupTable& g, const int64_t* part_size,
                                  int64_t* out, hipStream_t stream);

hipError_t launch_owner_map(int32_t W, int32_t num_params, const int32_t* pid_offsets,
                            const int32_t* pids, int64_t pids_capacity, const GroupTable& g,
                            int32_t* owner,
                            int32_t* counts, hipStream_t stream);

hipError_t launch_reduce_scatter(int32_t W, int32_t dtype, const void* in, int64_t ld_in,
                                 void* out, int64_t ld_out, int64_t M, int32_t pre_div,
                                 hipStream_t stream);

hipError_t launch_reduce_scatter_v(int32_t W, int32_t dtype, const void* in, int64_t ld_in,
                                   void* out, int64_t ld_out, const int64_t* seg_start,
                                   int32_t pre_div, hipStream_t stream);

// The planned relayout's grid: tiles of kRelayoutTile destination vectors,
// one per one-wave workgroup; a plan holds one int64 record per tile, at
// tile_slot(t, count): the absolute source vector of the tile's first
// vector when the whole tile copies from one piece with its source on a
// vector boundary, else -1.
constexpr int64_t kRelayoutTile = 64;
inline int64_t relayout_tile_count(int32_t dtype, int64_t out_numel) {
  const int64_t E = 16 / (dtype == DC_BF16 ? 2 : 4);
  const int64_t nvec = (out_numel + E - 1) / E;
  return (nvec + kRelayoutTile - 1) / kRelayoutTile;
}

// tiles == nullptr: every tile searches the piece table.
hipError_t launch_relayout(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                           int64_t ld_out, int64_t bucket_col, int64_t bucket_numel,
                           const dc_piece* pieces, int32_t npieces, int64_t out_numel,
                           const int64_t* tiles, hipStream_t stream);

hipError_t launch_flush_buffers(int32_t W, int32_t dtype, int64_t bucket_numel, const dc_task* tasks,
                                int32_t num_tasks, const void* const* in_ptrs, void* const* out_ptrs,
                                const dc_comm* comms, int32_t num_comms, int32_t pre_div,
                                hipStream_t stream, const dc_tile* tiles = nullptr);

// The planned fused flush's tiles over a bucket of n coordinates, from
// coordinate 0: kBufTile slots of E elements (16 bytes) each, one per thread
// of a one-wave workgroup.  Against two per thread: +4% at W = 8 bf16 with
// 12 workgroups per compute unit, +1.3% at W = 16 fp32.
#ifndef DC_BUF_TILE
#define DC_BUF_TILE 64
#endif
constexpr int64_t kBufTile = DC_BUF_TILE;
inline int64_t buffer_tiles(int32_t dtype, int64_t n) {
  const int64_t E = dtype == DC_BF16 ? 8 : 4;
  return ((n + E - 1) / E + kBufTile - 1) / kBufTile;
}

hipError_t launch_reduce_scatter_ring(int32_t W, int32_t dtype, const void* in, int64_t ld_in,
                                      void* out, int64_t ld_out, int64_t M, int32_t pre_div,
                                      hipStream_t stream);

hipError_t launch_all_gather_step(int32_t W, int32_t dtype, const void* in, int64_t ld_in,
                                  void* out, int64_t ld_out, int64_t L, int32_t algo,
                                  int32_t step, hipStream_t stream);

hipError_t launch_all_gather(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                             int64_t ld_out, int64_t L, int32_t order, int32_t step,
                             hipStream_t stream);

hipError_t launch_accumulate(int32_t rows, const float* x, int64_t ld_x, float* acc,
                             int64_t ld_acc, int64_t M, int32_t init, hipStream_t stream);

hipError_t launch_deferred_reduce(int32_t W, const float* acc, int64_t ld_acc, float* out,
                                  int64_t ld_out, int64_t M, int32_t out_rows,
                                  hipStream_t stream);

hipError_t launch_accumulate_reduce(int32_t W, const float* x, int64_t ld_x, float* acc,
                                    int64_t ld_acc, int32_t init, int32_t keep_acc, float* out,
                                    int64_t ld_out, int32_t out_rows, int64_t M,
                                    hipStream_t stream);

hipError_t launch_round_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t stream);

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

hipError_t launch_stream_rows(const void* src, int64_t src_ld_vec, int32_t rows_read, void* dst,
                              int64_t dst_ld_vec, int32_t rows_written, int64_t nvec,
                              hipStream_t stream);

hipError_t launch_stream_rows_shaped(const void* src, int64_t src_ld_vec, int32_t rows_read,
                                     void* dst, int64_t dst_ld_vec, int32_t rows_written,
                                     int64_t nvec, int32_t group, int32_t cap, hipStream_t stream);

}  // namespace dc
