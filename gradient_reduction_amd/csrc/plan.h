// Launchers of the device-side planners (plan.hip), called by api.hip after
// their host-side argument checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dc.h"

namespace dc {

struct PlanLaunch {
  int32_t W;
  int32_t dtype;
  int64_t c0;            // first slab column of the bucket
  int64_t numel;         // bucket columns
  const dc_task* tasks;  // device
  int32_t ntasks;
  const int32_t* owner;  // device or null (owner-map mode)
  const int64_t* flat;   // device or null (ZeRO-2 mode, with psize)
  const int64_t* psize;
  int32_t nparams;
  int32_t ncomms;
  dc_tile* tiles;        // device, one record per plan tile
  int64_t* root_tiles;   // device or null: count of whole tiles with a root
};

// Writes every tile record of the bucket's plan (and the root count) on the
// stream; nothing when the bucket has no tiles and no count is asked for.
hipError_t launch_plan_flush(const PlanLaunch& a, hipStream_t stream);

// The fused flush's plan (dc_plan_flush_buffers' records): `count` tiles of
// kBufTile slots over a bucket of `numel` columns.
hipError_t launch_plan_flush_buffers(int32_t dtype, int64_t numel, const dc_task* tasks,
                                     int32_t ntasks, dc_tile* tiles, int64_t count,
                                     hipStream_t stream);

// The relayout's tile plan (dc_plan_relayout_tiles' records): `count`
// destination tiles of kRelayoutTile vectors.
hipError_t launch_plan_relayout_tiles(int32_t dtype, int64_t bucket_col, int64_t bucket_numel,
                                      const dc_piece* pieces, int32_t npieces, int64_t out_numel,
                                      int64_t* tiles, int64_t count, hipStream_t stream);

}  // namespace dc
