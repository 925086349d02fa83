// C ABI of libdc (declared in include/dc.h): host-side argument checks,
// error reporting, the host-only probe and task-table check, and the kernel
// launches.  Every check runs before the first HIP call, so a rejected call
// touches no device state.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "dc.h"
#include "internal.h"
#include "plan.h"

namespace {

thread_local std::string g_last_error;

dc_status fail(dc_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

dc_status ok() {
  g_last_error.clear();
  return DC_OK;
}

dc_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int elem_bytes(int32_t dtype) { return dtype == DC_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) share a byte.
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// Largest row stride, column count or byte count accepted: rows * ld * 4
// bytes (rows up to 65535) and W * ld * 16 then stay inside int64, so no size
// arithmetic below can wrap.
constexpr int64_t kMaxExtent = (int64_t)1 << 44;

dc_status check_extent(const char* name, int64_t n) {
  if (n > kMaxExtent) return fail(DC_ERR_SHAPE, "%s=%lld exceeds 2^44", name, (long long)n);
  return DC_OK;
}

dc_status check_w(int32_t W) {
  if (W < 1 || W > DC_MAX_W) return fail(DC_ERR_ARG, "W=%d outside [1, %d]", W, DC_MAX_W);
  return DC_OK;
}

dc_status check_dtype(int32_t dtype) {
  if (dtype != DC_BF16 && dtype != DC_F32) return fail(DC_ERR_DTYPE, "unknown dtype %d", dtype);
  return DC_OK;
}

// A [rows, ld] slab: non-NULL, 16-byte aligned base and stride, ld >= cols.
dc_status check_slab(const char* name, const void* p, int64_t ld, int64_t cols, int32_t dtype) {
  if (p == nullptr) return fail(DC_ERR_NULL, "%s is NULL", name);
  if (ld > kMaxExtent || cols > kMaxExtent)
    return fail(DC_ERR_SHAPE, "%s: ld=%lld or %lld columns exceeds 2^44", name, (long long)ld, (long long)cols);
  if (ld < 1 || ld < cols) return fail(DC_ERR_SHAPE, "%s: ld=%lld < %lld columns", name, (long long)ld, (long long)cols);
  if (!aligned16(p) || (ld * elem_bytes(dtype)) % 16 != 0)
    return fail(DC_ERR_ALIGN, "%s: base or row stride (ld=%lld) not 16-byte aligned", name, (long long)ld);
  return DC_OK;
}

dc_status check_groups(int32_t num_params, int32_t num_groups, const int32_t* group_begin) {
  if (num_params < 0) return fail(DC_ERR_ARG, "num_params=%d < 0", num_params);
  if (num_groups < 1 || num_groups > DC_MAX_GROUPS)
    return fail(DC_ERR_ARG, "num_groups=%d outside [1, %d]", num_groups, DC_MAX_GROUPS);
  if (group_begin == nullptr) return fail(DC_ERR_NULL, "group_begin is NULL");
  if (group_begin[0] != 0 || group_begin[num_groups] != num_params)
    return fail(DC_ERR_SHAPE, "group_begin must run from 0 to num_params=%d", num_params);
  for (int g = 0; g < num_groups; ++g)
    if (group_begin[g + 1] < group_begin[g]) return fail(DC_ERR_SHAPE, "group_begin decreases at group %d", g);
  return DC_OK;
}

dc_status check_comms(int32_t W, const dc_comm* comms, int32_t num_comms) {
  if (comms == nullptr) return fail(DC_ERR_NULL, "comms is NULL");
  if (num_comms < 1 || num_comms > DC_MAX_COMMS)
    return fail(DC_ERR_ARG, "num_comms=%d outside [1, %d]", num_comms, DC_MAX_COMMS);
  if (comms[0].size != W || comms[0].stride != 1)
    return fail(DC_ERR_ARG, "comms[0] must be the data-parallel comm {W=%d, 1}", W);
  for (int k = 0; k < num_comms; ++k) {
    const int32_t c = comms[k].size, s = comms[k].stride;
    if (c < 1 || W % c != 0) return fail(DC_ERR_ARG, "comms[%d].size=%d does not divide W=%d", k, c, W);
    if (s != 1 && s != W / c) return fail(DC_ERR_ARG, "comms[%d].stride=%d is neither 1 nor W/size", k, s);
  }
  return DC_OK;
}

// The data-parallel group: the same world size, and group rank i is global
// rank i for every i ([DS] Design points: groups reduced over another
// communicator take no part in the owner map).
bool dp_group(int32_t W, int32_t g, const int32_t* group_comm_size,
              const int32_t* group_rank_to_global) {
  if (group_comm_size[g] != W) return false;
  for (int i = 0; i < W; ++i)
    if (group_rank_to_global[(int64_t)g * W + i] != i) return false;
  return true;
}

// The ranks holding task t's param: every rank whose optimizer partition
// (group rank, in every block of a sub-communicator) is in the param's
// partition list.  hd gets W flags.  The probe's `kept` and the copy-out
// targets of the fused flush both come from here.
dc_status task_holders(int32_t W, const dc_task& k, int32_t t, const int32_t* pid_offsets,
                       const int32_t* pids, const dc_comm* comms, char* hd) {
  const int32_t c = comms[k.comm].size, s = comms[k.comm].stride;
  std::fill(hd, hd + W, 0);
  const int32_t o0 = pid_offsets[k.param], o1 = pid_offsets[k.param + 1];
  if (o1 > o0 && pids == nullptr) return fail(DC_ERR_NULL, "pids is NULL");
  for (int32_t e = o0; e < o1; ++e) {
    const int32_t q = pids[e];
    if (q < 0 || q >= c)
      return fail(DC_ERR_TASKS, "task %d: param %d: partition %d outside its comm of %d", t,
                  k.param, q, c);
    for (int32_t blk = 0; blk < W / c; ++blk) hd[(s == 1 ? blk * c : blk) + q * s] = 1;
  }
  return DC_OK;
}

}  // namespace

extern "C" {

const char* dc_version(void) { return "dc 0.1.0 (gfx950)"; }

const char* dc_strerror(dc_status status) {
  switch (status) {
    case DC_OK: return "ok";
    case DC_ERR_NULL: return "a required pointer is NULL";
    case DC_ERR_ARG: return "an argument is out of range or buffers overlap";
    case DC_ERR_SHAPE: return "sizes or strides do not fit together";
    case DC_ERR_ALIGN: return "a slab base or stride is not 16-byte aligned";
    case DC_ERR_DTYPE: return "unknown dtype";
    case DC_ERR_TASKS: return "the task table breaks its contract";
    case DC_ERR_HIP: return "a HIP call failed";
    case DC_ERR_UNSUPPORTED: return "not supported by this library";
    default: return "unknown status";
  }
}

const char* dc_last_error(void) { return g_last_error.c_str(); }

dc_status dc_partition_ids(int32_t W, int32_t num_params, const int64_t* numel,
                           int32_t num_groups, const int32_t* group_begin,
                           const int32_t* group_parts, int64_t* flat_offset, int64_t* part_size,
                           int32_t* pid_offsets, int32_t* pids, int64_t pids_capacity,
                           void* stream) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_groups(num_params, num_groups, group_begin))) return st;
  if (group_parts == nullptr) return fail(DC_ERR_NULL, "group_parts is NULL");
  if (part_size == nullptr || pid_offsets == nullptr) return fail(DC_ERR_NULL, "part_size or pid_offsets is NULL");
  if (num_params > 0 && (numel == nullptr || flat_offset == nullptr || pids == nullptr))
    return fail(DC_ERR_NULL, "numel, flat_offset or pids is NULL");
  int64_t need = num_params;
  for (int g = 0; g < num_groups; ++g) {
    if (group_parts[g] < 1 || group_parts[g] > DC_MAX_W)
      return fail(DC_ERR_ARG, "group_parts[%d]=%d outside [1, %d]", g, group_parts[g], DC_MAX_W);
    need += group_parts[g] - 1;
  }
  if (pids_capacity < need || pids_capacity > INT32_MAX)
    return fail(DC_ERR_SHAPE, "pids_capacity=%lld, need %lld (at most 2^31-1)", (long long)pids_capacity, (long long)need);
  dc::GroupTable g{};
  g.num_groups = num_groups;
  for (int k = 0; k <= num_groups; ++k) g.begin[k] = group_begin[k];
  for (int k = 0; k < num_groups; ++k) g.parts[k] = group_parts[k];
  return hip_status(dc::launch_partition_ids(num_params, numel, g, flat_offset, part_size,
                                             pid_offsets, pids, pids_capacity,
                                             static_cast<hipStream_t>(stream)),
                    "partition ids launch");
}

dc_status dc_build_owner_map(int32_t W, int32_t num_params, const int32_t* pid_offsets,
                             const int32_t* pids, int64_t pids_capacity, int32_t num_groups,
                             const int32_t* group_begin, const int32_t* group_comm_size,
                             const int32_t* group_rank_to_global, int32_t* owner, int32_t* counts,
                             void* stream) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_groups(num_params, num_groups, group_begin))) return st;
  if (group_comm_size == nullptr || group_rank_to_global == nullptr)
    return fail(DC_ERR_NULL, "group_comm_size or group_rank_to_global is NULL");
  if (pid_offsets == nullptr || counts == nullptr) return fail(DC_ERR_NULL, "pid_offsets or counts is NULL");
  if (num_params > 0 && owner == nullptr) return fail(DC_ERR_NULL, "owner is NULL");
  if (pids_capacity < 0) return fail(DC_ERR_ARG, "pids_capacity < 0");
  if (pids_capacity > 0 && pids == nullptr) return fail(DC_ERR_NULL, "pids is NULL");
  dc::GroupTable g{};
  g.num_groups = num_groups;
  for (int k = 0; k <= num_groups; ++k) g.begin[k] = group_begin[k];
  for (int k = 0; k < num_groups; ++k) {
    g.eligible[k] = dp_group(W, k, group_comm_size, group_rank_to_global);
    g.parts[k] = group_comm_size[k];
  }
  return hip_status(dc::launch_owner_map(W, num_params, pid_offsets, pids, pids_capacity, g, owner,
                                         counts, static_cast<hipStream_t>(stream)),
                    "owner map launch");
}

dc_status dc_validate_tasks(int32_t W, const dc_task* tasks, int32_t num_tasks,
                            int64_t bucket_numel, int32_t num_params, const dc_comm* comms,
                            int32_t num_comms) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_comms(W, comms, num_comms))) return st;
  if (num_tasks < 0) return fail(DC_ERR_ARG, "num_tasks=%d < 0", num_tasks);
  if (num_tasks > 0 && tasks == nullptr) return fail(DC_ERR_NULL, "tasks is NULL");
  int64_t pos = 0;
  for (int32_t t = 0; t < num_tasks; ++t) {
    const dc_task& k = tasks[t];
    if (k.offset != pos) return fail(DC_ERR_TASKS, "task %d: offset %lld, expected %lld (sorted and packed)", t, (long long)k.offset, (long long)pos);
    if (k.numel < 0) return fail(DC_ERR_TASKS, "task %d: numel %lld < 0", t, (long long)k.numel);
    if (k.param < 0 || k.param >= num_params) return fail(DC_ERR_TASKS, "task %d: param %d outside [0, %d)", t, k.param, num_params);
    if (k.comm < 0 || k.comm >= num_comms) return fail(DC_ERR_TASKS, "task %d: comm %d outside [0, %d)", t, k.comm, num_comms);
    pos += k.numel;
  }
  if (pos != bucket_numel) return fail(DC_ERR_TASKS, "tasks cover %lld columns, bucket has %lld", (long long)pos, (long long)bucket_numel);
  return ok();
}

}  // extern "C"

namespace {

dc_status flush_common(const char* fn, int32_t W, int32_t dtype, const void* slab_in, int64_t ld_in,
                       void* slab_out, int64_t ld_out, int64_t bucket_col, int64_t bucket_numel,
                       const dc_task* tasks, int32_t num_tasks, const int32_t* owner,
                       const int64_t* flat, const int64_t* psize, int32_t num_params,
                       const dc_comm* comms, int32_t num_comms, int32_t pre_div, void* stream,
                       const dc_tile* tiles = nullptr, int64_t num_tiles = -1,
                       int64_t root_tiles = 0) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_dtype(dtype)) || (st = check_comms(W, comms, num_comms))) return st;
  if (bucket_col < 0 || bucket_numel < 0)
    return fail(DC_ERR_ARG, "bucket_col=%lld, bucket_numel=%lld", (long long)bucket_col, (long long)bucket_numel);
  if ((st = check_extent("bucket_col", bucket_col)) || (st = check_extent("bucket_numel", bucket_numel))) return st;
  const int64_t end = bucket_col + bucket_numel;
  if ((st = check_slab("slab_in", slab_in, ld_in, end, dtype)) ||
      (st = check_slab("slab_out", slab_out, ld_out, end, dtype)))
    return st;
  if (num_tasks < 0 || num_params < 0) return fail(DC_ERR_ARG, "num_tasks or num_params < 0");
  if (num_tasks > 0 && tasks == nullptr) return fail(DC_ERR_NULL, "tasks is NULL");
  if (pre_div != 0 && pre_div != 1) return fail(DC_ERR_ARG, "pre_div=%d", pre_div);
  const int64_t b = elem_bytes(dtype);
  if (slab_in == slab_out) {
    if (ld_in != ld_out) return fail(DC_ERR_ARG, "in-place flush needs ld_in == ld_out");
  } else if (overlaps(slab_in, W * ld_in * b, slab_out, W * ld_out * b)) {
    return fail(DC_ERR_ARG, "slab_in and slab_out overlap without being the same slab");
  }
  if (num_tiles >= 0) {  // planned
    const int64_t want = dc::plan_tiles(dtype, bucket_col, end).count;
    if (tiles == nullptr && want > 0) return fail(DC_ERR_NULL, "tiles is NULL");
    if (num_tiles != want)
      return fail(DC_ERR_SHAPE, "num_tiles=%lld, the bucket has %lld tiles", (long long)num_tiles,
                  (long long)want);
  }
  dc::FlushLaunch a{};
  a.W = W;
  a.dtype = dtype;
  a.pre_div = pre_div;
  a.in = slab_in;
  a.out = slab_out;
  a.ld_in = ld_in;
  a.ld_out = ld_out;
  a.c0 = bucket_col;
  a.c1 = end;
  a.tasks = tasks;
  a.ntasks = num_tasks;
  a.owner = owner;
  a.flat = flat;
  a.psize = psize;
  a.nparams = num_params;
  a.ncomms = num_comms;
  for (int k = 0; k < num_comms; ++k) a.comms[k] = {comms[k].size, comms[k].stride};
  a.tiles = num_tiles >= 0 ? tiles : nullptr;
  a.ntiles = num_tiles >= 0 ? num_tiles : 0;
  a.root_tiles = num_tiles >= 0 ? root_tiles : 0;
  return hip_status(dc::launch_flush(a, static_cast<hipStream_t>(stream)), fn);
}

}  // namespace

extern "C" {

dc_status dc_flush_bucket(int32_t W, int32_t dtype, const void* slab_in, int64_t ld_in,
                          void* slab_out, int64_t ld_out, int64_t bucket_col,
                          int64_t bucket_numel, const dc_task* tasks, int32_t num_tasks,
                          const int32_t* owner, int32_t num_params, const dc_comm* comms,
                          int32_t num_comms, int32_t pre_div, void* stream) {
  return flush_common("flush launch", W, dtype, slab_in, ld_in, slab_out, ld_out, bucket_col,
                      bucket_numel, tasks, num_tasks, owner, nullptr, nullptr, num_params, comms,
                      num_comms, pre_div, stream);
}

dc_status dc_flush_bucket_zero2(int32_t W, int32_t dtype, const void* slab_in, int64_t ld_in,
                                void* slab_out, int64_t ld_out, int64_t bucket_col,
                                int64_t bucket_numel, const dc_task* tasks, int32_t num_tasks,
                                const int64_t* flat_offset, const int64_t* part_size,
                                int32_t num_params, const dc_comm* comms, int32_t num_comms,
                                int32_t pre_div, void* stream) {
  if (num_tasks > 0 && (flat_offset == nullptr || part_size == nullptr))
    return fail(DC_ERR_NULL, "flat_offset or part_size is NULL");
  return flush_common("ZeRO-2 flush launch", W, dtype, slab_in, ld_in, slab_out, ld_out,
                      bucket_col, bucket_numel, tasks, num_tasks, nullptr, flat_offset, part_size,
                      num_params, comms, num_comms, pre_div, stream);
}

dc_status dc_flush_bucket_planned(int32_t W, int32_t dtype, const void* slab_in, int64_t ld_in,
                                  void* slab_out, int64_t ld_out, int64_t bucket_col,
                                  int64_t bucket_numel, const dc_task* tasks, int32_t num_tasks,
                                  const int32_t* owner, const int64_t* flat_offset,
                                  const int64_t* part_size, int32_t num_params,
                                  const dc_comm* comms, int32_t num_comms, int32_t pre_div,
                                  const dc_tile* tiles, int64_t num_tiles, int64_t root_tiles,
                                  void* stream) {
  if ((flat_offset == nullptr) != (part_size == nullptr))
    return fail(DC_ERR_NULL, "flat_offset and part_size go together");
  if (flat_offset != nullptr && owner != nullptr)
    return fail(DC_ERR_ARG, "ZeRO-2 mode (flat_offset given) takes no owner map");
  dc_status st;
  if ((st = check_extent("num_tiles", num_tiles))) return st;
  if (num_tiles < 0) return fail(DC_ERR_ARG, "num_tiles < 0");
  if (root_tiles < 0 || root_tiles > num_tiles)
    return fail(DC_ERR_ARG, "root_tiles=%lld outside [0, num_tiles=%lld]", (long long)root_tiles,
                (long long)num_tiles);
  return flush_common("planned flush launch", W, dtype, slab_in, ld_in, slab_out, ld_out,
                      bucket_col, bucket_numel, tasks, num_tasks, owner, flat_offset, part_size,
                      num_params, comms, num_comms, pre_div, stream, tiles, num_tiles, root_tiles);
}

dc_status dc_plan_flush(int32_t W, int32_t dtype, int64_t bucket_col, int64_t bucket_numel,
                        const dc_task* tasks, int32_t num_tasks, const int32_t* owner,
                        const int64_t* flat_offset, const int64_t* part_size, int32_t num_params,
                        const dc_comm* comms, int32_t num_comms, dc_tile* tiles,
                        int64_t capacity, int64_t* num_tiles, int64_t* root_tiles) {
  dc_status st;
  if ((st = check_dtype(dtype))) return st;
  if (num_tiles == nullptr) return fail(DC_ERR_NULL, "num_tiles is NULL");
  if (bucket_col < 0 || bucket_numel < 0)
    return fail(DC_ERR_ARG, "bucket_col=%lld, bucket_numel=%lld", (long long)bucket_col, (long long)bucket_numel);
  if ((st = check_extent("bucket_col", bucket_col)) || (st = check_extent("bucket_numel", bucket_numel)))
    return st;
  if ((flat_offset == nullptr) != (part_size == nullptr))
    return fail(DC_ERR_NULL, "flat_offset and part_size go together");
  if (flat_offset != nullptr && owner != nullptr)
    return fail(DC_ERR_ARG, "ZeRO-2 mode (flat_offset given) takes no owner map");
  if ((st = dc_validate_tasks(W, tasks, num_tasks, bucket_numel, num_params, comms, num_comms)))
    return st;
  const int64_t c0 = bucket_col, c1 = bucket_col + bucket_numel;
  const dc::FlushTiles g = dc::plan_tiles(dtype, c0, c1);
  *num_tiles = g.count;
  if (tiles == nullptr) return ok();  // size query
  if (capacity < g.count)
    return fail(DC_ERR_SHAPE, "capacity=%lld < %lld tiles", (long long)capacity, (long long)g.count);
  int64_t roots = 0;
  if (g.count > 0 && num_tasks == 0) {
    for (int64_t b = 0; b < g.count; ++b) tiles[b] = dc_tile{0, -1, -1, 0};
    if (root_tiles != nullptr) *root_tiles = 0;
    return ok();
  }
  const int64_t E = dtype == DC_BF16 ? 8 : 4;
  // tasks are sorted and packed: walk them alongside the tiles
  int32_t k = 0;
  for (int64_t b = 0; b < g.count; ++b) {
    const int64_t t0 = b * g.tile, t1 = std::min(t0 + g.tile, g.nv);
    const int64_t f_lo = (g.v0 + t0) * E - c0, f_hi = (g.v0 + t1) * E - c0;
    const int64_t lo = std::max(f_lo, (int64_t)0), hi = std::min(f_hi, bucket_numel);
    // first: the last task starting at or before lo; last: the last starting before hi
    while (k + 1 < num_tasks && tasks[k + 1].offset <= lo) ++k;
    int32_t last = k;
    while (last + 1 < num_tasks && tasks[last + 1].offset < hi) ++last;
    if (tasks[0].offset >= hi) last = -1;
    dc_tile rec{k, last, -1, 0};
    const dc_task& t = tasks[k];
    if (last == k && f_lo >= 0 && f_hi <= bucket_numel && t.offset <= f_lo &&
        f_hi <= t.offset + t.numel) {
      int32_t root = -1;
      bool whole = true;
      if (t.comm == 0) {
        if (flat_offset != nullptr) {
          const int64_t S = part_size[t.param];
          if (S > 0) {
            const int64_t a = flat_offset[t.param];
            const int64_t q0 = (a + (f_lo - t.offset)) / S, q1 = (a + (f_hi - 1 - t.offset)) / S;
            if (q0 == q1 && q0 >= 0 && q0 < W) root = (int32_t)q0;
            else whole = false;
          }
        } else if (owner != nullptr && owner[t.param] >= 0 && owner[t.param] < W) {
          root = owner[t.param];
        }
      }
      if (whole) {
        rec.root = root;
        rec.flags = 1 | (t.comm << 8);
        roots += root >= 0;
      }
    }
    tiles[dc::tile_slot(b, g.count)] = rec;
  }
  if (root_tiles != nullptr) *root_tiles = roots;
  return ok();
}

dc_status dc_plan_flush_device(int32_t W, int32_t dtype, int64_t bucket_col, int64_t bucket_numel,
                               const dc_task* tasks, int32_t num_tasks, const int32_t* owner,
                               const int64_t* flat_offset, const int64_t* part_size,
                               int32_t num_params, const dc_comm* comms, int32_t num_comms,
                               dc_tile* tiles, int64_t capacity, int64_t* num_tiles,
                               int64_t* root_tiles, void* stream) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_dtype(dtype)) || (st = check_comms(W, comms, num_comms))) return st;
  if (num_tiles == nullptr) return fail(DC_ERR_NULL, "num_tiles is NULL");
  if (bucket_col < 0 || bucket_numel < 0)
    return fail(DC_ERR_ARG, "bucket_col=%lld, bucket_numel=%lld", (long long)bucket_col, (long long)bucket_numel);
  if ((st = check_extent("bucket_col", bucket_col)) || (st = check_extent("bucket_numel", bucket_numel)))
    return st;
  if (num_tasks < 0 || num_params < 0) return fail(DC_ERR_ARG, "num_tasks or num_params < 0");
  if ((flat_offset == nullptr) != (part_size == nullptr))
    return fail(DC_ERR_NULL, "flat_offset and part_size go together");
  if (flat_offset != nullptr && owner != nullptr)
    return fail(DC_ERR_ARG, "ZeRO-2 mode (flat_offset given) takes no owner map");
  const dc::FlushTiles g = dc::plan_tiles(dtype, bucket_col, bucket_col + bucket_numel);
  *num_tiles = g.count;
  if (tiles == nullptr) return ok();  // size query: nothing is launched
  if (capacity < g.count)
    return fail(DC_ERR_SHAPE, "capacity=%lld < %lld tiles", (long long)capacity, (long long)g.count);
  if (num_tasks > 0 && tasks == nullptr) return fail(DC_ERR_NULL, "tasks is NULL");
  dc::PlanLaunch a{};
  a.W = W;
  a.dtype = dtype;
  a.c0 = bucket_col;
  a.numel = bucket_numel;
  a.tasks = tasks;
  a.ntasks = num_tasks;
  a.owner = owner;
  a.flat = flat_offset;
  a.psize = part_size;
  a.nparams = num_params;
  a.ncomms = num_comms;
  a.tiles = tiles;
  a.root_tiles = root_tiles;
  return hip_status(dc::launch_plan_flush(a, static_cast<hipStream_t>(stream)), "device flush planner launch");
}

dc_status dc_flush_bucket_buffers(int32_t W, int32_t dtype, int64_t bucket_numel,
                                  const dc_task* tasks, int32_t num_tasks,
                                  const void* const* in_ptrs, void* const* out_ptrs,
                                  const dc_comm* comms, int32_t num_comms, int32_t pre_div,
                                  void* stream) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_dtype(dtype)) || (st = check_comms(W, comms, num_comms))) return st;
  if (bucket_numel < 0 || num_tasks < 0)
    return fail(DC_ERR_ARG, "bucket_numel=%lld, num_tasks=%d", (long long)bucket_numel, num_tasks);
  if (num_tasks > 0 && (tasks == nullptr || in_ptrs == nullptr || out_ptrs == nullptr))
    return fail(DC_ERR_NULL, "tasks, in_ptrs or out_ptrs is NULL");
  if (pre_div != 0 && pre_div != 1) return fail(DC_ERR_ARG, "pre_div=%d", pre_div);
  return hip_status(dc::launch_flush_buffers(W, dtype, bucket_numel, tasks, num_tasks, in_ptrs, out_ptrs,
                                             comms, num_comms, pre_div, static_cast<hipStream_t>(stream)),
                    "buffer flush launch");
}

dc_status dc_plan_flush_buffers(int32_t W, int32_t dtype, int64_t bucket_numel, const dc_task* tasks,
                                int32_t num_tasks, const dc_comm* comms, int32_t num_comms,
                                dc_tile* tiles, int64_t capacity, int64_t* num_tiles) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_dtype(dtype)) || (st = check_comms(W, comms, num_comms))) return st;
  if (num_tiles == nullptr) return fail(DC_ERR_NULL, "num_tiles is NULL");
  if (bucket_numel < 0 || num_tasks < 0) return fail(DC_ERR_ARG, "bucket_numel or num_tasks < 0");
  if ((st = check_extent("bucket_numel", bucket_numel))) return st;
  if (num_tasks > 0 && tasks == nullptr) return fail(DC_ERR_NULL, "tasks is NULL");
  int64_t end = 0;
  for (int32_t t = 0; t < num_tasks; ++t) {
    const dc_task& k = tasks[t];
    if (k.numel < 0 || k.offset < end || k.offset + k.numel > bucket_numel)
      return fail(DC_ERR_TASKS, "task %d: offset %lld numel %lld (sorted, disjoint, inside %lld)", t,
                  (long long)k.offset, (long long)k.numel, (long long)bucket_numel);
    if (k.comm < 0 || k.comm >= num_comms) return fail(DC_ERR_TASKS, "task %d: comm %d", t, k.comm);
    end = k.offset + k.numel;
  }
  const int64_t count = num_tasks > 0 ? dc::buffer_tiles(dtype, bucket_numel) : 0;
  *num_tiles = count;
  if (tiles == nullptr) return ok();  // size query
  if (capacity < count)
    return fail(DC_ERR_SHAPE, "capacity=%lld < %lld tiles", (long long)capacity, (long long)count);
  const int64_t E = dtype == DC_BF16 ? 8 : 4;
  const int64_t nslots = (bucket_numel + E - 1) / E;
  int32_t k = 0;
  for (int64_t b = 0; b < count; ++b) {
    const int64_t s0 = b * dc::kBufTile, s1 = std::min(s0 + dc::kBufTile, nslots);
    const int64_t lo = s0 * E, hi = std::min(s1 * E, bucket_numel);
    // first: the last task starting at or before lo; last: the last starting before hi
    while (k + 1 < num_tasks && tasks[k + 1].offset <= lo) ++k;
    int32_t last = k;
    while (last + 1 < num_tasks && tasks[last + 1].offset < hi) ++last;
    if (tasks[0].offset >= hi) last = -1;
    const dc_task& t = tasks[k];
    const bool whole = last == k && t.comm == 0 && t.offset % E == 0 && t.offset <= lo &&
                       s1 * E <= t.offset + t.numel;
    tiles[dc::tile_slot(b, count)] = dc_tile{k, last, -1, whole ? 1 : 0};
  }
  return ok();
}

dc_status dc_plan_flush_buffers_device(int32_t W, int32_t dtype, int64_t bucket_numel,
                                       const dc_task* tasks, int32_t num_tasks,
                                       const dc_comm* comms, int32_t num_comms, dc_tile* tiles,
                                       int64_t capacity, int64_t* num_tiles, void* stream) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_dtype(dtype)) || (st = check_comms(W, comms, num_comms))) return st;
  if (num_tiles == nullptr) return fail(DC_ERR_NULL, "num_tiles is NULL");
  if (bucket_numel < 0 || num_tasks < 0) return fail(DC_ERR_ARG, "bucket_numel or num_tasks < 0");
  if ((st = check_extent("bucket_numel", bucket_numel))) return st;
  const int64_t count = num_tasks > 0 ? dc::buffer_tiles(dtype, bucket_numel) : 0;
  *num_tiles = count;
  if (tiles == nullptr) return ok();  // size query: nothing is launched
  if (capacity < count)
    return fail(DC_ERR_SHAPE, "capacity=%lld < %lld tiles", (long long)capacity, (long long)count);
  if (num_tasks > 0 && tasks == nullptr) return fail(DC_ERR_NULL, "tasks is NULL");
  return hip_status(dc::launch_plan_flush_buffers(dtype, bucket_numel, tasks, num_tasks, tiles, count,
                                                  static_cast<hipStream_t>(stream)),
                    "device fused-flush planner launch");
}

dc_status dc_flush_bucket_buffers_planned(int32_t W, int32_t dtype, int64_t bucket_numel,
                                          const dc_task* tasks, int32_t num_tasks,
                                          const void* const* in_ptrs, void* const* out_ptrs,
                                          const dc_comm* comms, int32_t num_comms, int32_t pre_div,
                                          const dc_tile* tiles, int64_t num_tiles, void* stream) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_dtype(dtype)) || (st = check_comms(W, comms, num_comms))) return st;
  if (bucket_numel < 0 || num_tasks < 0)
    return fail(DC_ERR_ARG, "bucket_numel=%lld, num_tasks=%d", (long long)bucket_numel, num_tasks);
  if ((st = check_extent("bucket_numel", bucket_numel)) || (st = check_extent("num_tiles", num_tiles))) return st;
  if (num_tasks > 0 && (tasks == nullptr || in_ptrs == nullptr || out_ptrs == nullptr))
    return fail(DC_ERR_NULL, "tasks, in_ptrs or out_ptrs is NULL");
  if (pre_div != 0 && pre_div != 1) return fail(DC_ERR_ARG, "pre_div=%d", pre_div);
  const int64_t want = num_tasks > 0 ? dc::buffer_tiles(dtype, bucket_numel) : 0;
  if (num_tiles != want)
    return fail(DC_ERR_SHAPE, "num_tiles=%lld, the bucket has %lld tiles", (long long)num_tiles, (long long)want);
  if (want > 0 && tiles == nullptr) return fail(DC_ERR_NULL, "tiles is NULL");
  return hip_status(dc::launch_flush_buffers(W, dtype, bucket_numel, tasks, num_tasks, in_ptrs, out_ptrs,
                                             comms, num_comms, pre_div, static_cast<hipStream_t>(stream),
                                             tiles),
                    "planned buffer flush launch");
}

dc_status dc_validate_buffer_tasks(int32_t W, int32_t dtype, const dc_task* tasks, int32_t num_tasks,
                                   int64_t bucket_numel, const dc_comm* comms, int32_t num_comms,
                                   const void* const* in_ptrs, void* const* out_ptrs) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_dtype(dtype)) || (st = check_comms(W, comms, num_comms))) return st;
  if (num_tasks < 0 || bucket_numel < 0) return fail(DC_ERR_ARG, "num_tasks or bucket_numel < 0");
  if (num_tasks > 0 && (tasks == nullptr || in_ptrs == nullptr || out_ptrs == nullptr))
    return fail(DC_ERR_NULL, "tasks, in_ptrs or out_ptrs is NULL");
  int64_t pos = 0;
  for (int32_t t = 0; t < num_tasks; ++t) {
    const dc_task& k = tasks[t];
    if (k.numel < 0) return fail(DC_ERR_TASKS, "task %d: numel %lld < 0", t, (long long)k.numel);
    if (k.offset < pos) return fail(DC_ERR_TASKS, "task %d: offset %lld overlaps the previous task (ends at %lld)", t, (long long)k.offset, (long long)pos);
    if (k.offset + k.numel > bucket_numel) return fail(DC_ERR_TASKS, "task %d ends past bucket_numel=%lld", t, (long long)bucket_numel);
    if (k.comm < 0 || k.comm >= num_comms) return fail(DC_ERR_TASKS, "task %d: comm %d outside [0, %d)", t, k.comm, num_comms);
    pos = k.offset + k.numel;
  }
  // byte intervals; an input identical to its own output is the in-place pair
  struct Iv { uintptr_t a, b; int out; int32_t t, r; };
  std::vector<Iv> iv;
  const uintptr_t eb = (uintptr_t)elem_bytes(dtype);
  for (int32_t t = 0; t < num_tasks; ++t) {
    if (tasks[t].numel == 0) continue;
    const uintptr_t len = (uintptr_t)tasks[t].numel * eb;
    for (int32_t r = 0; r < W; ++r) {
      const uintptr_t in = reinterpret_cast<uintptr_t>(in_ptrs[(int64_t)t * W + r]);
      const uintptr_t out = reinterpret_cast<uintptr_t>(out_ptrs[(int64_t)t * W + r]);
      if (in == 0) return fail(DC_ERR_TASKS, "task %d rank %d: input pointer is NULL", t, r);
      if (out != 0) iv.push_back({out, out + len, 1, t, r});
      if (out != in) iv.push_back({in, in + len, 0, t, r});
    }
  }
  std::sort(iv.begin(), iv.end(), [](const Iv& x, const Iv& y) { return x.a < y.a || (x.a == y.a && x.out > y.out); });
  uintptr_t end_all = 0, end_out = 0;
  int32_t who_all = -1, who_out = -1, rank_all = -1, rank_out = -1;
  for (const Iv& x : iv) {
    if (x.out && x.a < end_all)
      return fail(DC_ERR_TASKS, "output of task %d rank %d overlaps a buffer of task %d rank %d", x.t, x.r, who_all, rank_all);
    if (!x.out && x.a < end_out)
      return fail(DC_ERR_TASKS, "input of task %d rank %d overlaps the output of task %d rank %d", x.t, x.r, who_out, rank_out);
    if (x.b > end_all) { end_all = x.b; who_all = x.t; rank_all = x.r; }
    if (x.out && x.b > end_out) { end_out = x.b; who_out = x.t; rank_out = x.r; }
  }
  return ok();
}

dc_status dc_probe_flush(int32_t W, int32_t dtype, const dc_task* tasks, int32_t num_tasks,
                         const int32_t* owner, int32_t num_params, const int32_t* pid_offsets,
                         const int32_t* pids, const dc_comm* comms, int32_t num_comms,
                         int32_t pre_div, dc_probe* out) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_dtype(dtype)) || (st = check_comms(W, comms, num_comms))) return st;
  if (out == nullptr) return fail(DC_ERR_NULL, "out is NULL");
  if (num_tasks < 0 || num_params < 0) return fail(DC_ERR_ARG, "num_tasks or num_params < 0");
  if (num_tasks > 0 && (tasks == nullptr || pid_offsets == nullptr))
    return fail(DC_ERR_NULL, "tasks or pid_offsets is NULL");
  std::memset(out, 0, sizeof *out);
  out->tasks = num_tasks;
  out->pre_div = pre_div;
  out->dtype = dtype;
  std::vector<char> wr(W), hd(W);
  for (int32_t t = 0; t < num_tasks; ++t) {
    const dc_task& k = tasks[t];
    if (k.param < 0 || k.param >= num_params || k.comm < 0 || k.comm >= num_comms || k.numel < 0)
      return fail(DC_ERR_TASKS, "task %d has an out-of-range param, comm or numel", t);
    int32_t root = (k.comm == 0 && owner != nullptr) ? owner[k.param] : -1;
    if (root >= W) root = -1;
    out->reduced_elems += k.numel;
    if (root >= 0) {
      out->owner_tasks += 1;
      out->owner_elems += k.numel;
    }
    std::fill(wr.begin(), wr.end(), 0);
    if (root >= 0) wr[root] = 1;
    else std::fill(wr.begin(), wr.end(), 1);
    if ((st = task_holders(W, k, t, pid_offsets, pids, comms, hd.data()))) return st;
    for (int r = 0; r < W; ++r) {
      if (wr[r]) out->written[r] += k.numel;
      if (hd[r]) out->kept[r] += k.numel;
    }
  }
  for (int r = 0; r < W; ++r) out->discarded[r] = out->written[r] - out->kept[r];
  return ok();
}

dc_status dc_holders(int32_t W, const dc_task* tasks, int32_t num_tasks, int32_t num_params,
                     const int32_t* pid_offsets, const int32_t* pids, const dc_comm* comms,
                     int32_t num_comms, uint8_t* holders) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_comms(W, comms, num_comms))) return st;
  if (num_tasks < 0 || num_params < 0) return fail(DC_ERR_ARG, "num_tasks or num_params < 0");
  if (num_tasks > 0 && (tasks == nullptr || pid_offsets == nullptr || holders == nullptr))
    return fail(DC_ERR_NULL, "tasks, pid_offsets or holders is NULL");
  std::vector<char> hd(W);
  for (int32_t t = 0; t < num_tasks; ++t) {
    const dc_task& k = tasks[t];
    if (k.param < 0 || k.param >= num_params || k.comm < 0 || k.comm >= num_comms)
      return fail(DC_ERR_TASKS, "task %d has an out-of-range param or comm", t);
    if ((st = task_holders(W, k, t, pid_offsets, pids, comms, hd.data()))) return st;
    for (int r = 0; r < W; ++r) holders[(int64_t)t * W + r] = (uint8_t)hd[r];
  }
  return ok();
}

dc_status dc_param_part_size(int32_t W, int32_t num_params, int32_t num_groups,
                             const int32_t* group_begin, const int32_t* group_comm_size,
                             const int32_t* group_rank_to_global, const int64_t* part_size,
                             int64_t* param_part_size, void* stream) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_groups(num_params, num_groups, group_begin))) return st;
  if (group_comm_size == nullptr || group_rank_to_global == nullptr || part_size == nullptr)
    return fail(DC_ERR_NULL, "group_comm_size, group_rank_to_global or part_size is NULL");
  if (num_params > 0 && param_part_size == nullptr) return fail(DC_ERR_NULL, "param_part_size is NULL");
  dc::GroupTable g{};
  g.num_groups = num_groups;
  for (int k = 0; k <= num_groups; ++k) g.begin[k] = group_begin[k];
  for (int k = 0; k < num_groups; ++k) {
    g.eligible[k] = dp_group(W, k, group_comm_size, group_rank_to_global);
    g.parts[k] = group_comm_size[k];
  }
  return hip_status(dc::launch_param_part_size(num_params, g, part_size, param_part_size,
                                               static_cast<hipStream_t>(stream)),
                    "param part size launch");
}

dc_status dc_plan_relayout(int32_t W, const dc_task* tasks, int32_t num_tasks,
                           const int64_t* flat_offset, const int64_t* part_size,
                           int32_t num_params, dc_piece* pieces, int32_t pieces_capacity,
                           int32_t* num_pieces, int64_t* seg_start) {
  dc_status st;
  if ((st = check_w(W))) return st;
  if (num_tasks < 0 || num_params < 0) return fail(DC_ERR_ARG, "num_tasks or num_params < 0");
  if (seg_start == nullptr || num_pieces == nullptr) return fail(DC_ERR_NULL, "seg_start or num_pieces is NULL");
  if (num_tasks > 0 && (tasks == nullptr || flat_offset == nullptr || part_size == nullptr))
    return fail(DC_ERR_NULL, "tasks, flat_offset or part_size is NULL");
  // pass 1: segment sizes and the piece count; pass 2: the pieces, each at
  // its segment's cursor
  std::vector<int64_t> count(W, 0), cur(W, 0);
  int64_t total = 0;
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      seg_start[0] = 0;
      for (int q = 0; q < W; ++q) seg_start[q + 1] = seg_start[q] + count[q];
      *num_pieces = (int32_t)total;
      if (pieces == nullptr) return ok();  // size query
      if (total > pieces_capacity)
        return fail(DC_ERR_SHAPE, "pieces_capacity=%d < %lld pieces", pieces_capacity, (long long)total);
      for (int q = 0; q < W; ++q) cur[q] = seg_start[q];
    }
    int64_t np = 0;
    for (int32_t t = 0; t < num_tasks; ++t) {
      const dc_task& k = tasks[t];
      if (k.param < 0 || k.param >= num_params || k.numel < 0)
        return fail(DC_ERR_TASKS, "task %d has an out-of-range param or numel", t);
      const int64_t S = k.comm == 0 ? part_size[k.param] : 0;
      if (S <= 0 || k.numel == 0) continue;
      const int64_t a = flat_offset[k.param];
      const int64_t q0 = a / S, q1 = (a + k.numel - 1) / S;
      if (a < 0 || q1 >= W)
        return fail(DC_ERR_TASKS, "task %d: partitions %lld..%lld outside [0, %d)", t, (long long)q0,
                    (long long)q1, W);
      for (int64_t q = q0; q <= q1; ++q) {
        const int64_t e0 = std::max<int64_t>(0, q * S - a);
        const int64_t e1 = std::min<int64_t>(k.numel, (q + 1) * S - a);
        if (pass == 0) {
          count[q] += e1 - e0;
        } else {
          pieces[np] = dc_piece{k.offset + e0, cur[q], e1 - e0, 0};
          cur[q] += e1 - e0;
        }
        ++np;
      }
    }
    if (pass == 0) {
      total = np;
      if (total > INT32_MAX) return fail(DC_ERR_SHAPE, "too many pieces");
    }
  }
  std::sort(pieces, pieces + total, [](const dc_piece& x, const dc_piece& y) { return x.dst < y.dst; });
  return ok();
}

// Checks and launch shared by the searched and the planned relayout
// (tiles == nullptr: searched).
static dc_status relayout_common(int32_t W, int32_t dtype, const void* slab_in, int64_t ld_in, void* out,
                                 int64_t ld_out, int64_t bucket_col, int64_t bucket_numel,
                                 const dc_piece* pieces, int32_t num_pieces, int64_t out_numel,
                                 const int64_t* tiles, void* stream) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_dtype(dtype))) return st;
  if (bucket_col < 0 || bucket_numel < 0 || out_numel < 0 || num_pieces < 0)
    return fail(DC_ERR_ARG, "negative bucket_col, bucket_numel, out_numel or num_pieces");
  if ((st = check_extent("bucket_col", bucket_col)) || (st = check_extent("bucket_numel", bucket_numel)))
    return st;
  if ((st = check_slab("slab_in", slab_in, ld_in, bucket_col + bucket_numel, dtype)) ||
      (st = check_slab("out", out, ld_out, out_numel, dtype)))
    return st;
  if (num_pieces > 0 && pieces == nullptr) return fail(DC_ERR_NULL, "pieces is NULL");
  const int64_t b = elem_bytes(dtype);
  if (overlaps(slab_in, W * ld_in * b, out, W * ld_out * b)) return fail(DC_ERR_ARG, "slab_in and out overlap");
  return hip_status(dc::launch_relayout(W, dtype, slab_in, ld_in, out, ld_out, bucket_col, bucket_numel,
                                        pieces, num_pieces, out_numel, tiles,
                                        static_cast<hipStream_t>(stream)),
                    tiles != nullptr ? "planned relayout launch" : "relayout launch");
}

dc_status dc_relayout_bucket(int32_t W, int32_t dtype, const void* slab_in, int64_t ld_in,
                             void* out, int64_t ld_out, int64_t bucket_col, int64_t bucket_numel,
                             const dc_piece* pieces, int32_t num_pieces, int64_t out_numel,
                             void* stream) {
  return relayout_common(W, dtype, slab_in, ld_in, out, ld_out, bucket_col, bucket_numel, pieces,
                         num_pieces, out_numel, nullptr, stream);
}

dc_status dc_plan_relayout_tiles(int32_t dtype, int64_t bucket_col, int64_t bucket_numel,
                                 const dc_piece* pieces, int32_t num_pieces, int64_t out_numel,
                                 int64_t* tiles, int64_t tiles_capacity, int64_t* num_tiles) {
  dc_status st;
  if ((st = check_dtype(dtype))) return st;
  if (bucket_col < 0 || bucket_numel < 0 || out_numel < 0 || num_pieces < 0)
    return fail(DC_ERR_ARG, "negative bucket_col, bucket_numel, out_numel or num_pieces");
  if ((st = check_extent("bucket_col", bucket_col)) || (st = check_extent("bucket_numel", bucket_numel)) ||
      (st = check_extent("out_numel", out_numel)))
    return st;
  if (num_tiles == nullptr) return fail(DC_ERR_NULL, "num_tiles is NULL");
  if (num_pieces > 0 && pieces == nullptr) return fail(DC_ERR_NULL, "pieces is NULL");
  for (int32_t k = 0; k < num_pieces; ++k) {
    if (pieces[k].len < 0) return fail(DC_ERR_ARG, "piece %d has a negative length", k);
    if (k > 0 && pieces[k].dst < pieces[k - 1].dst) return fail(DC_ERR_ARG, "pieces not sorted by dst at %d", k);
  }
  const int64_t n = dc::relayout_tile_count(dtype, out_numel);
  *num_tiles = n;
  if (tiles == nullptr) return ok();  // size query
  if (tiles_capacity < n)
    return fail(DC_ERR_SHAPE, "tiles_capacity=%lld < %lld tiles", (long long)tiles_capacity, (long long)n);
  // one sweep over the tiles in destination order beside the pieces.  A
  // destination column belongs to the last piece starting at or before it
  // (as in the searched relayout); a tile copies straight from piece k when
  // all its columns belong to k -- k covers the tile and no later piece
  // starts inside it -- and its source run starts on a vector and stays in
  // the bucket
  const int64_t E = 16 / elem_bytes(dtype), span = dc::kRelayoutTile * E;
  int32_t k = 0;
  for (int64_t t = 0; t < n; ++t) {
    const int64_t d0 = t * span, d1 = d0 + span;
    while (k + 1 < num_pieces && pieces[k + 1].dst <= d0) ++k;
    int64_t rec = -1;
    if (num_pieces > 0 && d1 <= out_numel && pieces[k].dst <= d0 && d1 <= pieces[k].dst + pieces[k].len &&
        (k + 1 == num_pieces || pieces[k + 1].dst >= d1)) {
      const int64_t src0 = pieces[k].src + (d0 - pieces[k].dst);
      if (src0 >= 0 && src0 + span <= bucket_numel && (bucket_col + src0) % E == 0) rec = (bucket_col + src0) / E;
    }
    tiles[dc::tile_slot(t, n)] = rec;
  }
  return ok();
}

dc_status dc_plan_relayout_tiles_device(int32_t dtype, int64_t bucket_col, int64_t bucket_numel,
                                        const dc_piece* pieces, int32_t num_pieces,
                                        int64_t out_numel, int64_t* tiles, int64_t tiles_capacity,
                                        int64_t* num_tiles, void* stream) {
  dc_status st;
  if ((st = check_dtype(dtype))) return st;
  if (bucket_col < 0 || bucket_numel < 0 || out_numel < 0 || num_pieces < 0)
    return fail(DC_ERR_ARG, "negative bucket_col, bucket_numel, out_numel or num_pieces");
  if ((st = check_extent("bucket_col", bucket_col)) || (st = check_extent("bucket_numel", bucket_numel)) ||
      (st = check_extent("out_numel", out_numel)))
    return st;
  if (num_tiles == nullptr) return fail(DC_ERR_NULL, "num_tiles is NULL");
  const int64_t n = dc::relayout_tile_count(dtype, out_numel);
  *num_tiles = n;
  if (tiles == nullptr) return ok();  // size query: nothing is launched
  if (tiles_capacity < n)
    return fail(DC_ERR_SHAPE, "tiles_capacity=%lld < %lld tiles", (long long)tiles_capacity, (long long)n);
  if (num_pieces > 0 && pieces == nullptr) return fail(DC_ERR_NULL, "pieces is NULL");
  return hip_status(dc::launch_plan_relayout_tiles(dtype, bucket_col, bucket_numel, pieces, num_pieces,
                                                   out_numel, tiles, n, static_cast<hipStream_t>(stream)),
                    "device relayout planner launch");
}

dc_status dc_relayout_bucket_planned(int32_t W, int32_t dtype, const void* slab_in, int64_t ld_in,
                                     void* out, int64_t ld_out, int64_t bucket_col, int64_t bucket_numel,
                                     const dc_piece* pieces, int32_t num_pieces, int64_t out_numel,
                                     const int64_t* tiles, int64_t num_tiles, void* stream) {
  dc_status st;
  if ((st = check_dtype(dtype))) return st;
  if (out_numel > 0 && num_pieces > 0) {
    const int64_t n = dc::relayout_tile_count(dtype, out_numel);
    if (num_tiles != n)
      return fail(DC_ERR_SHAPE, "num_tiles=%lld, the plan of out_numel=%lld has %lld", (long long)num_tiles,
                  (long long)out_numel, (long long)n);
    if (tiles == nullptr) return fail(DC_ERR_NULL, "tiles is NULL");
  }
  return relayout_common(W, dtype, slab_in, ld_in, out, ld_out, bucket_col, bucket_numel, pieces,
                         num_pieces, out_numel, tiles, stream);
}

dc_status dc_reduce_scatter_v(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                              int64_t ld_out, const int64_t* seg_start, int32_t pre_div,
                              void* stream) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_dtype(dtype))) return st;
  if (seg_start == nullptr) return fail(DC_ERR_NULL, "seg_start is NULL");
  if (pre_div != 0 && pre_div != 1) return fail(DC_ERR_ARG, "pre_div=%d", pre_div);
  if (seg_start[0] != 0) return fail(DC_ERR_SHAPE, "seg_start[0] must be 0");
  int64_t maxlen = 0;
  for (int q = 0; q < W; ++q) {
    if (seg_start[q + 1] < seg_start[q]) return fail(DC_ERR_SHAPE, "seg_start decreases at %d", q);
    maxlen = std::max<int64_t>(maxlen, seg_start[q + 1] - seg_start[q]);
  }
  if ((st = check_slab("in", in, ld_in, seg_start[W], dtype)) || (st = check_slab("out", out, ld_out, maxlen, dtype)))
    return st;
  const int64_t b = elem_bytes(dtype);
  if (overlaps(in, W * ld_in * b, out, W * ld_out * b)) return fail(DC_ERR_ARG, "in and out overlap");
  return hip_status(dc::launch_reduce_scatter_v(W, dtype, in, ld_in, out, ld_out, seg_start, pre_div,
                                                static_cast<hipStream_t>(stream)),
                    "reduce-scatter-v launch");
}

dc_status dc_reduce_scatter(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                            int64_t ld_out, int64_t M, int32_t pre_div, void* stream) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_dtype(dtype))) return st;
  if (M < 0) return fail(DC_ERR_ARG, "M=%lld < 0", (long long)M);
  if (M % W != 0) return fail(DC_ERR_SHAPE, "M=%lld is not a multiple of W=%d (pad with zeros)", (long long)M, W);
  if (pre_div != 0 && pre_div != 1) return fail(DC_ERR_ARG, "pre_div=%d", pre_div);
  if ((st = check_slab("in", in, ld_in, M, dtype)) || (st = check_slab("out", out, ld_out, M / W, dtype))) return st;
  const int64_t b = elem_bytes(dtype);
  if (overlaps(in, W * ld_in * b, out, W * ld_out * b)) return fail(DC_ERR_ARG, "in and out overlap");
  return hip_status(dc::launch_reduce_scatter(W, dtype, in, ld_in, out, ld_out, M, pre_div,
                                              static_cast<hipStream_t>(stream)),
                    "reduce-scatter launch");
}

dc_status dc_all_gather(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                        int64_t ld_out, int64_t shard_numel, int32_t order, int32_t step,
                        void* stream) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_dtype(dtype))) return st;
  if (shard_numel < 0) return fail(DC_ERR_ARG, "shard_numel < 0");
  if ((st = check_extent("shard_numel", shard_numel))) return st;
  if (order != DC_ORDER_RANK && order != DC_ORDER_RING) return fail(DC_ERR_ARG, "order=%d", order);
  if (step < -1 || step >= W) return fail(DC_ERR_ARG, "step=%d outside [-1, W)", step);
  if ((st = check_slab("in", in, ld_in, shard_numel, dtype)) ||
      (st = check_slab("out", out, ld_out, W * shard_numel, dtype)))
    return st;
  const int64_t b = elem_bytes(dtype);
  if (overlaps(in, W * ld_in * b, out, W * ld_out * b)) return fail(DC_ERR_ARG, "in and out overlap");
  return hip_status(dc::launch_all_gather(W, dtype, in, ld_in, out, ld_out, shard_numel, order, step,
                                          static_cast<hipStream_t>(stream)),
                    "all-gather launch");
}

dc_status dc_reduce_scatter_ring(int32_t W, int32_t dtype, const void* in, int64_t ld_in,
                                 void* out, int64_t ld_out, int64_t M, int32_t pre_div,
                                 void* stream) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_dtype(dtype))) return st;
  if (M < 0) return fail(DC_ERR_ARG, "M=%lld < 0", (long long)M);
  if (M % W != 0) return fail(DC_ERR_SHAPE, "M=%lld is not a multiple of W=%d (pad with zeros)", (long long)M, W);
  if (pre_div != 0 && pre_div != 1) return fail(DC_ERR_ARG, "pre_div=%d", pre_div);
  if ((st = check_slab("in", in, ld_in, M, dtype)) || (st = check_slab("out", out, ld_out, M / W, dtype))) return st;
  const int64_t b = elem_bytes(dtype);
  if (overlaps(in, W * ld_in * b, out, W * ld_out * b)) return fail(DC_ERR_ARG, "in and out overlap");
  return hip_status(dc::launch_reduce_scatter_ring(W, dtype, in, ld_in, out, ld_out, M, pre_div,
                                                   static_cast<hipStream_t>(stream)),
                    "ring reduce-scatter launch");
}

dc_status dc_all_gather_step(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                             int64_t ld_out, int64_t shard_numel, int32_t algo, int32_t step,
                             void* stream) {
  dc_status st;
  if ((st = check_w(W)) || (st = check_dtype(dtype))) return st;
  if (shard_numel < 0) return fail(DC_ERR_ARG, "shard_numel < 0");
  if ((st = check_extent("shard_numel", shard_numel))) return st;
  int32_t steps;
  if (algo == DC_SCHED_RING) {
    steps = W - 1;
  } else if (algo == DC_SCHED_BIDIR) {
    steps = W / 2;  // ceil((W-1)/2)
  } else if (algo == DC_SCHED_RD) {
    if ((W & (W - 1)) != 0) return fail(DC_ERR_ARG, "recursive doubling needs W a power of two, got %d", W);
    steps = 0;
    for (int d = 1; d < W; d <<= 1) ++steps;
  } else {
    return fail(DC_ERR_ARG, "algo=%d", algo);
  }
  if (step < 0 || step > steps) return fail(DC_ERR_ARG, "step=%d outside [0, %d]", step, steps);
  if ((st = check_slab("in", in, ld_in, shard_numel, dtype)) ||
      (st = check_slab("out", out, ld_out, W * shard_numel, dtype)))
    return st;
  const int64_t b = elem_bytes(dtype);
  if (overlaps(in, W * ld_in * b, out, W * ld_out * b)) return fail(DC_ERR_ARG, "in and out overlap");
  return hip_status(dc::launch_all_gather_step(W, dtype, in, ld_in, out, ld_out, shard_numel, algo, step,
                                               static_cast<hipStream_t>(stream)),
                    "all-gather step launch");
}

dc_status dc_accumulate(int32_t rows, const float* x, int64_t ld_x, float* acc, int64_t ld_acc,
                        int64_t M, int32_t init, void* stream) {
  dc_status st;
  if (rows < 1 || rows > 65535) return fail(DC_ERR_ARG, "rows=%d outside [1, 65535]", rows);
  if (M < 0) return fail(DC_ERR_ARG, "M < 0");
  if (init != 0 && init != 1) return fail(DC_ERR_ARG, "init=%d", init);
  if ((st = check_slab("x", x, ld_x, M, DC_F32)) || (st = check_slab("acc", acc, ld_acc, M, DC_F32))) return st;
  if (static_cast<const void*>(x) == static_cast<const void*>(acc)) {
    if (ld_x != ld_acc) return fail(DC_ERR_ARG, "x == acc needs ld_x == ld_acc");
  } else if (overlaps(x, rows * ld_x * 4, acc, rows * ld_acc * 4)) {
    return fail(DC_ERR_ARG, "x and acc overlap");
  }
  return hip_status(dc::launch_accumulate(rows, x, ld_x, acc, ld_acc, M, init,
                                          static_cast<hipStream_t>(stream)),
                    "accumulate launch");
}

dc_status dc_deferred_reduce(int32_t W, const float* acc, int64_t ld_acc, float* out,
                             int64_t ld_out, int64_t M, int32_t out_rows, void* stream) {
  dc_status st;
  if ((st = check_w(W))) return st;
  if (out_rows != 1 && out_rows != W) return fail(DC_ERR_ARG, "out_rows=%d is neither 1 nor W", out_rows);
  if (M < 0) return fail(DC_ERR_ARG, "M < 0");
  if ((st = check_slab("acc", acc, ld_acc, M, DC_F32)) || (st = check_slab("out", out, ld_out, M, DC_F32))) return st;
  if (static_cast<const void*>(acc) == static_cast<const void*>(out)) {
    if (ld_acc != ld_out) return fail(DC_ERR_ARG, "acc == out needs ld_acc == ld_out");
  } else if (overlaps(acc, W * ld_acc * 4, out, out_rows * ld_out * 4)) {
    return fail(DC_ERR_ARG, "acc and out overlap");
  }
  return hip_status(dc::launch_deferred_reduce(W, acc, ld_acc, out, ld_out, M, out_rows,
                                               static_cast<hipStream_t>(stream)),
                    "deferred reduce launch");
}

dc_status dc_accumulate_reduce(int32_t W, const float* x, int64_t ld_x, float* acc, int64_t ld_acc,
                               int32_t init, int32_t keep_acc, float* out, int64_t ld_out,
                               int32_t out_rows, int64_t M, void* stream) {
  dc_status st;
  if ((st = check_w(W))) return st;
  if (out_rows != 1 && out_rows != W) return fail(DC_ERR_ARG, "out_rows=%d is neither 1 nor W", out_rows);
  if (M < 0) return fail(DC_ERR_ARG, "M < 0");
  if ((init != 0 && init != 1) || (keep_acc != 0 && keep_acc != 1))
    return fail(DC_ERR_ARG, "init=%d keep_acc=%d", init, keep_acc);
  if ((st = check_slab("x", x, ld_x, M, DC_F32)) || (st = check_slab("acc", acc, ld_acc, M, DC_F32)) ||
      (st = check_slab("out", out, ld_out, M, DC_F32)))
    return st;
  const void *xv = x, *av = acc, *ov = out;
  if (xv == av) {
    if (ld_x != ld_acc) return fail(DC_ERR_ARG, "x == acc needs ld_x == ld_acc");
  } else if (overlaps(x, W * ld_x * 4, acc, W * ld_acc * 4)) {
    return fail(DC_ERR_ARG, "x and acc overlap");
  }
  if (overlaps(x, W * ld_x * 4, out, out_rows * ld_out * 4)) return fail(DC_ERR_ARG, "x and out overlap");
  if (av == ov) {
    if (ld_acc != ld_out || keep_acc) return fail(DC_ERR_ARG, "out == acc needs ld_out == ld_acc and keep_acc = 0");
  } else if (overlaps(acc, W * ld_acc * 4, out, out_rows * ld_out * 4)) {
    return fail(DC_ERR_ARG, "acc and out overlap");
  }
  return hip_status(dc::launch_accumulate_reduce(W, x, ld_x, acc, ld_acc, init, keep_acc, out, ld_out,
                                                 out_rows, M, static_cast<hipStream_t>(stream)),
                    "accumulate-reduce launch");
}

dc_status dc_round_bf16(const float* in, uint16_t* out, int64_t n, void* stream) {
  if (n < 0) return fail(DC_ERR_ARG, "n < 0");
  if (n > 0 && (in == nullptr || out == nullptr)) return fail(DC_ERR_NULL, "in or out is NULL");
  return hip_status(dc::launch_round_bf16(in, out, n, static_cast<hipStream_t>(stream)), "round launch");
}

dc_status dc_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return fail(DC_ERR_SHAPE, "bytes=%lld is not a multiple of 16", (long long)bytes);
  if (check_extent("bytes", bytes)) return DC_ERR_SHAPE;
  if (bytes > 0 && (src == nullptr || dst == nullptr)) return fail(DC_ERR_NULL, "src or dst is NULL");
  if (!aligned16(src) || !aligned16(dst)) return fail(DC_ERR_ALIGN, "src or dst not 16-byte aligned");
  if (overlaps(src, bytes, dst, bytes)) return fail(DC_ERR_ARG, "src and dst overlap");
  return hip_status(dc::launch_stream_copy(src, dst, bytes, static_cast<hipStream_t>(stream)), "copy launch");
}

dc_status dc_stream_rows(const void* src, int64_t src_ld_vec, int32_t rows_read, void* dst,
                         int64_t dst_ld_vec, int32_t rows_written, int64_t nvec, void* stream) {
  if (!((rows_read == 4 || rows_read == 8 || rows_read == 16) &&
        (rows_written == 1 || rows_written == rows_read)))
    return fail(DC_ERR_UNSUPPORTED, "rows_read=%d rows_written=%d (need 4/8/16 and 1 or rows_read)",
                rows_read, rows_written);
  if (check_extent("src_ld_vec", src_ld_vec) || check_extent("dst_ld_vec", dst_ld_vec)) return DC_ERR_SHAPE;
  if (nvec < 0 || src_ld_vec < nvec || dst_ld_vec < nvec)
    return fail(DC_ERR_SHAPE, "nvec=%lld with row strides %lld and %lld vectors", (long long)nvec,
                (long long)src_ld_vec, (long long)dst_ld_vec);
  if (nvec > 0 && (src == nullptr || dst == nullptr)) return fail(DC_ERR_NULL, "src or dst is NULL");
  if (!aligned16(src) || !aligned16(dst)) return fail(DC_ERR_ALIGN, "src or dst not 16-byte aligned");
  if (overlaps(src, rows_read * src_ld_vec * 16, dst, rows_written * dst_ld_vec * 16))
    return fail(DC_ERR_ARG, "src and dst overlap");
  return hip_status(dc::launch_stream_rows(src, src_ld_vec, rows_read, dst, dst_ld_vec, rows_written,
                                           nvec, static_cast<hipStream_t>(stream)),
                    "stream rows launch");
}

dc_status dc_stream_rows_shaped(const void* src, int64_t src_ld_vec, int32_t rows_read, void* dst,
                                int64_t dst_ld_vec, int32_t rows_written, int64_t nvec,
                                int32_t group, int32_t cap, void* stream) {
  if (group != 1 && group != 2 && group != 4) return fail(DC_ERR_UNSUPPORTED, "group=%d (1, 2 or 4)", group);
  if (cap < 0 || cap > 64) return fail(DC_ERR_ARG, "cap=%d outside [0, 64]", cap);
  const bool wide = rows_written == 4 || rows_written == 8 || rows_written == 16;
  if (!(((rows_read == 4 || rows_read == 8 || rows_read == 16) &&
         (rows_written == 1 || rows_written == rows_read)) ||
        (rows_read == 1 && wide) || (rows_read == 8 && rows_written == 4)))
    return fail(DC_ERR_UNSUPPORTED,
                "rows_read=%d rows_written=%d (need 4/8/16 and 1 or rows_read, 1 and 4/8/16, or 8 and 4)",
                rows_read, rows_written);
  if (check_extent("src_ld_vec", src_ld_vec) || check_extent("dst_ld_vec", dst_ld_vec)) return DC_ERR_SHAPE;
  if (nvec < 0 || src_ld_vec < nvec || dst_ld_vec < nvec)
    return fail(DC_ERR_SHAPE, "nvec=%lld with row strides %lld and %lld vectors", (long long)nvec,
                (long long)src_ld_vec, (long long)dst_ld_vec);
  if (nvec > 0 && (src == nullptr || dst == nullptr)) return fail(DC_ERR_NULL, "src or dst is NULL");
  if (!aligned16(src) || !aligned16(dst)) return fail(DC_ERR_ALIGN, "src or dst not 16-byte aligned");
  if (overlaps(src, rows_read * src_ld_vec * 16, dst, rows_written * dst_ld_vec * 16))
    return fail(DC_ERR_ARG, "src and dst overlap");
  return hip_status(dc::launch_stream_rows_shaped(src, src_ld_vec, rows_read, dst, dst_ld_vec,
                                                  rows_written, nvec, group, cap,
                                                  static_cast<hipStream_t>(stream)),
                    "shaped stream rows launch");
}

}  // extern "C"
