/* A plain C11 client of libdc.so, used by the GPU tests: device memory from
 * hipMalloc, the owner map built on the device, one bucket flush (searched,
 * and again from a host-made and a device-made plan) and one reduce-scatter
 * through the C ABI, results copied back.  No Python and no torch in this
 * file: it shows that the ABI needs nothing but the HIP runtime.
 *
 * One data-parallel parameter group over W ranks; the bucket holds every
 * parameter in order (task t = parameter t on communicator 0).
 *
 *   slab_in   host [W, ld] elements of dtype (bf16 as uint16)
 *   numel     host int64[P] parameter sizes; their sum is the bucket's size
 *   owner_out host int32[P]: the owner map the device built
 *   flush_out host [W, ld]: the flushed slab (rows the flush does not write
 *             keep the input)
 *   rs_out    host [W, ld_rs] or NULL: reduce-scatter of the input slab's first
 *             M = W * ld_rs columns (when M fits the bucket)
 *   planned_out host [W, ld] or NULL: the same flush from a plan made on the
 *             host with dc_plan_flush (the owner map copied back first); the
 *             plan is also built on the device with dc_plan_flush_device and
 *             the flush run again from it
 * Returns 0, a DC_ERR_* code from the library, 100 + a HIP error code, or 200
 * when the device-built plan, its root count or its flush differs from the
 * host plan's. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "dc.h"

#define HIP_TRY(x)                      \
  do {                                  \
    hipError_t e_ = (x);                \
    if (e_ != hipSuccess) {             \
      rc = 100 + (int)e_;               \
      goto done;                        \
    }                                   \
  } while (0)
#define DC_TRY(x)        \
  do {                   \
    dc_status s_ = (x);  \
    if (s_ != DC_OK) {   \
      rc = (int)s_;      \
      goto done;         \
    }                    \
  } while (0)

int c_client_run(int32_t W, int32_t dtype, const void* slab_in, int64_t ld, int32_t P,
                 const int64_t* numel, int32_t reduce_to_owner, int32_t pre_div,
                 int32_t* owner_out, void* flush_out, int64_t ld_rs, void* rs_out,
                 void* planned_out) {
  int rc = 0;
  const size_t eb = dtype == DC_BF16 ? 2 : 4;
  const size_t slab_bytes = (size_t)W * (size_t)ld * eb;
  int64_t total = 0;
  for (int32_t i = 0; i < P; ++i) total += numel[i];
  const int64_t pids_cap = (int64_t)P + W - 1;
  const int32_t group_begin[2] = {0, P};
  const int32_t group_parts[1] = {W};
  const int32_t group_comm_size[1] = {W};
  int32_t* rank_to_global = (int32_t*)malloc(sizeof(int32_t) * (size_t)W);
  dc_task* tasks = (dc_task*)calloc((size_t)(P > 0 ? P : 1), sizeof(dc_task));
  const dc_comm comms[1] = {{W, 1}};
  void *d_in = NULL, *d_out = NULL, *d_rs = NULL, *d_out2 = NULL;
  dc_tile *tiles = NULL, *tiles2 = NULL;
  dc_tile *d_tiles = NULL, *d_tiles2 = NULL;
  int64_t* d_roots = NULL;
  void* planned2 = NULL;
  int64_t *d_numel = NULL, *d_flat = NULL, *d_psize = NULL;
  int32_t *d_pid_off = NULL, *d_pids = NULL, *d_owner = NULL, *d_counts = NULL;
  dc_task* d_tasks = NULL;
  hipStream_t stream = NULL;
  if (rank_to_global == NULL || tasks == NULL) {
    rc = DC_ERR_ARG;
    goto done;
  }
  for (int32_t i = 0; i < W; ++i) rank_to_global[i] = i;
  {
    int64_t off = 0;
    for (int32_t t = 0; t < P; ++t) {
      tasks[t].offset = off;
      tasks[t].numel = numel[t];
      tasks[t].param = t;
      tasks[t].comm = 0;
      tasks[t].reserved = 0;
      off += numel[t];
    }
  }
  DC_TRY(dc_validate_tasks(W, tasks, P, total, P, comms, 1));

  HIP_TRY(hipStreamCreate(&stream));
  HIP_TRY(hipMalloc(&d_in, slab_bytes));
  HIP_TRY(hipMalloc(&d_out, slab_bytes));
  HIP_TRY(hipMalloc((void**)&d_numel, sizeof(int64_t) * (size_t)(P > 0 ? P : 1)));
  HIP_TRY(hipMalloc((void**)&d_flat, sizeof(int64_t) * (size_t)(P > 0 ? P : 1)));
  HIP_TRY(hipMalloc((void**)&d_psize, sizeof(int64_t)));
  HIP_TRY(hipMalloc((void**)&d_pid_off, sizeof(int32_t) * (size_t)(P + 1)));
  HIP_TRY(hipMalloc((void**)&d_pids, sizeof(int32_t) * (size_t)pids_cap));
  HIP_TRY(hipMalloc((void**)&d_owner, sizeof(int32_t) * (size_t)(P > 0 ? P : 1)));
  HIP_TRY(hipMalloc((void**)&d_counts, sizeof(int32_t) * 2));
  HIP_TRY(hipMalloc((void**)&d_tasks, sizeof(dc_task) * (size_t)(P > 0 ? P : 1)));
  HIP_TRY(hipMemcpyAsync(d_in, slab_in, slab_bytes, hipMemcpyHostToDevice, stream));
  HIP_TRY(hipMemcpyAsync(d_out, slab_in, slab_bytes, hipMemcpyHostToDevice, stream));
  HIP_TRY(hipMemcpyAsync(d_numel, numel, sizeof(int64_t) * (size_t)P, hipMemcpyHostToDevice,
                         stream));
  HIP_TRY(hipMemcpyAsync(d_tasks, tasks, sizeof(dc_task) * (size_t)P, hipMemcpyHostToDevice,
                         stream));

  DC_TRY(dc_partition_ids(W, P, d_numel, 1, group_begin, group_parts, d_flat, d_psize, d_pid_off,
                          d_pids, pids_cap, stream));
  DC_TRY(dc_build_owner_map(W, P, d_pid_off, d_pids, pids_cap, 1, group_begin, group_comm_size,
                            rank_to_global, d_owner, d_counts, stream));
  DC_TRY(dc_flush_bucket(W, dtype, d_in, ld, d_out, ld, 0, total, d_tasks, P,
                         reduce_to_owner ? d_owner : NULL, P, comms, 1, pre_div, stream));
  if (rs_out != NULL) {
    HIP_TRY(hipMalloc(&d_rs, (size_t)W * (size_t)ld_rs * eb));
    DC_TRY(dc_reduce_scatter(W, dtype, d_in, ld, d_rs, ld_rs, (int64_t)W * ld_rs, pre_div,
                             stream));
    HIP_TRY(hipMemcpyAsync(rs_out, d_rs, (size_t)W * (size_t)ld_rs * eb, hipMemcpyDeviceToHost,
                           stream));
  }
  HIP_TRY(hipMemcpyAsync(owner_out, d_owner, sizeof(int32_t) * (size_t)P, hipMemcpyDeviceToHost,
                         stream));
  HIP_TRY(hipMemcpyAsync(flush_out, d_out, slab_bytes, hipMemcpyDeviceToHost, stream));
  HIP_TRY(hipStreamSynchronize(stream));
  if (planned_out != NULL) {
    /* plan on the host from the owner map just copied back, then flush again */
    int64_t ntiles = 0, roots = 0;
    const int32_t* own = reduce_to_owner ? owner_out : NULL;
    DC_TRY(dc_plan_flush(W, dtype, 0, total, tasks, P, own, NULL, NULL, P, comms, 1, NULL, 0, &ntiles,
                         NULL));
    tiles = (dc_tile*)calloc((size_t)(ntiles > 0 ? ntiles : 1), sizeof(dc_tile));
    if (tiles == NULL) {
      rc = DC_ERR_ARG;
      goto done;
    }
    DC_TRY(dc_plan_flush(W, dtype, 0, total, tasks, P, own, NULL, NULL, P, comms, 1, tiles, ntiles,
                         &ntiles, &roots));
    HIP_TRY(hipMalloc(&d_out2, slab_bytes));
    HIP_TRY(hipMalloc((void**)&d_tiles, sizeof(dc_tile) * (size_t)(ntiles > 0 ? ntiles : 1)));
    HIP_TRY(hipMemcpyAsync(d_out2, slab_in, slab_bytes, hipMemcpyHostToDevice, stream));
    HIP_TRY(hipMemcpyAsync(d_tiles, tiles, sizeof(dc_tile) * (size_t)ntiles, hipMemcpyHostToDevice,
                           stream));
    DC_TRY(dc_flush_bucket_planned(W, dtype, d_in, ld, d_out2, ld, 0, total, d_tasks, P,
                                   reduce_to_owner ? d_owner : NULL, NULL, NULL, P, comms, 1, pre_div,
                                   d_tiles, ntiles, roots, stream));
    HIP_TRY(hipMemcpyAsync(planned_out, d_out2, slab_bytes, hipMemcpyDeviceToHost, stream));
    HIP_TRY(hipStreamSynchronize(stream));
    /* the same plan built on the device from the device task table and owner
       map, and the flush again from it: the records and the output must be
       the host plan's, byte for byte (else 200) */
    {
      int64_t ntiles_dev = 0, roots_host = 0;
      HIP_TRY(hipMalloc((void**)&d_tiles2, sizeof(dc_tile) * (size_t)(ntiles > 0 ? ntiles : 1)));
      HIP_TRY(hipMalloc((void**)&d_roots, sizeof(int64_t)));
      DC_TRY(dc_plan_flush_device(W, dtype, 0, total, d_tasks, P, reduce_to_owner ? d_owner : NULL,
                                  NULL, NULL, P, comms, 1, d_tiles2, ntiles, &ntiles_dev, d_roots,
                                  stream));
      tiles2 = (dc_tile*)calloc((size_t)(ntiles > 0 ? ntiles : 1), sizeof(dc_tile));
      planned2 = malloc(slab_bytes);
      if (tiles2 == NULL || planned2 == NULL) {
        rc = DC_ERR_ARG;
        goto done;
      }
      HIP_TRY(hipMemcpyAsync(tiles2, d_tiles2, sizeof(dc_tile) * (size_t)ntiles, hipMemcpyDeviceToHost,
                             stream));
      HIP_TRY(hipMemcpyAsync(&roots_host, d_roots, sizeof(int64_t), hipMemcpyDeviceToHost, stream));
      HIP_TRY(hipMemcpyAsync(d_out2, slab_in, slab_bytes, hipMemcpyHostToDevice, stream));
      DC_TRY(dc_flush_bucket_planned(W, dtype, d_in, ld, d_out2, ld, 0, total, d_tasks, P,
                                     reduce_to_owner ? d_owner : NULL, NULL, NULL, P, comms, 1, pre_div,
                                     d_tiles2, ntiles, roots, stream));
      HIP_TRY(hipMemcpyAsync(planned2, d_out2, slab_bytes, hipMemcpyDeviceToHost, stream));
      HIP_TRY(hipStreamSynchronize(stream));
      if (ntiles_dev != ntiles || roots_host != roots ||
          memcmp(tiles2, tiles, sizeof(dc_tile) * (size_t)ntiles) != 0 ||
          memcmp(planned2, planned_out, slab_bytes) != 0)
        rc = 200;
    }
  }

done:
  if (stream != NULL) hipStreamSynchronize(stream);
  hipFree(d_in);
  hipFree(d_out);
  hipFree(d_rs);
  hipFree(d_numel);
  hipFree(d_flat);
  hipFree(d_psize);
  hipFree(d_pid_off);
  hipFree(d_pids);
  hipFree(d_owner);
  hipFree(d_counts);
  hipFree(d_tasks);
  hipFree(d_out2);
  hipFree(d_tiles);
  hipFree(d_tiles2);
  hipFree(d_roots);
  if (stream != NULL) hipStreamDestroy(stream);
  free(tiles);
  free(tiles2);
  free(planned2);
  free(rank_to_global);
  free(tasks);
  return rc;
}
