/*
 * dc.h - C ABI of libdc.so, a data-parallel gradient-reduction path for one
 * MI355X (gfx950) GPU.
 *
 * W simulated data-parallel ranks are the rows of a [W, ld] gradient slab in
 * device memory (row r = rank r's gradient; row-major; `ld` = row stride in
 * elements).  Every device entry point enqueues work on the given HIP stream
 * and returns at once; its results are valid once that stream reaches them.
 *
 * Pages cited (by title and section):
 *   [DS] DeepSpeed issue "[REQUEST] DeepCompile ZeRO-1: reduce-to-owner
 *        instead of AllReduce"
 *   [MT] MaxText PR "Defer the data-parallel gradient all-reduce to update()
 *        under gradient accumulation"
 *   [AG] "AllGather" (collective-communication notes)
 *
 * Typical use:
 *   once per layout   dc_partition_ids, then dc_build_owner_map (device
 *                     tables); per bucket, dc_validate_tasks on the host
 *                     copy of its task table and a plan (dc_plan_flush on
 *                     the host, or dc_plan_flush_device)
 *   every step        per bucket, as its gradients are complete,
 *                     dc_flush_bucket_planned (dc_flush_bucket without a
 *                     plan; dc_flush_bucket_buffers[_planned] to read each
 *                     rank's own gradient buffers and write the grad buffers)
 *   under gradient    dc_accumulate for each micro-batch, then one
 *   accumulation      dc_deferred_reduce (or dc_accumulate_reduce for the
 *                     last micro-batch) ([MT] What)
 *   collectives       dc_reduce_scatter / dc_all_gather and their ring-order,
 *                     step-by-step and relaid (dc_relayout_bucket +
 *                     dc_reduce_scatter_v) forms
 *
 * Conventions shared by every function:
 *   - Return value: DC_OK (0) or one of the DC_ERR_* codes below.  Argument
 *     checks run on the host before anything is enqueued; a failed check
 *     enqueues nothing.  dc_last_error() gives a message for the calling
 *     thread's last failure.  No C++ exception crosses this boundary.
 *   - "device" pointers are HIP device (or managed) memory; "host" pointers
 *     are ordinary host memory read synchronously during the call.
 *   - The caller owns every buffer.  The library allocates nothing, keeps no
 *     pointer after the call returns (device pointers are used by the
 *     enqueued kernels until they finish) and never synchronizes the stream.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *   - dtype: DC_BF16 (bfloat16 stored as uint16 bit patterns) or DC_F32.
 *   - Slab base pointers must be 16-byte aligned and `ld` a multiple of 16
 *     bytes (8 bf16 or 4 fp32 elements), else DC_ERR_ALIGN.
 *   - Row strides, column counts and byte counts above 2^44 are DC_ERR_SHAPE,
 *     so that no size computed from them can overflow int64.
 *   - Sums are folded in fp32 in ascending rank order (member order within a
 *     communicator), starting from the first contribution, and rounded once
 *     to the dtype (round to nearest even; NaN -> quiet NaN 0x7FC0|sign for
 *     bf16).  fp32 arithmetic keeps subnormals and is never contracted.
 */
#ifndef DC_H
#define DC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dc_status;

#define DC_OK 0
#define DC_ERR_NULL 1        /* a required pointer is NULL */
#define DC_ERR_ARG 2         /* a scalar argument is out of range, or buffers overlap */
#define DC_ERR_SHAPE 3       /* sizes or strides do not fit together */
#define DC_ERR_ALIGN 4       /* a slab base or stride is not 16-byte aligned */
#define DC_ERR_DTYPE 5       /* unknown dtype */
#define DC_ERR_TASKS 6       /* a task table breaks its contract (dc_validate_tasks) */
#define DC_ERR_HIP 7         /* a HIP launch or runtime call failed */
#define DC_ERR_UNSUPPORTED 8 /* a valid request this library does not handle */

#define DC_BF16 0
#define DC_F32 1

#define DC_ORDER_RANK 0
#define DC_ORDER_RING 1

#define DC_SCHED_RING 0      /* all-gather step schedules (dc_all_gather_step) */
#define DC_SCHED_BIDIR 1
#define DC_SCHED_RD 2

#define DC_MAX_W 64          /* simulated ranks per slab */
#define DC_MAX_GROUPS 64     /* parameter groups per owner map */
#define DC_MAX_COMMS 8       /* communicators per flush */

/* One bucket entry: a whole parameter's gradient ([DS] "Describe
 * alternatives": buckets hold one full-parameter task each, in gradient
 * arrival order).  32 bytes.
 *   offset   first column of the task, relative to the bucket's first column
 *   numel    columns of the task (>= 0)
 *   param    index into the owner map
 *   comm     index into the flush's communicator table
 * For the slab flushes a bucket's table is sorted and packed: offset[0] = 0,
 * offset[t+1] = offset[t] + numel[t], and the numels sum to the bucket size.
 * dc_flush_bucket_buffers takes sorted, disjoint tasks with gaps allowed (its
 * offsets are coordinates only) and does not read `param`.  `reserved` is
 * not read by any entry point. */
typedef struct {
  int64_t offset;
  int64_t numel;
  int32_t param;
  int32_t comm;
  int64_t reserved;
} dc_task;

/* A communicator over the W ranks ([DS] Design points, groups reduced over a
 * different communicator, e.g. MoE experts): `size` c divides W and the ranks
 * split into W/c blocks; block b's members are {b*c + i} when stride == 1,
 * or {b + i*W/c} when stride == W/c (i = 0..c-1).  Entry 0 of every table is
 * the data-parallel communicator {W, 1}. */
typedef struct {
  int32_t size;
  int32_t stride;
} dc_comm;

/* Probe record of one flush ([DS] problem statement, the probe report, and
 * "reduce_probe").  Per rank r: written[r] = elements the flush writes to row
 * r, kept[r] = elements of tasks whose parameter rank r holds (its partition
 * appears in the parameter's partition list), discarded[r] = written - kept. */
typedef struct {
  int32_t tasks;
  int32_t owner_tasks;
  int32_t pre_div;
  int32_t dtype;
  int64_t reduced_elems;
  int64_t owner_elems;
  int64_t written[DC_MAX_W];
  int64_t kept[DC_MAX_W];
  int64_t discarded[DC_MAX_W];
} dc_probe;

/* One piece of a bucket relayout: bucket columns [src, src+len) move to
 * relaid columns [dst, dst+len).  32 bytes. */
typedef struct {
  int64_t src;
  int64_t dst;
  int64_t len;
  int64_t reserved;
} dc_piece;

/* One tile record of a planned bucket flush (dc_plan_flush).  The planned
 * flush cuts a bucket into plan tiles of 64 consecutive 16-byte column
 * vectors (1 KiB of each row; tile b of a bucket starting at column c covers
 * the row's vectors [v0 + 64 b, v0 + 64 (b + 1)), v0 = floor(c / E / 64) * 64
 * with E elements per vector, clipped to the bucket's last vector), one
 * workgroup per tile, and this record says which tasks a tile overlaps and,
 * when the whole tile lies inside one task and the bucket, which rows
 * receive its sums.  16 bytes.  A plan of n records keeps them XCD-major, in
 * the order the 8 XCDs run the tiles: the record of tile b sits at index
 * (b mod 8) floor(n/8) + min(b mod 8, n mod 8) + floor(b/8).
 *   first, last   indices of the first and last task overlapping the tile
 *                 (last < first: none)
 *   root          whole tile inside one task: the row that alone receives
 *                 the sums (the owner, or under ZeRO-2 the partition's rank),
 *                 or -1 for every member of each block (AllReduce)
 *   flags         bit 0: the whole tile lies inside task `first` and the
 *                 bucket; bits 8..15: that task's communicator */
typedef struct {
  int32_t first;
  int32_t last;
  int32_t root;
  int32_t flags;
} dc_tile;

/* Library version string (static storage). */
const char* dc_version(void);

/* Static description of a status code. */
const char* dc_strerror(dc_status status);

/* Message of the calling thread's last failed call ("" if none). */
const char* dc_last_error(void);

/* Partition lists ([DS] Design points, the owner map: the ZeRO
 * optimizer's param_to_partition_ids lists every optimizer partition holding
 * a piece of a parameter).  For each group g, the params
 * group_begin[g] .. group_begin[g+1]-1 are laid end to end in declaration
 * order (flat offset a_i = sum of earlier sizes in the group); the group's
 * T_g elements split into group_parts[g] equal partitions of
 * S_g = ceil(T_g / group_parts[g]) elements (the last one shorter); a
 * non-empty param's list is floor(a_i/S_g) .. floor((a_i+n_i-1)/S_g), an
 * empty param's list is empty.
 *   numel         device int64[num_params], each in [0, 2^48)
 *   group_begin   host int32[num_groups+1], non-decreasing, 0 .. num_params
 *   group_parts   host int32[num_groups], each in [1, DC_MAX_W]
 *   flat_offset   device int64[num_params] out: a_i
 *   part_size     device int64[num_groups] out: S_g
 *   pid_offsets   device int32[num_params+1] out: CSR row starts
 *   pids          device int32[pids_capacity] out: CSR entries
 * pids_capacity must be at least num_params + sum_g (group_parts[g] - 1),
 * the largest count any sizes can produce, else DC_ERR_SHAPE.  Sizes outside
 * [0, 2^48) are not checked on the host; the kernel treats a negative size
 * as 0.  One workgroup scans all groups. */
dc_status dc_partition_ids(int32_t W, int32_t num_params, const int64_t* numel,
                           int32_t num_groups, const int32_t* group_begin,
                           const int32_t* group_parts, int64_t* flat_offset, int64_t* part_size,
                           int32_t* pid_offsets, int32_t* pids, int64_t pids_capacity,
                           void* stream);

/* Owner map ([DS] Design points): a param whose partition list has a
 * single element is held by one rank only and gets that rank as its owner; a
 * param listed in two or more partitions (it straddles a partition
 * boundary) or in none gets -1, meaning AllReduce.  A group takes part only when its communicator is the
 * data-parallel one: group_comm_size[g] == W and group rank i maps to global
 * rank i for every i; every param of another group gets -1.
 *   pid_offsets, pids      device CSR from dc_partition_ids; pids_capacity is
 *                          the length of pids (entries beyond it are not read)
 *   group_begin            host int32[num_groups+1] (as for dc_partition_ids)
 *   group_comm_size        host int32[num_groups]
 *   group_rank_to_global   host int32[num_groups * W], row g = group g's
 *                          group rank -> global rank map (pad with -1)
 *   owner                  device int32[num_params] out
 *   counts                 device int32[2*num_groups] out: counts[2g] = params
 *                          with an owner, counts[2g+1] = params with two or
 *                          more entries (at most group_parts[g]-1)
 * Entries of pids outside [0, W) are reported as no owner. */
dc_status dc_build_owner_map(int32_t W, int32_t num_params, const int32_t* pid_offsets,
                             const int32_t* pids, int64_t pids_capacity, int32_t num_groups,
                             const int32_t* group_begin,
                             const int32_t* group_comm_size, const int32_t* group_rank_to_global,
                             int32_t* owner, int32_t* counts, void* stream);

/* Host check of a bucket's task table (run once when the bucket layout is
 * built): sorted and packed from offset 0, numel >= 0 summing to
 * bucket_numel, param in [0, num_params), comm in [0, num_comms); comms[0] is
 * {W, 1} and every comm's size divides W with stride 1 or W/size.
 * tasks and comms are host arrays.  Returns DC_ERR_TASKS with a message
 * naming the first broken entry. */
dc_status dc_validate_tasks(int32_t W, const dc_task* tasks, int32_t num_tasks,
                            int64_t bucket_numel, int32_t num_params, const dc_comm* comms,
                            int32_t num_comms);

/* Bucket flush ([DS] problem statement and "Describe the solution").
 * For every task t, column j of the bucket inside t, and block of the task's
 * communicator (c members m_0 < ... < m_{c-1}):
 *   v_k = pre_div ? round_dtype(fp32(x[m_k][j]) / c) : x[m_k][j]
 *   y   = round_dtype(((v_0 + v_1) + ...) + v_{c-1})      (fp32)
 * A task on comm 0 whose param has owner o >= 0 writes y to row o only (the
 * reduce-to-owner branch: same sum, same operand order, one destination);
 * every other task writes y to every member of the block (AllReduce).
 * owner == NULL is the empty map: every task AllReduces, bit for bit the path
 * without owners ([DS] Design points, "No native flag").  Elements the flush
 * does not write keep their contents.
 *   slab_in, ld_in     device [W, ld_in] gradients (bf16 or fp32 per dtype)
 *   slab_out, ld_out   device [W, ld_out] results; may equal slab_in (same
 *                      ld) for an in-place flush; partial overlap is DC_ERR_ARG
 *   bucket_col         first slab column of the bucket
 *   bucket_numel       columns of the bucket; bucket_col + bucket_numel must
 *                      not exceed ld_in or ld_out
 *   tasks, num_tasks   device dc_task[num_tasks] (see dc_validate_tasks)
 *   owner, num_params  device int32[num_params] from dc_build_owner_map, or NULL
 *   comms, num_comms   host dc_comm[num_comms], 1 <= num_comms <= DC_MAX_COMMS
 *   pre_div            0 or 1
 * The task table is read on the device and is not checked here (validate it
 * once with dc_validate_tasks).  A table that breaks the contract still
 * never makes the kernel touch memory outside the bucket's columns of the
 * two slabs: an out-of-range param or owner entry means AllReduce, an
 * out-of-range comm means comm 0, and columns no task covers are not
 * written. */
dc_status dc_flush_bucket(int32_t W, int32_t dtype, const void* slab_in, int64_t ld_in,
                          void* slab_out, int64_t ld_out, int64_t bucket_col,
                          int64_t bucket_numel, const dc_task* tasks, int32_t num_tasks,
                          const int32_t* owner, int32_t num_params, const dc_comm* comms,
                          int32_t num_comms, int32_t pre_div, void* stream);

/* ZeRO-2 owner path ([DS] "Follow-up": ZeRO-2 keeps real per-rank buffers at
 * offsets, so the reduce-to-owner optimization extends to every piece of a
 * parameter).  Same fold as dc_flush_bucket, but on the data-parallel comm
 * (comm 0) every element goes to the rank whose optimizer partition holds it:
 * element e of a task of param i sits at flat position flat_offset[i] + e of
 * its group and belongs to partition floor((flat_offset[i] + e) /
 * part_size[i]); the sum is written to that row only.  A task whose param has
 * part_size 0 (a group on another communicator), or any task on another
 * comm, AllReduces within its blocks as in dc_flush_bucket.
 *   flat_offset   device int64[num_params]: dc_partition_ids' flat offsets
 *   part_size     device int64[num_params]: S of the param's group, or 0
 * Other arguments, checks and guarantees as in dc_flush_bucket (a partition
 * index outside [0, W) means AllReduce for that element). */
dc_status dc_flush_bucket_zero2(int32_t W, int32_t dtype, const void* slab_in, int64_t ld_in,
                                void* slab_out, int64_t ld_out, int64_t bucket_col,
                                int64_t bucket_numel, const dc_task* tasks, int32_t num_tasks,
                                const int64_t* flat_offset, const int64_t* part_size,
                                int32_t num_params, const dc_comm* comms, int32_t num_comms,
                                int32_t pre_div, void* stream);

/* Plan of a bucket flush ([DS] Design points: the roots of a bucket's
 * collectives are computed for the whole bucket before any reduction).
 * Host only, once per bucket layout: for every plan tile (see dc_tile) over
 * columns [bucket_col, bucket_col + bucket_numel), the tasks it overlaps
 * and, for a tile inside one task, the rows its sums go to:
 *   owner-map mode (flat_offset == NULL): the owner owner[param] of a task on
 *   comm 0 when owner is given and the entry lies in [0, W), else -1;
 *   ZeRO-2 mode (flat_offset and part_size given, owner NULL): for a task on
 *   comm 0 whose param has part_size S > 0, the partition
 *   floor((flat_offset[param] + e) / S) when every element e of the tile
 *   lies in the same one inside [0, W) (otherwise the tile is not whole),
 *   else -1.
 *   tasks, num_tasks      host dc_task[num_tasks]; must pass dc_validate_tasks
 *                         (else DC_ERR_TASKS)
 *   owner                 host int32[num_params] or NULL
 *   flat_offset, part_size host int64[num_params] or NULL (ZeRO-2)
 *   comms, num_comms      host, as for dc_flush_bucket
 *   tiles, capacity       host dc_tile[capacity] out; NULL asks for the count
 *   num_tiles             out: the tile count, a function of dtype,
 *                         bucket_col and bucket_numel only
 *   root_tiles            out (may be NULL): tiles whose sums go to one row
 *                         (whole tiles with root >= 0), set with the tiles
 * Fewer than *num_tiles slots is DC_ERR_SHAPE.  The plan stays valid while
 * the layout, owner map (or partition sizes) and dtype stay the same. */
dc_status dc_plan_flush(int32_t W, int32_t dtype, int64_t bucket_col, int64_t bucket_numel,
                        const dc_task* tasks, int32_t num_tasks, const int32_t* owner,
                        const int64_t* flat_offset, const int64_t* part_size, int32_t num_params,
                        const dc_comm* comms, int32_t num_comms, dc_tile* tiles,
                        int64_t capacity, int64_t* num_tiles, int64_t* root_tiles);

/* The plan of dc_plan_flush computed on the device ([DS] Design points: a
 * bucket's reduction destinations are settled for the whole bucket before
 * it is reduced), for callers whose task table and owner map (or ZeRO-2
 * partition sizes) live in device memory: no host copy and no
 * synchronization.  The records are those dc_plan_flush writes for the same
 * arguments, bit for bit, and serve dc_flush_bucket_planned the same way.
 * One thread per tile binary-searches the task offsets.
 *   tasks                 device dc_task[num_tasks]; must be a table that
 *                         passes dc_validate_tasks (not checked here: another
 *                         table gives other records, and its params and
 *                         communicators index owner, flat_offset and
 *                         part_size only inside [0, num_params) and
 *                         [0, num_comms))
 *   owner                 device int32[num_params] or NULL (owner-map mode)
 *   flat_offset, part_size device int64[num_params] or NULL (ZeRO-2, as for
 *                         dc_plan_flush)
 *   comms, num_comms      host, as for dc_flush_bucket (checked)
 *   tiles, capacity       device dc_tile[capacity] out; NULL asks for the
 *                         count only (nothing is launched)
 *   num_tiles             host out: the tile count (as dc_plan_flush's)
 *   root_tiles            device int64 out, or NULL: set on the stream to
 *                         the count dc_plan_flush reports as root_tiles
 *                         (whole tiles with root >= 0); a caller that does
 *                         not read it back may pass num_tiles for
 *                         reduce-to-owner or ZeRO-2 buckets and 0 otherwise to
 *                         dc_flush_bucket_planned, which uses it only to pick
 *                         the launch shape
 * Fewer than *num_tiles slots is DC_ERR_SHAPE.  Stream-ordered: the plan is
 * ready for a planned flush later on the same stream. */
dc_status dc_plan_flush_device(int32_t W, int32_t dtype, int64_t bucket_col, int64_t bucket_numel,
                               const dc_task* tasks, int32_t num_tasks, const int32_t* owner,
                               const int64_t* flat_offset, const int64_t* part_size,
                               int32_t num_params, const dc_comm* comms, int32_t num_comms,
                               dc_tile* tiles, int64_t capacity, int64_t* num_tiles,
                               int64_t* root_tiles, void* stream);

/* Bucket flush with a plan (dc_plan_flush): the same results, bit for bit,
 * as dc_flush_bucket (flat_offset == NULL) or dc_flush_bucket_zero2
 * (flat_offset and part_size given, owner NULL) with the same arguments.  A
 * tile the plan marks whole streams its vectors with no search of the task
 * table and no staging; other tiles use the record's task range.  The
 * launch also keeps fewer workgroups resident per compute unit (it reserves
 * LDS it does not use): fewer, longer streams of loads in flight at once
 * measured faster for this access mix.
 *   tiles, num_tiles   device dc_tile[num_tiles] from dc_plan_flush for this
 *                      bucket, dtype, layout and map; num_tiles must equal
 *                      the planned count (else DC_ERR_SHAPE)
 *   root_tiles         the count dc_plan_flush reported, in [0, num_tiles]
 *                      (else DC_ERR_ARG); it only picks the residency cap:
 *                      buckets whose tiles mostly write one row keep more
 *                      workgroups per compute unit than those that write
 *                      every row, and any value gives the same results
 * Other arguments and checks as in dc_flush_bucket.  The plan is read on
 * the device and not checked: a stale or altered plan can give wrong sums,
 * and write columns of slab_out's rows outside the bucket but inside its
 * tile grid (the 64-vector tiles that cover the bucket), but never makes the
 * kernel touch memory outside the two slabs' W rows of ld columns (task
 * indices, roots and communicators are clamped to their ranges). */
dc_status dc_flush_bucket_planned(int32_t W, int32_t dtype, const void* slab_in, int64_t ld_in,
                                  void* slab_out, int64_t ld_out, int64_t bucket_col,
                                  int64_t bucket_numel, const dc_task* tasks, int32_t num_tasks,
                                  const int32_t* owner, const int64_t* flat_offset,
                                  const int64_t* part_size, int32_t num_params,
                                  const dc_comm* comms, int32_t num_comms, int32_t pre_div,
                                  const dc_tile* tiles, int64_t num_tiles, int64_t root_tiles,
                                  void* stream);

/* Bucket flush with copy-in and copy-out fused in ([DS] problem statement:
 * gradients enter the bucket from every rank and, after the reduction, the
 * copy-out moves the result into each rank's gradient buffer, skipping the
 * ranks whose buffer is empty; "Describe the solution": copy-out unchanged
 * and still correct).  No bucket is staged: rank r's gradient of task t is
 * read from in_ptrs[t*W + r] and the sum is written to out_ptrs[t*W + r]
 * for every member r of the block whose pointer is not NULL (a NULL pointer
 * is an empty buffer and is never written).  For every task t, element
 * e < numel and block of the task's communicator (members m_0 < ... < m_{c-1}):
 *   v_k = pre_div ? round_dtype(fp32(in_ptrs[t*W + m_k][e]) / c) : in_ptrs[t*W + m_k][e]
 *   y   = round_dtype(((v_0 + v_1) + ...) + v_{c-1})      (fp32)
 * the same values, in the same order, as dc_flush_bucket on a bucket filled
 * from those buffers; with exactly one non-NULL output (the owner) it is the
 * reduce-to-owner flush followed by the copy-out.
 *   bucket_numel       extent of the task coordinates: offsets and numel of
 *                      the tasks place them in [0, bucket_numel)
 *   tasks, num_tasks   device dc_task[num_tasks] sorted by offset, disjoint
 *                      (gaps allowed); param is not used; an out-of-range
 *                      comm means comm 0
 *   in_ptrs            device array [num_tasks * W] of device pointers, each
 *                      to numel elements of the dtype (rank r's gradient)
 *   out_ptrs           device array [num_tasks * W] of device pointers or NULL
 *   comms, num_comms   host dc_comm[num_comms] as in dc_flush_bucket
 *   pre_div            0 or 1
 * An output may be the same buffer as its own input (in place); otherwise
 * outputs must not overlap each other or any input (check the tables once
 * with dc_validate_buffer_tasks).  A task whose offset is a multiple of 16
 * bytes' worth of elements and whose pointers are all 16-byte aligned runs on
 * 16-byte vectors; any other element runs one at a time. */
dc_status dc_flush_bucket_buffers(int32_t W, int32_t dtype, int64_t bucket_numel,
                                  const dc_task* tasks, int32_t num_tasks,
                                  const void* const* in_ptrs, void* const* out_ptrs,
                                  const dc_comm* comms, int32_t num_comms, int32_t pre_div,
                                  void* stream);

/* Plan of a fused flush (dc_flush_bucket_buffers' tables), host only, once
 * per registration: the fused kernel cuts the bucket's coordinates
 * [0, bucket_numel) into tiles of 64 slots of 16 bytes (slot v covers
 * coordinates [v E, v E + E), E elements per 16 bytes), and tile b's record
 * names the first task starting at or before the tile and the last starting
 * inside it (last < first: none), and sets flags bit 0 when the tile's slots
 * all lie inside that one task, the task is on the data-parallel comm and its
 * offset is a multiple of E; root is -1.  Records are XCD-major as in
 * dc_tile.
 *   tasks, comms        host copies: tasks sorted, disjoint, inside the
 *                       bucket, comm in range (else DC_ERR_TASKS)
 *   tiles, capacity     host dc_tile[capacity] out; NULL asks for the count
 *   num_tiles           out: ceil(ceil(bucket_numel / E) / 64), 0 with no
 *                       tasks; fewer slots than that is DC_ERR_SHAPE */
dc_status dc_plan_flush_buffers(int32_t W, int32_t dtype, int64_t bucket_numel, const dc_task* tasks,
                                int32_t num_tasks, const dc_comm* comms, int32_t num_comms,
                                dc_tile* tiles, int64_t capacity, int64_t* num_tiles);

/* dc_plan_flush_buffers' records computed on the device, bit for bit, from a
 * task table in device memory (one thread per tile, binary search of the
 * task offsets): no host copy and no synchronization.
 *   tasks             device dc_task[num_tasks] in buffer coordinates; must
 *                     pass dc_validate_buffer_tasks (not checked here:
 *                     another table gives other records, every read and
 *                     write stays in the table and the plan)
 *   comms, num_comms  host, checked as for dc_plan_flush_buffers
 *   tiles, capacity   device dc_tile[capacity] out; NULL asks for the count
 *                     only (nothing is launched)
 *   num_tiles         host out: the tile count (dc_plan_flush_buffers')
 * Fewer than *num_tiles slots is DC_ERR_SHAPE.  Stream-ordered. */
dc_status dc_plan_flush_buffers_device(int32_t W, int32_t dtype, int64_t bucket_numel,
                                       const dc_task* tasks, int32_t num_tasks,
                                       const dc_comm* comms, int32_t num_comms, dc_tile* tiles,
                                       int64_t capacity, int64_t* num_tiles, void* stream);

/* dc_flush_bucket_buffers with a plan from dc_plan_flush_buffers: the same
 * results, bit for bit.  A tile the plan marks whole, whose task the kernel
 * finds covering the tile and whose W input and output pointers are 16-byte
 * aligned, streams from the task's pointer row with no search and no staging;
 * every other tile takes the staged path over the record's task range.
 *   tiles, num_tiles   device dc_tile[num_tiles]; num_tiles must equal the
 *                      planned count (else DC_ERR_SHAPE)
 * Other arguments as in dc_flush_bucket_buffers.  The plan is read on the
 * device and not checked: a stale plan can leave columns unwritten or give
 * wrong sums, but the kernel checks a whole tile's task before using its
 * pointers, so it never addresses memory outside the registered buffers. */
dc_status dc_flush_bucket_buffers_planned(int32_t W, int32_t dtype, int64_t bucket_numel,
                                          const dc_task* tasks, int32_t num_tasks,
                                          const void* const* in_ptrs, void* const* out_ptrs,
                                          const dc_comm* comms, int32_t num_comms, int32_t pre_div,
                                          const dc_tile* tiles, int64_t num_tiles, void* stream);

/* Host check of the tables of dc_flush_bucket_buffers (run once when the
 * buffers are registered): tasks sorted by offset, disjoint, numel >= 0,
 * inside [0, bucket_numel), comm in [0, num_comms); comms as in
 * dc_validate_tasks; a non-NULL input for every rank of every non-empty task;
 * no output overlapping another output or any input other than its own (an
 * output equal to its own input is the in-place case).  tasks, comms and the
 * two pointer tables are host copies (the pointer values are compared, never
 * dereferenced).  Returns DC_ERR_TASKS with a message naming the first
 * problem. */
dc_status dc_validate_buffer_tasks(int32_t W, int32_t dtype, const dc_task* tasks, int32_t num_tasks,
                                   int64_t bucket_numel, const dc_comm* comms, int32_t num_comms,
                                   const void* const* in_ptrs, void* const* out_ptrs);

/* Probe counts of one flush ([DS] "reduce_probe"), on the host from
 * metadata only (no device access, no synchronization).  tasks, owner (or
 * NULL for the empty map), pid_offsets/pids (the CSR of dc_partition_ids)
 * and comms are host arrays.  Holders of a param on a sub-communicator are,
 * in every block, the members whose in-block index is in its list. */
dc_status dc_probe_flush(int32_t W, int32_t dtype, const dc_task* tasks, int32_t num_tasks,
                         const int32_t* owner, int32_t num_params, const int32_t* pid_offsets,
                         const int32_t* pids, const dc_comm* comms, int32_t num_comms,
                         int32_t pre_div, dc_probe* out);

/* Holders of every task's param ([DS] problem statement: the copy-out after
 * the reduction writes each rank's gradient buffer and skips the ranks
 * whose buffer is empty; a rank keeps a buffer for a param when its
 * optimizer partition holds part of it, [DS] Design points).  Host only:
 * holders[t*W + r] = 1 when rank r's partition (its group rank, in every
 * block of a sub-communicator) is in the partition list of task t's param,
 * else 0 -- the ranks whose elements dc_probe_flush counts as kept, and the
 * outputs a fused flush (dc_flush_bucket_buffers) writes.
 *   tasks, num_tasks        host dc_task[num_tasks]; param in [0, num_params)
 *                           and comm in [0, num_comms) (else DC_ERR_TASKS)
 *   pid_offsets, pids       host CSR from dc_partition_ids
 *   comms, num_comms        host, as for dc_flush_bucket
 *   holders                 host uint8[num_tasks * W] out
 * A partition id outside its communicator is DC_ERR_TASKS. */
dc_status dc_holders(int32_t W, const dc_task* tasks, int32_t num_tasks, int32_t num_params,
                     const int32_t* pid_offsets, const int32_t* pids, const dc_comm* comms,
                     int32_t num_comms, uint8_t* holders);

/* Per-param ZeRO-2 partition sizes ([DS] "Follow-up": the ZeRO-2 owner path
 * sends every element to the rank whose partition holds it): for every
 * param of group g, param_part_size = part_size[g] (dc_partition_ids' S_g)
 * when g is on the data-parallel communicator -- the rule of
 * dc_build_owner_map: group_comm_size[g] == W and group rank i is global
 * rank i -- and 0 otherwise (such params keep AllReduce within their
 * blocks).  This is the part_size argument of dc_flush_bucket_zero2,
 * dc_plan_flush and dc_plan_relayout.
 *   group_begin, group_comm_size, group_rank_to_global  host, as for
 *                                                       dc_build_owner_map
 *   part_size          device int64[num_groups] from dc_partition_ids
 *   param_part_size    device int64[num_params] out */
dc_status dc_param_part_size(int32_t W, int32_t num_params, int32_t num_groups,
                             const int32_t* group_begin, const int32_t* group_comm_size,
                             const int32_t* group_rank_to_global, const int64_t* part_size,
                             int64_t* param_part_size, void* stream);

/* Relayout plan for a reduce-scatter over a bucket ([DS] "Describe
 * alternatives": a reduce-scatter needs the bucket laid out contiguously by
 * destination rank).  Every element of a task on the data-parallel comm whose
 * param has part_size > 0 belongs to partition
 * q = floor((flat_offset[param] + e) / part_size[param]); segment q of the
 * relaid bucket holds those elements in bucket order, and the segments follow
 * each other (q = 0..W-1).  Other tasks are not relaid.  Host only.
 *   tasks, num_tasks         host dc_task[] of the bucket (as validated by
 *                            dc_validate_tasks)
 *   flat_offset, part_size   host int64[num_params] (as for
 *                            dc_flush_bucket_zero2)
 *   pieces                   host dc_piece[pieces_capacity] out, sorted by
 *                            dst; NULL asks for the count only
 *   num_pieces               out: the number of pieces (at most num_tasks +
 *                            (W-1) per partitioned group in the bucket)
 *   seg_start                host int64[W+1] out: segment boundaries
 * Fewer than num_pieces slots is DC_ERR_SHAPE; a partition index outside
 * [0, W) is DC_ERR_TASKS. */
dc_status dc_plan_relayout(int32_t W, const dc_task* tasks, int32_t num_tasks,
                           const int64_t* flat_offset, const int64_t* part_size,
                           int32_t num_params, dc_piece* pieces, int32_t pieces_capacity,
                           int32_t* num_pieces, int64_t* seg_start);

/* Apply a relayout plan to every row: out[r][dst + i] = slab_in[r][bucket_col
 * + src + i] for each piece and i < len (pure data movement).
 *   slab_in, ld_in   device [W, ld_in]; the bucket is columns
 *                    [bucket_col, bucket_col + bucket_numel)
 *   out, ld_out      device [W, ld_out], ld_out >= out_numel; must not
 *                    overlap slab_in
 *   pieces           device dc_piece[num_pieces] sorted by dst
 * Only columns [0, out_numel) of `out` are written; a piece reaching outside
 * the bucket or outside [0, out_numel) is clipped, never followed. */
dc_status dc_relayout_bucket(int32_t W, int32_t dtype, const void* slab_in, int64_t ld_in,
                             void* out, int64_t ld_out, int64_t bucket_col, int64_t bucket_numel,
                             const dc_piece* pieces, int32_t num_pieces, int64_t out_numel,
                             void* stream);

/* Tile plan for dc_relayout_bucket_planned: the relayout above, taken to
 * the grain of the kernel's tiles once per bucket layout ([DS] Design
 * points: a bucket's layout is fixed, so what its flush needs is worked out
 * ahead of it).  The relaid bucket's columns [0, out_numel) fall into tiles
 * of 64 16-byte vectors (512 bf16 or 256 fp32 columns); one int64 per
 * tile, in an order private to the library, records where a tile copies
 * from when all of its columns belong to one piece (a column belongs to the
 * last piece whose dst is at or before it, if that piece reaches it) and
 * the piece's source run for the tile starts on a 16-byte vector of the
 * slab and stays in the bucket.  Host only.
 *   dtype, bucket_col, bucket_numel, pieces, num_pieces, out_numel
 *                    as for dc_relayout_bucket (pieces on the host, sorted
 *                    by dst as dc_plan_relayout writes them)
 *   tiles            host int64[tiles_capacity] out; NULL asks for the
 *                    count only
 *   num_tiles        out: ceil(ceil(out_numel / E) / 64), E = 8 (bf16) or
 *                    4 (fp32)
 * A negative piece length or pieces out of dst order is DC_ERR_ARG; fewer
 * than num_tiles slots is DC_ERR_SHAPE. */
dc_status dc_plan_relayout_tiles(int32_t dtype, int64_t bucket_col, int64_t bucket_numel,
                                 const dc_piece* pieces, int32_t num_pieces, int64_t out_numel,
                                 int64_t* tiles, int64_t tiles_capacity, int64_t* num_tiles);

/* dc_plan_relayout_tiles' records computed on the device, bit for bit, from
 * a piece table in device memory (one thread per destination tile, binary
 * search of the pieces' destinations): no host copy and no synchronization.
 *   pieces            device dc_piece[num_pieces]; must be sorted by dst with
 *                     no negative length (not checked here: another table
 *                     gives other records, every read and write stays in the
 *                     table and the plan)
 *   tiles, capacity   device int64[capacity] out; NULL asks for the count
 *                     only (nothing is launched)
 *   num_tiles         host out: the tile count (dc_plan_relayout_tiles')
 * Other arguments and checks as for dc_plan_relayout_tiles.  Stream-ordered. */
dc_status dc_plan_relayout_tiles_device(int32_t dtype, int64_t bucket_col, int64_t bucket_numel,
                                        const dc_piece* pieces, int32_t num_pieces,
                                        int64_t out_numel, int64_t* tiles, int64_t tiles_capacity,
                                        int64_t* num_tiles, void* stream);

/* dc_relayout_bucket from a tile plan: the same result, bit for bit.  A
 * tile with a record copies straight from it; any other tile searches the
 * pieces as dc_relayout_bucket does.  Arguments as for dc_relayout_bucket,
 * plus
 *   tiles, num_tiles  device int64[num_tiles] from dc_plan_relayout_tiles
 *                     on the same dtype, bucket, pieces and out_numel;
 *                     num_tiles must be the count it gives (else
 *                     DC_ERR_SHAPE)
 * A record is checked against the bucket before it is used: a plan made for
 * other pieces can misplace data inside the bucket's columns of `out`, but
 * never reads or writes outside them. */
dc_status dc_relayout_bucket_planned(int32_t W, int32_t dtype, const void* slab_in, int64_t ld_in,
                                     void* out, int64_t ld_out, int64_t bucket_col, int64_t bucket_numel,
                                     const dc_piece* pieces, int32_t num_pieces, int64_t out_numel,
                                     const int64_t* tiles, int64_t num_tiles, void* stream);

/* Reduce-scatter with variable shards: shard q is columns
 * [seg_start[q], seg_start[q+1]) of `in`, and
 *   out[q][k] = round_dtype(fold over r of pre(in[r][seg_start[q] + k]))
 * with the flush's fold and pre-division by W.
 *   seg_start     host int64[W+1], non-decreasing from 0, seg_start[W] <= ld_in
 *   out, ld_out   device [W, ld_out], ld_out >= the longest shard; no overlap */
dc_status dc_reduce_scatter_v(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                              int64_t ld_out, const int64_t* seg_start, int32_t pre_div,
                              void* stream);

/* ReduceScatter ([AG] duality with ReduceScatter: M elements in per node,
 * M/N out, a reduction plus a split).  With L = M / W:
 *   out[s][k] = round_dtype(fold over r of pre(in[r][s*L + k]))   k < L
 * using the flush's fold and pre-division (by W).
 *   in, ld_in     device [W, ld_in], ld_in >= M
 *   out, ld_out   device [W, ld_out], ld_out >= L; must not overlap `in`
 * M % W != 0 is DC_ERR_SHAPE (pad with zeros to a multiple of W). */
dc_status dc_reduce_scatter(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                            int64_t ld_out, int64_t M, int32_t pre_div, void* stream);

/* AllGather ([AG] semantic definition and Ring AllGather).  Shard s is
 * row s of `in` (L = shard_numel columns).
 *   DC_ORDER_RANK: out[i][s*L + k] = in[s][k] - every node ends with
 *                  [A_0, ..., A_{W-1}].
 *   DC_ORDER_RING: out[i][p*L + k] = in[(i - p) mod W][k] - position p of
 *                  node i holds the chunk a ring all-gather delivers at step
 *                  p (own chunk first, then one chunk per step from the left
 *                  neighbour).
 * step = -1 writes every position; step = s in [0, W) writes chunk s (rank
 * order) or position s (ring order) only, so a ring can be replayed step by
 * step.
 *   in, ld_in     device [W, ld_in], ld_in >= L
 *   out, ld_out   device [W, ld_out], ld_out >= W*L; must not overlap `in` */
dc_status dc_all_gather(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                        int64_t ld_out, int64_t shard_numel, int32_t order, int32_t step,
                        void* stream);

/* Ring-order ReduceScatter: the sum a ring reduce-scatter produces.  A ring
 * passes partial sums to the right, each node adding its own contribution,
 * so chunk s is folded in rank order s, s+1, ..., s-1 (mod W) instead of
 * 0..W-1 ([DS] Numerics: the summation order changes with the algorithm,
 * which is why owner and AllReduce results need not be bit-identical):
 *   out[s][k] = round_dtype(fold over j = 0..W-1 of pre(in[(s+j) mod W][s*L + k]))
 * Arguments, layout and checks as in dc_reduce_scatter. */
dc_status dc_reduce_scatter_ring(int32_t W, int32_t dtype, const void* in, int64_t ld_in,
                                 void* out, int64_t ld_out, int64_t M, int32_t pre_div,
                                 void* stream);

/* One step of an AllGather schedule ([AG] Ring AllGather, bidirectional
 * ring, Recursive Doubling AllGather) executed on one GPU: row i of `out`
 * ([W, W*L]) is node i's buffer, and every chunk is stored at its own index,
 * so after the last step every row is the rank-order concatenation.
 *   step 0            node i places its own shard: out[i][i*L + k] = in[i][k]
 *   DC_SCHED_RING     steps 1..W-1: node i receives chunk (i - step) mod W
 *                     from node i-1
 *   DC_SCHED_BIDIR    steps 1..ceil((W-1)/2): node i receives chunk
 *                     (i - step) mod W from node i-1 and chunk (i + step)
 *                     mod W from node i+1 (once when they coincide)
 *   DC_SCHED_RD       steps 1..log2 W (W a power of two): node i receives
 *                     the 2^(step-1) chunks held by node i XOR 2^(step-1)
 * Steps must run in order on the same buffers.  Other arguments as in
 * dc_all_gather; a step outside the schedule is DC_ERR_ARG. */
dc_status dc_all_gather_step(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                             int64_t ld_out, int64_t shard_numel, int32_t algo, int32_t step,
                             void* stream);

/* Replica-local accumulation ([MT] What: unreduced per-replica partial
 * sums accumulate locally across micro-batches).  fp32 only:
 *   acc[r][j] = acc[r][j] + x[r][j]        r < rows, j < M
 * and with init = 1 the accumulator starts from zero: acc = +0.0f + x.
 *   x, ld_x       device [rows, ld_x] fp32
 *   acc, ld_acc   device [rows, ld_acc] fp32, updated in place; may equal x */
dc_status dc_accumulate(int32_t rows, const float* x, int64_t ld_x, float* acc, int64_t ld_acc,
                        int64_t M, int32_t init, void* stream);

/* Deferred cross-replica reduce ([MT] What: the single all-reduce that
 * update() emits).  fp32 only:
 *   out[i][j] = fold over r = 0..W-1 of acc[r][j]        i < out_rows, j < M
 * out_rows is 1 (one reduced copy) or W (every replica gets the sum).  With
 * out_rows = 1 and W rows of one micro-batch this is also the
 * per-micro-batch reduce of the status quo.
 *   acc, ld_acc   device [W, ld_acc] fp32
 *   out, ld_out   device [out_rows, ld_out] fp32; may equal acc (same ld) */
dc_status dc_deferred_reduce(int32_t W, const float* acc, int64_t ld_acc, float* out,
                             int64_t ld_out, int64_t M, int32_t out_rows, void* stream);

/* Accumulation and the deferred reduce fused for the last micro-batch of a step: the same fp32
 * operations as dc_accumulate followed by dc_deferred_reduce, in one pass
 * (bit-identical results), without writing the accumulator and reading it
 * back ([MT] What: the accumulated partial sums feed the single reduce in
 * update()).  For every j < M:
 *   a_r = init ? +0.0f + x[r][j] : acc[r][j] + x[r][j]      r < W
 *   acc[r][j] = a_r                      only when keep_acc = 1
 *   out[i][j] = fold over r = 0..W-1 of a_r                  i < out_rows
 *   x, ld_x       device [W, ld_x] fp32
 *   acc, ld_acc   device [W, ld_acc] fp32 (not read when init = 1); may
 *                 equal x (same ld)
 *   out, ld_out   device [out_rows, ld_out] fp32, out_rows 1 or W; may equal
 *                 acc (same ld) only when keep_acc = 0; must not overlap x
 * Algorithmic bytes: W*M*4 read of x, W*M*4 read of acc unless init,
 * W*M*4 written to acc if keep_acc, out_rows*M*4 written. */
dc_status dc_accumulate_reduce(int32_t W, const float* x, int64_t ld_x, float* acc, int64_t ld_acc,
                               int32_t init, int32_t keep_acc, float* out, int64_t ld_out,
                               int32_t out_rows, int64_t M, void* stream);

/* fp32 -> bf16 with the rounding the flush uses (round to nearest even, NaN
 * -> 0x7FC0|sign), n elements, device arrays; a self-check of the
 * conversion on the GPU. */
dc_status dc_round_bf16(const float* in, uint16_t* out, int64_t n, void* stream);

/* Plain 16-byte streaming copy of `bytes` (a multiple of 16; both pointers
 * 16-byte aligned, not overlapping): the achievable-bandwidth reference the
 * measurements compare against. */
dc_status dc_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Access-mix reference for measurements: for each of `nvec` 16-byte column
 * vectors, read it from rows_read rows of `src` (rows src_ld_vec vectors
 * apart), xor them, and store the result to rows_written rows of `dst`
 * (rows dst_ld_vec vectors apart).  No other arithmetic, so its bandwidth is
 * what the memory system gives the flush's access mix (W rows read, one row
 * or W rows written).  rows_read is 4, 8 or 16 and rows_written 1 or
 * rows_read (else DC_ERR_UNSUPPORTED); pointers 16-byte aligned; the two
 * regions must not overlap. */
dc_status dc_stream_rows(const void* src, int64_t src_ld_vec, int32_t rows_read, void* dst,
                         int64_t dst_ld_vec, int32_t rows_written, int64_t nvec, void* stream);

/* The access-mix reference at a launch shape of the planned flush: the same
 * xor stream as dc_stream_rows, but each one-wave workgroup takes `group`
 * (1, 2 or 4) runs of 64 vectors -- with one row written their results are
 * stored together after the last load -- at most `cap` workgroups stay
 * resident per compute unit (0: no cap, at most 64), and the stores use the
 * planned flush's cache policies.  A sweep over shapes that includes a
 * kernel's own gives a reference its access mix cannot beat with xor for
 * arithmetic.  Other arguments and checks as in dc_stream_rows, except
 * that rows_read 1 with rows_written 4, 8 or 16 (the all-gather's mix: one
 * row read, every row written) and rows_read 8 with rows_written 4 (the
 * W = 4 fused accumulate-reduce's: accumulators and micro-batch read, every
 * replica row written) are also supported; a group outside {1, 2, 4} is
 * DC_ERR_UNSUPPORTED. */
dc_status dc_stream_rows_shaped(const void* src, int64_t src_ld_vec, int32_t rows_read, void* dst,
                                int64_t dst_ld_vec, int32_t rows_written, int64_t nvec,
                                int32_t group, int32_t cap, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DC_H */
