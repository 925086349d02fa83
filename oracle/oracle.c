/*
 * CPU oracle for the data-parallel gradient-reduction path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * CPU-baseline leg of bench.py may load this library.  It shares no code,
 * header or constant with the GPU library (gradient_reduction_amd/); the
 * only thing the two sides have in common is the seeded input generator in
 * synth/.
 *
 * Plain, slow, obviously correct loops.  Build with
 *   gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math
 * so that every float operation below is one IEEE-754 binary32 operation
 * rounded to nearest-even (x86-64 SSE arithmetic, no contraction, no flush to
 * zero).
 *
 * Pages followed (cited by title and section):
 *  [DS]  DeepSpeed issue "[REQUEST] DeepCompile ZeRO-1: reduce-to-owner
 *        instead of AllReduce".
 *  [MT]  MaxText PR "Defer the data-parallel gradient all-reduce to update()
 *        under gradient accumulation".
 *  [AG]  "AllGather" (collective-communication notes).
 *
 * Precision readings (the pages do not fix them): sums run in fixed rank
 * order 0..c-1 of the communicator, accumulate in fp32 starting from the
 * first contribution, and round once to the gradient dtype at the end;
 * pre-division rounds each contribution to the dtype; bf16 NaN results are
 * the canonical quiet NaN 0x7FC0 with the input's sign.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_BF16 0
#define OR_F32 1

/* ------------------------------------------------------------------------ */
/* Numbers                                                                   */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 one. */
float or_bf16_to_f32(uint16_t b) { return f32_from_bits((uint32_t)b << 16); }

/* fp32 -> bf16, round to nearest, ties to even.  For a finite value the two
 * bf16 candidates are the fp32 pattern truncated to its top 16 bits and the
 * next pattern up in magnitude; the discarded low half decides which one is
 * nearer (above 0x8000: up, below: down, exactly 0x8000: the even one).
 * Magnitude grows with the pattern, and a carry out of the largest finite
 * value lands on infinity, as round-to-nearest requires. */
uint16_t or_f32_to_bf16(float f) {
  uint32_t u = bits_from_f32(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
    return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
  uint32_t hi = u >> 16;
  uint32_t lo = u & 0xFFFFu;
  if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;
  return (uint16_t)hi;
}

/* Array form of or_f32_to_bf16. */
void or_f32_to_bf16_array(const float* x, uint16_t* out, int64_t n) {
  for (int64_t k = 0; k < n; ++k) out[k] = or_f32_to_bf16(x[k]);
}

static float load_val(int dtype, const void* base, int64_t ld, int64_t row, int64_t col) {
  if (dtype == OR_BF16) return or_bf16_to_f32(((const uint16_t*)base)[row * ld + col]);
  return ((const float*)base)[row * ld + col];
}

/* round_dtype: to bf16 and back (exact), or the identity for fp32. */
static float round_dtype(int dtype, float v) {
  if (dtype == OR_BF16) return or_bf16_to_f32(or_f32_to_bf16(v));
  return v;
}

static void store_val(int dtype, void* base, int64_t ld, int64_t row, int64_t col, float v) {
  if (dtype == OR_BF16)
    ((uint16_t*)base)[row * ld + col] = or_f32_to_bf16(v);
  else
    ((float*)base)[row * ld + col] = v;
}

/* One contribution after the optional pre-division.
 * [DS] Design points, "Summation semantics untouched": pre-division divides
 * by the world size before the sum; read per contribution, by the size of the
 * communicator the sum runs over, rounded to the gradient dtype. */
static float contribution(int dtype, float x, int pre_div, int c) {
  if (!pre_div) return x;
  return round_dtype(dtype, x / (float)c);
}

/* Member i of block b of a communicator of size c and member stride s over
 * W ranks: contiguous blocks {b*c + i} when s == 1, else strided {b + i*s}. */
static int member(int b, int i, int c, int s) { return (s == 1 ? b * c : b) + i * s; }

/* ------------------------------------------------------------------------ */
/* Partition ids ([DS] Design points, owner map: param_to_partition_ids   */
/* lists every optimizer partition holding a piece of each parameter).       */
/* ------------------------------------------------------------------------ */

/* Per group g (params group_begin[g] .. group_begin[g+1]-1 in declaration
 * order): flat offsets a_i = sum of earlier sizes, total T_g, partition size
 * S_g = ceil(T_g / p_g) (equal partitions, the last one shorter), and for a
 * non-empty param the partitions floor(a_i/S_g) .. floor((a_i+n_i-1)/S_g).
 * Output is CSR: pids[pid_offsets[i] .. pid_offsets[i+1]).  Returns the pid
 * count, or -1 when `cap` is too small. */
int64_t or_partition_ids(int32_t P, const int64_t* numel, int32_t G, const int32_t* group_begin,
                         const int32_t* group_parts, int64_t* flat_offset, int64_t* part_size,
                         int32_t* pid_offsets, int32_t* pids, int64_t cap) {
  int64_t pos = 0;
  for (int32_t g = 0; g < G; ++g) {
    int64_t T = 0;
    for (int32_t i = group_begin[g]; i < group_begin[g + 1]; ++i) T += numel[i];
    int64_t p = group_parts[g];
    int64_t S = (T + p - 1) / p;
    part_size[g] = S;
    int64_t a = 0;
    for (int32_t i = group_begin[g]; i < group_begin[g + 1]; ++i) {
      flat_offset[i] = a;
      pid_offsets[i] = (int32_t)pos;
      if (numel[i] > 0) {
        int64_t first = a / S, last = (a + numel[i] - 1) / S;
        for (int64_t q = first; q <= last; ++q) {
          if (pos >= cap) return -1;
          pids[pos++] = (int32_t)q;
        }
      }
      a += numel[i];
    }
  }
  pid_offsets[P] = (int32_t)pos;
  return pos;
}

/* [DS] Design points, MoE groups: a group takes part only when its
 * communicator is DeepCompile's data-parallel one: same world size, and group
 * rank i is global rank i for every i. */
void or_group_eligible(int32_t W, int32_t G, const int32_t* comm_size,
                       const int32_t* rank_to_global, int32_t* eligible) {
  for (int32_t g = 0; g < G; ++g) {
    int ok = comm_size[g] == W;
    for (int32_t i = 0; ok && i < W; ++i) ok = rank_to_global[(int64_t)g * W + i] == i;
    eligible[g] = ok;
  }
}

/* Owner map ([DS] Design points, the owner map): a param whose partition
 * list has a single element is held by one rank only, the rank that element
 * names, and gets that rank as its owner; a param listed in two or more
 * partitions (a straddler), in none, or in an excluded group gets -1, which
 * the flush treats as AllReduce.  counts[2g] = owners, counts[2g+1] =
 * straddlers (params with two or more entries) in group g. */
void or_owner_map(int32_t P, const int32_t* pid_offsets, const int32_t* pids, int32_t G,
                  const int32_t* group_begin, const int32_t* eligible, int32_t* owner,
                  int32_t* counts) {
  (void)P;
  for (int32_t g = 0; g < G; ++g) {
    counts[2 * g] = 0;
    counts[2 * g + 1] = 0;
    for (int32_t i = group_begin[g]; i < group_begin[g + 1]; ++i) {
      int32_t n = pid_offsets[i + 1] - pid_offsets[i];
      owner[i] = (eligible[g] && n == 1) ? pids[pid_offsets[i]] : -1;
      if (owner[i] >= 0) counts[2 * g] += 1;
      if (n >= 2) counts[2 * g + 1] += 1;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Bucket flush ([DS] problem statement and "Describe the solution").       */
/* ------------------------------------------------------------------------ */

/* For every task t and every column j of it, for every block of the task's
 * communicator: fold the members' contributions in ascending member order in
 * fp32, round to the dtype, then write.  A task on the data-parallel comm
 * (comm 0) whose parameter has an owner writes the owner's row only (the
 * reduce-to-owner branch: same reduction, same operand order, one
 * destination); every other task writes the sum to every member of its block
 * (AllReduce).  owner == NULL is the empty map: AllReduce everything.  No
 * other output element is written. */
void or_flush(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out, int64_t ld_out,
              int64_t bucket_col, int32_t n_tasks, const int64_t* t_off, const int64_t* t_numel,
              const int32_t* t_param, const int32_t* t_comm, const int32_t* owner,
              const int32_t* comm_size, const int32_t* comm_stride, int32_t pre_div) {
  for (int32_t t = 0; t < n_tasks; ++t) {
    int c = comm_size[t_comm[t]];
    int s = comm_stride[t_comm[t]];
    int nb = W / c;
    int root = (t_comm[t] == 0 && owner != NULL) ? owner[t_param[t]] : -1;
    for (int64_t j = bucket_col + t_off[t]; j < bucket_col + t_off[t] + t_numel[t]; ++j) {
      for (int b = 0; b < nb; ++b) {
        float acc = 0.0f;
        for (int i = 0; i < c; ++i) {
          float v = contribution(dtype, load_val(dtype, in, ld_in, member(b, i, c, s), j), pre_div, c);
          acc = (i == 0) ? v : acc + v;
        }
        /* the buffer may be the input too: every read above precedes the writes */
        if (root >= 0) {
          store_val(dtype, out, ld_out, root, j, acc);
        } else {
          for (int i = 0; i < c; ++i) store_val(dtype, out, ld_out, member(b, i, c, s), j, acc);
        }
      }
    }
  }
}

/* ZeRO-2 owner path ([DS] "Follow-up": ZeRO-2 keeps real per-rank buffers at
 * offsets, so the same optimization applies to every piece of a parameter).
 * Element e of a task on the data-parallel comm whose group is partitioned
 * (part_size[param] = S > 0) lies at flat position a + e of its group, where
 * a = flat_offset[param]; it belongs to partition floor((a + e) / S), and the
 * sum is written to that rank only.  Tasks on other communicators, or with
 * S = 0, AllReduce within their blocks exactly as in or_flush. */
void or_flush_zero2(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                    int64_t ld_out, int64_t bucket_col, int32_t n_tasks, const int64_t* t_off,
                    const int64_t* t_numel, const int32_t* t_param, const int32_t* t_comm,
                    const int64_t* flat_offset, const int64_t* part_size,
                    const int32_t* comm_size, const int32_t* comm_stride, int32_t pre_div) {
  for (int32_t t = 0; t < n_tasks; ++t) {
    int c = comm_size[t_comm[t]];
    int s = comm_stride[t_comm[t]];
    int nb = W / c;
    int64_t S = t_comm[t] == 0 ? part_size[t_param[t]] : 0;
    int64_t a = flat_offset[t_param[t]];
    int64_t start = bucket_col + t_off[t];
    for (int64_t j = start; j < start + t_numel[t]; ++j) {
      for (int b = 0; b < nb; ++b) {
        float acc = 0.0f;
        for (int i = 0; i < c; ++i) {
          float v = contribution(dtype, load_val(dtype, in, ld_in, member(b, i, c, s), j), pre_div, c);
          acc = (i == 0) ? v : acc + v;
        }
        if (S > 0) {
          store_val(dtype, out, ld_out, (a + (j - start)) / S, j, acc);
        } else {
          for (int i = 0; i < c; ++i) store_val(dtype, out, ld_out, member(b, i, c, s), j, acc);
        }
      }
    }
  }
}

/* Bucket flush with copy-in and copy-out done in place of the bucket
 * ([DS] problem statement: gradients reach the bucket from the ranks, and the
 * copy-out after the reduction skips every rank whose gradient buffer is
 * empty; "Describe the solution": copy-out is unchanged and still correct).
 * Rank r's gradient of task t lives at in[in_off[t*W + r] + e], e < numel;
 * rank r's gradient buffer for it at out[out_off[t*W + r] + e], or nowhere
 * when out_off is -1 (an empty buffer).  Every block of the task's
 * communicator folds its members in ascending order, exactly as the bucket
 * flush does, and the sum is copied into the buffer of every member that has
 * one; nothing else is written.  in and out are flat arrays of the dtype. */
void or_flush_buffers(int32_t W, int32_t dtype, const void* in, const int64_t* in_off, void* out,
                      const int64_t* out_off, int32_t n_tasks, const int64_t* t_numel,
                      const int32_t* t_comm, const int32_t* comm_size, const int32_t* comm_stride,
                      int32_t pre_div) {
  for (int32_t t = 0; t < n_tasks; ++t) {
    int c = comm_size[t_comm[t]];
    int s = comm_stride[t_comm[t]];
    int nb = W / c;
    for (int64_t e = 0; e < t_numel[t]; ++e) {
      for (int b = 0; b < nb; ++b) {
        float sum = 0.0f;
        for (int i = 0; i < c; ++i) {
          int r = member(b, i, c, s);
          float v = contribution(dtype, load_val(dtype, in, 0, 0, in_off[(int64_t)t * W + r] + e), pre_div, c);
          sum = (i == 0) ? v : sum + v;
        }
        for (int i = 0; i < c; ++i) {
          int r = member(b, i, c, s);
          int64_t o = out_off[(int64_t)t * W + r];
          if (o >= 0) store_val(dtype, out, 0, 0, o + e, sum);
        }
      }
    }
  }
}

/* Bucket relayout for a reduce-scatter ([DS] "Describe alternatives": a
 * reduce-scatter over the bucket needs the payload contiguous by destination
 * rank).  Every element of a data-parallel task with partition size S > 0
 * goes to segment q = floor((flat_offset + e) / S); segment q holds its
 * elements in arrival order (tasks in bucket order, elements in order), and
 * the segments follow each other, q = 0..W-1.  dest[c] = the relaid column
 * of bucket column c (-1 for an element of another task); seg_start[0..W]
 * = segment boundaries.  Returns the relaid length. */
int64_t or_relayout_map(int32_t W, int32_t n_tasks, const int64_t* t_off, const int64_t* t_numel,
                        const int32_t* t_param, const int32_t* t_comm, const int64_t* flat_offset,
                        const int64_t* part_size, int64_t bucket_numel, int64_t* dest,
                        int64_t* seg_start) {
  int64_t* count = (int64_t*)calloc((size_t)W, sizeof(int64_t));
  for (int64_t c = 0; c < bucket_numel; ++c) dest[c] = -1;
  /* pass 1: segment sizes */
  for (int32_t t = 0; t < n_tasks; ++t) {
    int64_t S = t_comm[t] == 0 ? part_size[t_param[t]] : 0;
    if (S <= 0) continue;
    for (int64_t e = 0; e < t_numel[t]; ++e) count[(flat_offset[t_param[t]] + e) / S] += 1;
  }
  seg_start[0] = 0;
  for (int q = 0; q < W; ++q) seg_start[q + 1] = seg_start[q] + count[q];
  /* pass 2: place elements in arrival order */
  for (int q = 0; q < W; ++q) count[q] = seg_start[q];
  for (int32_t t = 0; t < n_tasks; ++t) {
    int64_t S = t_comm[t] == 0 ? part_size[t_param[t]] : 0;
    if (S <= 0) continue;
    for (int64_t e = 0; e < t_numel[t]; ++e) {
      int64_t q = (flat_offset[t_param[t]] + e) / S;
      dest[t_off[t] + e] = count[q]++;
    }
  }
  free(count);
  return seg_start[W];
}

/* Apply a relayout map to every row: out[r][dest[c]] = in[r][bucket_col + c]. */
void or_relayout_apply(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                       int64_t ld_out, int64_t bucket_col, int64_t bucket_numel,
                       const int64_t* dest) {
  int64_t eb = dtype == OR_BF16 ? 2 : 4;
  for (int r = 0; r < W; ++r)
    for (int64_t c = 0; c < bucket_numel; ++c)
      if (dest[c] >= 0)
        memcpy((char*)out + ((int64_t)r * ld_out + dest[c]) * eb,
               (const char*)in + ((int64_t)r * ld_in + bucket_col + c) * eb, (size_t)eb);
}

/* Reduce-scatter with variable shards: out[q][k] = round_dtype(fold over r
 * of pre(in[r][seg_start[q] + k])) for k < seg_start[q+1] - seg_start[q];
 * pre-division by W. */
void or_reduce_scatter_v(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                         int64_t ld_out, const int64_t* seg_start, int32_t pre_div) {
  for (int q = 0; q < W; ++q) {
    for (int64_t k = 0; k < seg_start[q + 1] - seg_start[q]; ++k) {
      float acc = 0.0f;
      for (int r = 0; r < W; ++r) {
        float v = contribution(dtype, load_val(dtype, in, ld_in, r, seg_start[q] + k), pre_div, W);
        acc = (r == 0) ? v : acc + v;
      }
      store_val(dtype, out, ld_out, q, k, acc);
    }
  }
}

/* Probe ([DS] problem statement probe line; "reduce_probe").  Host-only
 * bookkeeping from metadata.  Holders of a parameter: the ranks whose
 * partition appears in its partition list (for a sub-communicator group,
 * in every block the member whose in-block index appears).  Written rows:
 * the owner alone for an owned task, every rank otherwise.
 * out64 = {reduced, owner_elems}, out32 = {tasks, owner_tasks}. */
void or_probe(int32_t W, int32_t n_tasks, const int64_t* t_numel, const int32_t* t_param,
              const int32_t* t_comm, const int32_t* owner, const int32_t* pid_offsets,
              const int32_t* pids, const int32_t* comm_size, const int32_t* comm_stride,
              int64_t* out64, int32_t* out32, int64_t* written, int64_t* kept, int64_t* discarded) {
  int64_t reduced = 0, owner_elems = 0;
  int32_t owner_tasks = 0;
  for (int r = 0; r < W; ++r) written[r] = kept[r] = discarded[r] = 0;
  for (int32_t t = 0; t < n_tasks; ++t) {
    int64_t n = t_numel[t];
    int p = t_param[t];
    int c = comm_size[t_comm[t]];
    int s = comm_stride[t_comm[t]];
    int root = (t_comm[t] == 0 && owner != NULL) ? owner[p] : -1;
    reduced += n;
    if (root >= 0) {
      owner_tasks += 1;
      owner_elems += n;
    }
    char* wr = (char*)calloc((size_t)W, 1);
    char* hd = (char*)calloc((size_t)W, 1);
    if (root >= 0) wr[root] = 1;
    else for (int r = 0; r < W; ++r) wr[r] = 1;
    for (int32_t k = pid_offsets[p]; k < pid_offsets[p + 1]; ++k)
      for (int b = 0; b < W / c; ++b) hd[member(b, pids[k], c, s)] = 1;
    for (int r = 0; r < W; ++r) {
      if (wr[r]) written[r] += n;
      if (hd[r]) kept[r] += n;
    }
    free(wr);
    free(hd);
  }
  for (int r = 0; r < W; ++r) discarded[r] = written[r] - kept[r];
  out64[0] = reduced;
  out64[1] = owner_elems;
  out32[0] = n_tasks;
  out32[1] = owner_tasks;
}

/* ------------------------------------------------------------------------ */
/* ReduceScatter ([AG] duality with ReduceScatter: M in, M/N out, a       */
/* reduction plus a split).  Shard s is columns [s*L, (s+1)*L), L = M/W.     */
/* ------------------------------------------------------------------------ */
void or_reduce_scatter(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                       int64_t ld_out, int64_t M, int32_t pre_div) {
  int64_t L = M / W;
  for (int s = 0; s < W; ++s) {
    for (int64_t k = 0; k < L; ++k) {
      float acc = 0.0f;
      for (int r = 0; r < W; ++r) {
        float v = contribution(dtype, load_val(dtype, in, ld_in, r, s * L + k), pre_div, W);
        acc = (r == 0) ? v : acc + v;
      }
      store_val(dtype, out, ld_out, s, k, acc);
    }
  }
}

/* Ring reduce-scatter, simulated as a ring passes partial sums ([AG] the
 * ring all-reduce is reduce-scatter followed by all-gather; the ring
 * reduce-scatter is the all-gather's data flow reversed with a reduction,
 * per the duality table).  W-1 steps; at step s (s = 0..W-2) node i sends
 * its partial sum of chunk (i - s) mod W to node i+1, which adds its own
 * contribution (pre-divided as in the flush) and keeps the result as its
 * partial of that chunk.  Chunk c starts at node c, so its sum is folded in
 * rank order c, c+1, ..., c-1 (mod W); it is complete at node c-1 after the
 * last step.  out[c][k] = the completed chunk c (rank-order shard layout). */
void or_reduce_scatter_ring(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                            int64_t ld_out, int64_t M, int32_t pre_div) {
  int64_t L = M / W;
  /* partial[i][c*L + k]: node i's running sum of chunk c */
  float* partial = (float*)malloc(sizeof(float) * (size_t)(W * (M > 0 ? M : 1)));
  float* msg = (float*)malloc(sizeof(float) * (size_t)(W * (L > 0 ? L : 1)));
  for (int i = 0; i < W; ++i)
    for (int64_t j = 0; j < M; ++j)
      partial[(int64_t)i * M + j] = contribution(dtype, load_val(dtype, in, ld_in, i, j), pre_div, W);
  for (int step = 0; step < W - 1; ++step) {
    /* every node sends first (messages), then every node adds */
    for (int i = 0; i < W; ++i) {
      int c = ((i - step) % W + W) % W;
      for (int64_t k = 0; k < L; ++k) msg[(int64_t)i * L + k] = partial[(int64_t)i * M + c * L + k];
    }
    for (int i = 0; i < W; ++i) {
      int src = (i - 1 + W) % W;
      int c = ((src - step) % W + W) % W;
      for (int64_t k = 0; k < L; ++k) {
        float own = contribution(dtype, load_val(dtype, in, ld_in, i, c * L + k), pre_div, W);
        partial[(int64_t)i * M + c * L + k] = msg[(int64_t)src * L + k] + own;
      }
    }
  }
  for (int c = 0; c < W; ++c) {
    int holder = (c - 1 + W) % W;
    for (int64_t k = 0; k < L; ++k) store_val(dtype, out, ld_out, c, k, partial[(int64_t)holder * M + c * L + k]);
  }
  free(partial);
  free(msg);
}

/* ------------------------------------------------------------------------ */
/* AllGather ([AG] semantic definition; Ring AllGather steps).               */
/* ------------------------------------------------------------------------ */

/* Ring schedule, simulated as the page describes it: node i starts with its
 * own chunk; at every step each node forwards to its right neighbour (i+1)
 * the chunk it received in the previous step (its own one at the first step)
 * and appends the chunk arriving from its left neighbour.
 * order[i*N + p] = the chunk at position p of node i after N-1 steps.
 * sends (optional): (N-1)*N records of {step, src, dst, chunk}. */
void or_ring_ag_schedule(int32_t N, int32_t* order, int32_t* sends) {
  int32_t* last = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  int32_t* incoming = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  for (int i = 0; i < N; ++i) {
    order[(int64_t)i * N + 0] = i;
    last[i] = i;
  }
  int rec = 0;
  for (int step = 1; step < N; ++step) {
    for (int src = 0; src < N; ++src) {
      int dst = (src + 1) % N;
      incoming[dst] = last[src];
      if (sends) {
        sends[rec * 4 + 0] = step;
        sends[rec * 4 + 1] = src;
        sends[rec * 4 + 2] = dst;
        sends[rec * 4 + 3] = last[src];
      }
      ++rec;
    }
    for (int i = 0; i < N; ++i) {
      order[(int64_t)i * N + step] = incoming[i];
      last[i] = incoming[i];
    }
  }
  free(last);
  free(incoming);
}

/* Recursive doubling ([AG] Recursive Doubling AllGather), N a power of two:
 * at step j = 1..log2 N node i swaps everything it holds with node
 * i XOR 2^(j-1).  partner[(j-1)*N + i]; recv_chunks[j-1] = chunks received by
 * each node at step j (in units of M/N); held_chunks[j-1] = chunks held
 * after step j.  Returns the step count, or -1 if N is not a power of two. */
int32_t or_rd_ag_schedule(int32_t N, int32_t* partner, int64_t* recv_chunks, int64_t* held_chunks) {
  if (N < 1 || (N & (N - 1)) != 0) return -1;
  /* held[i*N + c] = 1 if node i holds chunk c */
  char* held = (char*)calloc((size_t)N * N, 1);
  char* next = (char*)calloc((size_t)N * N, 1);
  for (int i = 0; i < N; ++i) held[(int64_t)i * N + i] = 1;
  int steps = 0;
  for (int d = 1; d < N; d <<= 1, ++steps) {
    int64_t recv0 = -1, held0 = -1;
    for (int i = 0; i < N; ++i) {
      int q = i ^ d;
      partner[(int64_t)steps * N + i] = q;
      int64_t recv = 0, cnt = 0;
      for (int c = 0; c < N; ++c) {
        recv += held[(int64_t)q * N + c];
        next[(int64_t)i * N + c] = held[(int64_t)i * N + c] | held[(int64_t)q * N + c];
        cnt += next[(int64_t)i * N + c];
      }
      if (i == 0) {
        recv0 = recv;
        held0 = cnt;
      } else if (recv != recv0 || cnt != held0) {
        recv0 = -2; /* nodes disagree: not a symmetric schedule */
      }
    }
    memcpy(held, next, (size_t)N * N);
    recv_chunks[steps] = recv0;
    held_chunks[steps] = held0;
  }
  free(held);
  free(next);
  return steps;
}

/* Step-by-step AllGather schedules ([AG] Ring AllGather, bidirectional ring,
 * Recursive Doubling AllGather), with every received chunk stored at its own
 * index (so the finished buffer is the rank-order concatenation).  Derives,
 * by simulating the schedule from the start, the transfers of step `step`
 * (1-based) as records {dst node, src node, chunk}; returns their count, or -1
 * when the step does not exist.  algo 0: ring (N-1 steps; every node forwards
 * to its right neighbour the chunk it received last), 1: bidirectional ring
 * (ceil((N-1)/2) steps; the same in both directions at once, a chunk
 * arriving from both sides at the last step taken once), 2: recursive
 * doubling (N a power of two, log2 N steps; node i swaps everything it holds
 * with node i XOR 2^(j-1)). */
int32_t or_ag_step_transfers(int32_t N, int32_t algo, int32_t step, int32_t* rec) {
  int32_t steps = algo == 0 ? N - 1 : algo == 1 ? N / 2 : 0;
  if (algo == 2) {
    if (N < 1 || (N & (N - 1)) != 0) return -1;
    for (int d = 1; d < N; d <<= 1) ++steps;
  }
  if (step < 1 || step > steps) return -1;
  char* held = (char*)calloc((size_t)N * N, 1);
  int32_t* from_left = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  int32_t* from_right = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  int32_t* nl = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  int32_t* nr = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  for (int i = 0; i < N; ++i) {
    held[(int64_t)i * N + i] = 1;
    from_left[i] = from_right[i] = i;
  }
  int32_t n = 0;
  for (int s = 1; s <= step; ++s) {
    n = 0;
    if (algo == 2) {
      int d = 1 << (s - 1);
      char* next = (char*)malloc((size_t)N * N);
      memcpy(next, held, (size_t)N * N);
      for (int i = 0; i < N; ++i) {
        int q = i ^ d;
        for (int c = 0; c < N; ++c)
          if (held[(int64_t)q * N + c] && !held[(int64_t)i * N + c]) {
            next[(int64_t)i * N + c] = 1;
            if (s == step) { rec[n * 3] = i; rec[n * 3 + 1] = q; rec[n * 3 + 2] = c; }
            ++n;
          }
      }
      memcpy(held, next, (size_t)N * N);
      free(next);
    } else {
      for (int i = 0; i < N; ++i) {
        int left = (i - 1 + N) % N, right = (i + 1) % N;
        nl[i] = from_left[left];   /* what the left neighbour forwards right */
        nr[i] = from_right[right]; /* what the right neighbour forwards left */
      }
      for (int i = 0; i < N; ++i) {
        int left = (i - 1 + N) % N, right = (i + 1) % N;
        if (!held[(int64_t)i * N + nl[i]]) {
          held[(int64_t)i * N + nl[i]] = 2;
          if (s == step) { rec[n * 3] = i; rec[n * 3 + 1] = left; rec[n * 3 + 2] = nl[i]; }
          ++n;
        }
        if (algo == 1 && !held[(int64_t)i * N + nr[i]]) {
          held[(int64_t)i * N + nr[i]] = 2;
          if (s == step) { rec[n * 3] = i; rec[n * 3 + 1] = right; rec[n * 3 + 2] = nr[i]; }
          ++n;
        }
      }
      for (int i = 0; i < N; ++i) {
        from_left[i] = nl[i];
        from_right[i] = nr[i];
      }
    }
  }
  free(held);
  free(from_left);
  free(from_right);
  free(nl);
  free(nr);
  return n;
}

/* Apply step `step` of a schedule to an all-gather buffer out[i][c*L + k]:
 * step 0 places every node's own shard (out[i][i*L + k] = in[i][k]); a later
 * step copies each transfer's chunk from the source node's row. */
int32_t or_all_gather_step(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                           int64_t ld_out, int64_t L, int32_t algo, int32_t step) {
  int64_t eb = dtype == OR_BF16 ? 2 : 4;
  if (step == 0) {
    for (int i = 0; i < W; ++i)
      memcpy((char*)out + ((int64_t)i * ld_out + (int64_t)i * L) * eb,
             (const char*)in + ((int64_t)i * ld_in) * eb, (size_t)(L * eb));
    return 0;
  }
  int32_t* rec = (int32_t*)malloc(sizeof(int32_t) * 3 * (size_t)W * W);
  int32_t n = or_ag_step_transfers(W, algo, step, rec);
  for (int32_t t = 0; t < n; ++t) {
    int dst = rec[t * 3], src = rec[t * 3 + 1], c = rec[t * 3 + 2];
    memcpy((char*)out + ((int64_t)dst * ld_out + (int64_t)c * L) * eb,
           (const char*)out + ((int64_t)src * ld_out + (int64_t)c * L) * eb, (size_t)(L * eb));
  }
  free(rec);
  return n;
}

/* order 0 (rank order): out[i][s*L + k] = in[s][k], the concatenation
 * [A_0, ..., A_{N-1}] on every node.  order 1 (ring arrival order): position
 * p of node i holds the chunk the ring schedule above delivers there.
 * step >= 0 writes one position only (chunk `step` in rank order, position
 * `step` in ring order). */
int32_t or_all_gather(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                      int64_t ld_out, int64_t L, int32_t order, int32_t step) {
  int64_t eb = dtype == OR_BF16 ? 2 : 4;
  int32_t* ring = (int32_t*)malloc(sizeof(int32_t) * (size_t)W * W);
  or_ring_ag_schedule(W, ring, NULL);
  for (int i = 0; i < W; ++i) {
    for (int p = 0; p < W; ++p) {
      if (step >= 0 && p != step) continue;
      int src = order == 0 ? p : ring[(int64_t)i * W + p];
      memcpy((char*)out + ((int64_t)i * ld_out + (int64_t)p * L) * eb,
             (const char*)in + ((int64_t)src * ld_in) * eb, (size_t)(L * eb));
    }
  }
  free(ring);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Deferred reduction ([MT] What): replica-local accumulation of    */
/* the unreduced per-micro-batch gradients, then one cross-replica sum.      */
/* ------------------------------------------------------------------------ */

/* acc[r][j] = acc[r][j] + x[r][j]; with init the accumulator starts from a
 * zero tree, so acc = +0.0f + x. */
void or_accumulate(int32_t rows, const float* x, int64_t ld_x, float* acc, int64_t ld_acc,
                   int64_t M, int32_t init) {
  for (int r = 0; r < rows; ++r)
    for (int64_t j = 0; j < M; ++j) {
      float a = init ? 0.0f : acc[r * ld_acc + j];
      acc[r * ld_acc + j] = a + x[r * ld_x + j];
    }
}

/* out[i][j] = fold over replicas r = 0..W-1 of acc[r][j] (fp32, rank order,
 * starting from acc[0][j]) for every output row i < out_rows. */
void or_deferred_reduce(int32_t W, const float* acc, int64_t ld_acc, float* out, int64_t ld_out,
                        int64_t M, int32_t out_rows) {
  for (int64_t j = 0; j < M; ++j) {
    float s = 0.0f;
    for (int r = 0; r < W; ++r) s = (r == 0) ? acc[r * ld_acc + j] : s + acc[r * ld_acc + j];
    for (int i = 0; i < out_rows; ++i) out[i * ld_out + j] = s;
  }
}
