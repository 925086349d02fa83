"""Column-block driver of the oracle, for whole-output checks at full size.

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: tests/, smoke() and
bench.py's CPU-baseline leg may use it, the product never does.

It runs the unchanged oracle functions (oracle/__init__.py over oracle.c) on
column ranges in host threads; the oracle's C calls release the GIL.  Every
output column of the flush, the reduce-scatter, the all-gather, the
accumulation and the deferred reduce is a function of that column's inputs
alone (and of the task it belongs to), so running the oracle on disjoint
column blocks in any order writes exactly what one call over the whole range
writes.  tests/test_oracle_columns.py checks that on small cases against one
whole call.

Inputs come from synth's host generator, never from the GPU path.
"""
import concurrent.futures
import os

import numpy as np

import synth
from . import flush, flush_zero2, partition_ids, group_eligible, owner_map, accumulate
from . import deferred_reduce, reduce_scatter, all_gather, BF16, F32

BLOCK = 1 << 18   # columns per block handed to one thread


def nthreads():
    """Host threads for the oracle: the CPUs this process may run on, at
    most 16 (a one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _np_dtype(dtype):
    return np.uint16 if dtype == BF16 else np.float32


def host_rows(w_dtype, seed, stream0, scale, rows, col0, n, stream_of=None):
    """[rows, n] host inputs: row r holds columns [col0, col0 + n) of
    generator stream stream0 + r (or stream_of(r)).  fp32 comes back as
    float32, bf16 as uint16 bit patterns."""
    out = np.empty((rows, max(n, 1)), synth.np_dtype(w_dtype))
    for r in range(rows):
        s = stream_of(r) if stream_of is not None else stream0 + r
        out[r, :n] = synth.fill_row(w_dtype, seed, s, scale, col0, n)
    return out.view(np.float32) if w_dtype == F32 else out


def _deal(items, k):
    lists = [[] for _ in range(k)]
    for i, it in enumerate(items):
        lists[i % k].append(it)
    return [x for x in lists if x]


def task_blocks(tasks, block=BLOCK):
    """Each task (offset, numel, param, comm) cut into column blocks:
    (offset, numel, param, comm, position of the block inside the task)."""
    out = []
    for off, n, p, c in tasks:
        for o in range(0, n, block):
            out.append((off + o, min(block, n - o), p, c, o))
    return out


def owner_of(w):
    """The oracle's owner map of a flush workload."""
    flat, ps, off, pids = partition_ids(w.numel, w.group_begin, w.group_parts())
    comm_sizes = [w.comms[c].size for c in w.group_comm]
    elig = group_eligible(w.W, comm_sizes, w.group_rank_to_global())
    owner, _ = owner_map(off, pids, w.group_begin, elig)
    return owner


def zero2_tables(w):
    """(flat offset of every param in its group, the group's partition size
    or 0 for a group off the data-parallel comm) from the oracle."""
    flat, ps, off, pids = partition_ids(w.numel, w.group_begin, w.group_parts())
    comm_sizes = [w.comms[c].size for c in w.group_comm]
    elig = group_eligible(w.W, comm_sizes, w.group_rank_to_global())
    psize = np.zeros(w.P, np.int64)
    for g in range(w.G):
        if elig[g]:
            psize[w.group_begin[g]:w.group_begin[g + 1]] = ps[g]
    return flat, psize


def flush_blocks(w, hin, hout, tasks, owner=None, zero2=None, pool=None, threads=None,
                 block=BLOCK):
    """The oracle flush of `tasks` (bucket-relative (offset, numel, param,
    comm), columns of hin/hout where column 0 is the bucket's first column),
    in column blocks over host threads.  zero2 = (flat, psize) runs the ZeRO-2
    flush: a block at position o inside its task is a task of its own whose
    param starts o elements further into the group."""
    W = w.W
    cs = [c.size for c in w.comms]
    cst = [c.stride for c in w.comms]
    blocks = task_blocks(tasks, block)
    k = threads or nthreads()

    def run(lst):
        offs = [b[0] for b in lst]
        ns = [b[1] for b in lst]
        cm = [b[3] for b in lst]
        if zero2 is None:
            flush(W, w.dtype, hin, hout, 0, offs, ns, [b[2] for b in lst], cm, owner, cs, cst,
                  w.pre_div)
        else:
            flat, psize = zero2
            fl = np.array([flat[b[2]] + b[4] for b in lst], np.int64)
            ps = np.array([psize[b[2]] for b in lst], np.int64)
            flush_zero2(W, w.dtype, hin, hout, 0, offs, ns, np.arange(len(lst)), cm, fl, ps, cs,
                        cst, w.pre_div)

    parts = _deal(blocks, k)
    if pool is not None:
        list(pool.map(run, parts))
    else:
        with concurrent.futures.ThreadPoolExecutor(k) as p:
            list(p.map(run, parts))
    return hout


def bucket_tasks(bk):
    return [(t.offset, t.numel, t.param, t.comm) for t in bk.tasks]


def flush_bucket(w, b, owner=None, zero2=None, init="zero", pool=None, block=BLOCK):
    """Oracle output [W, n] (raw bits for bf16, float32 for fp32) of bucket
    b of flush workload w, from host-generated inputs.  init: what the output
    holds before the flush: "zero", an int sentinel bit pattern, or "input"
    (an in-place flush: rows it does not write keep the input)."""
    bk = w.buckets[b]
    n = bk.numel
    hin = host_rows(w.dtype, w.value_seed, 0, w.scale, w.W, bk.col, n)
    if isinstance(init, str) and init == "input":
        hout = hin.copy()
    else:
        hout = np.zeros_like(hin)
        if not (isinstance(init, str) and init == "zero"):
            hout.view(np.uint16 if w.dtype == BF16 else np.uint32)[:] = init
    flush_blocks(w, hin, hout, bucket_tasks(bk), owner=owner, zero2=zero2, pool=pool,
                 block=block)
    del hin
    return hout[:, :n]


def deferred_columns(W, seed, scale, K, stream_of, col0, n, pool=None, threads=None,
                     block=1 << 16):
    """Oracle results over columns [col0, col0 + n) of K micro-batches of W
    replicas (micro-batch k, replica r from generator stream stream_of(k, r)):
      acc  [W, n]  the replica-local accumulation (init on the first)
      D    [n]     the deferred reduce of acc
      A    [n]     the status quo: every micro-batch reduced, the reduced
                   gradients accumulated (one row)
    Computed in column blocks over host threads."""
    k_threads = threads or nthreads()
    acc = np.empty((W, max(n, 1)), np.float32)
    D = np.empty((1, max(n, 1)), np.float32)
    A = np.empty((1, max(n, 1)), np.float32)
    # blocks of at most 65536 columns: the host generator then runs each
    # call on the calling thread (it goes parallel on its own only above that)
    blk = min(block, 1 << 16)
    starts = list(range(0, n, blk))

    def run(lst):
        for s in lst:
            m = min(blk, n - s)
            a = np.zeros((W, m), np.float32)
            q = np.zeros((1, m), np.float32)
            for k in range(K):
                x = np.empty((W, m), np.uint32)
                for r in range(W):
                    x[r] = synth.fill_row(F32, seed, stream_of(k, r), scale, col0 + s, m)
                xf = x.view(np.float32)
                accumulate(W, xf, a, m, 1 if k == 0 else 0)
                g = np.zeros((1, m), np.float32)
                deferred_reduce(W, xf, g, m, 1)
                accumulate(1, g, q, m, 1 if k == 0 else 0)
            d = np.zeros((1, m), np.float32)
            deferred_reduce(W, a, d, m, 1)
            acc[:, s:s + m] = a
            D[:, s:s + m] = d
            A[:, s:s + m] = q

    parts = _deal(starts, k_threads)
    if pool is not None:
        list(pool.map(run, parts))
    else:
        with concurrent.futures.ThreadPoolExecutor(k_threads) as p:
            list(p.map(run, parts))
    return acc[:, :n], D[0, :n], A[0, :n]


def reduce_scatter_columns(W, dtype, hin, M, pre_div, threads=None, block=BLOCK):
    """Oracle reduce-scatter [W, M/W] of host slab hin [W, >= M]: shard s
    column k folds column s*L + k of every row.  Shards are computed in
    blocks of k by running the oracle's reduce-scatter on the W-row slab of
    those columns of every shard (a smaller reduce-scatter with the same
    per-column operands)."""
    L = M // W
    out = np.zeros((W, max(L, 1)), hin.dtype)
    starts = list(range(0, L, block))

    def run(lst):
        for s in lst:
            m = min(block, L - s)
            sub = np.empty((W, W * m), hin.dtype)
            for q in range(W):
                sub[:, q * m:(q + 1) * m] = hin[:, q * L + s:q * L + s + m]
            o = np.zeros((W, m), hin.dtype)
            reduce_scatter(W, dtype, sub, o, W * m, pre_div)
            out[:, s:s + m] = o

    k = threads or nthreads()
    with concurrent.futures.ThreadPoolExecutor(k) as p:
        list(p.map(run, _deal(starts, k)))
    return out[:, :L]


def all_gather_rows(W, dtype, shards, L, order):
    """Oracle all-gather [W, W*L] of shards [W, >= L] (rank or ring order)."""
    out = np.zeros((W, max(W * L, 1)), shards.dtype)
    all_gather(W, dtype, np.ascontiguousarray(shards), out, L, order, -1)
    return out[:, :W * L]
