"""Helpers for the GPU parity tests: device slabs, the oracle side of a
workload, and sampled checks of full-size runs.

Inputs on both sides come from synth (device generator for the GPU slab,
host generator for the oracle), never from the GPU path's outputs.
"""
import sys

import numpy as np

import oracle
from gradient_reduction_amd import dc
import synth
from synth import workloads as wl

SENTINEL16 = 0x7E7E
SENTINEL32 = 0x7E7E7E7E


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch():
    import torch as t
    return t


def empty_slab(dtype, rows, ld, sentinel=True):
    t = torch()
    if dtype == wl.DT_BF16:
        x = t.empty((rows, ld), dtype=t.int16, device="cuda")
        if sentinel:
            x.fill_(SENTINEL16)
    else:
        x = t.empty((rows, ld), dtype=t.int32, device="cuda")
        if sentinel:
            x.fill_(SENTINEL32)
    return x


def gen_slab(dtype, rows, ld, ncols, seed, stream0, scale):
    """Device slab filled by the device generator (columns >= ncols hold the
    sentinel)."""
    t = torch()
    x = empty_slab(dtype, rows, ld)
    synth.fill_slab_device(dtype, seed, stream0, scale, rows, ld, ncols, x.data_ptr(),
                           t.cuda.current_stream().cuda_stream)
    return x


def host_slab(dtype, rows, ld, ncols, seed, stream0, scale):
    x = np.zeros((rows, ld), synth.np_dtype(dtype))
    x[:] = SENTINEL16 if dtype == wl.DT_BF16 else SENTINEL32
    for r in range(rows):
        x[r, :ncols] = synth.fill_row(dtype, seed, stream0 + r, scale, 0, ncols)
    if dtype == wl.DT_F32:
        return x.view(np.float32)
    return x


def to_host(x, dtype):
    a = x.cpu().numpy()
    return a.view(np.uint16) if dtype == wl.DT_BF16 else a.view(np.float32)


def bits(a, dtype):
    return a.view(np.uint16) if dtype == wl.DT_BF16 else a.view(np.uint32)


def oracle_owner(w):
    """Partition CSR and owner map of a flush workload, on the oracle."""
    flat, ps, off, pids = oracle.partition_ids(w.numel, w.group_begin, w.group_parts())
    comm_sizes = [w.comms[c].size for c in w.group_comm]
    elig = oracle.group_eligible(w.W, comm_sizes, w.group_rank_to_global())
    owner, counts = oracle.owner_map(off, pids, w.group_begin, elig)
    return flat, ps, off, pids, owner, counts


def oracle_flush_bucket(w, b, slab_in, slab_out, owner):
    bk = w.buckets[b]
    t_off = [t.offset for t in bk.tasks]
    t_numel = [t.numel for t in bk.tasks]
    t_param = [t.param for t in bk.tasks]
    t_comm = [t.comm for t in bk.tasks]
    oracle.flush(w.W, w.dtype, slab_in, slab_out, bk.col, t_off, t_numel, t_param, t_comm, owner,
                 [c.size for c in w.comms], [c.stride for c in w.comms], w.pre_div)


def psize_per_param(w):
    """ZeRO-2 partition size of each param's group (0 off the DP comm)."""
    flat, ps, off, pids = oracle.partition_ids(w.numel, w.group_begin, w.group_parts())
    comm_sizes = [w.comms[c].size for c in w.group_comm]
    elig = oracle.group_eligible(w.W, comm_sizes, w.group_rank_to_global())
    out = np.zeros(w.P, np.int64)
    for g in range(w.G):
        if elig[g]:
            out[w.group_begin[g]:w.group_begin[g + 1]] = ps[g]
    return flat, out


def oracle_flush_bucket_zero2(w, b, slab_in, slab_out, flat, psize):
    bk = w.buckets[b]
    oracle.flush_zero2(w.W, w.dtype, slab_in, slab_out, bk.col, [t.offset for t in bk.tasks],
                       [t.numel for t in bk.tasks], [t.param for t in bk.tasks],
                       [t.comm for t in bk.tasks], flat, psize, [c.size for c in w.comms],
                       [c.stride for c in w.comms], w.pre_div)


def sample_columns(w, per_bucket=64, seed=0):
    """Columns to check in a full-size flush: both ends of every task in a
    sample of tasks, the bucket edges, and random interior columns."""
    rng = np.random.default_rng(seed)
    cols = set()
    for bk in w.buckets:
        cols.update([bk.col, bk.col + bk.numel - 1])
        idx = rng.choice(len(bk.tasks), size=min(per_bucket, len(bk.tasks)), replace=False)
        for k in idx:
            t = bk.tasks[k]
            if t.numel == 0:
                continue
            a = bk.col + t.offset
            cols.update([a, a + t.numel - 1, a + int(rng.integers(0, t.numel))])
        cols.update((bk.col + rng.integers(0, bk.numel, per_bucket)).tolist())
    return np.array(sorted(c for c in cols if 0 <= c < w.total), np.int64)


def oracle_sampled_flush(w, cols, owner, zero2=False):
    """Oracle outputs [W, len(cols)] of the flush at the given slab columns,
    from host-generated inputs of just those columns (each column becomes a
    one-column task of its parameter; under ZeRO-2 the task's flat offset is
    moved to that column's position in the param)."""
    W = w.W
    n = len(cols)
    scale = w.scale
    rows = np.stack([synth.gather(w.dtype, w.value_seed, r, scale, cols) for r in range(W)])
    if w.dtype == wl.DT_F32:
        rows = rows.view(np.float32)
    ld = max(8, -(-n // 8) * 8)
    slab = np.zeros((W, ld), rows.dtype)
    slab[:, :n] = rows
    out = np.zeros_like(slab)
    if w.dtype == wl.DT_BF16:
        out[:] = SENTINEL16
    else:
        out.view(np.uint32)[:] = SENTINEL32
    # map every column to its task
    t_param, t_comm, t_pos = [], [], []
    starts = [bk.col for bk in w.buckets]
    for c in cols:
        b = int(np.searchsorted(starts, c, side="right")) - 1
        bk = w.buckets[b]
        rel = c - bk.col
        offs = [t.offset for t in bk.tasks]
        k = int(np.searchsorted(offs, rel, side="right")) - 1
        while bk.tasks[k].numel == 0 or not (bk.tasks[k].offset <= rel < bk.tasks[k].offset + bk.tasks[k].numel):
            k -= 1
        t_param.append(bk.tasks[k].param)
        t_comm.append(bk.tasks[k].comm)
        t_pos.append(rel - bk.tasks[k].offset)
    if zero2:
        flat, psize = psize_per_param(w)
        # one pseudo-param per sampled column, at its flat position
        sflat = np.array([flat[p] + e for p, e in zip(t_param, t_pos)], np.int64)
        spsize = np.array([psize[p] for p in t_param], np.int64)
        oracle.flush_zero2(W, w.dtype, slab, out, 0, np.arange(n), np.ones(n), np.arange(n),
                           t_comm, sflat, spsize, [c.size for c in w.comms],
                           [c.stride for c in w.comms], w.pre_div)
    else:
        oracle.flush(W, w.dtype, slab, out, 0, np.arange(n), np.ones(n), t_param, t_comm, owner,
                     [c.size for c in w.comms], [c.stride for c in w.comms], w.pre_div)
    return out[:, :n]


def planned_flush(W, dtype, x, ld_in, y, ld_out, col0, numel, tasks, d_tasks, P, comms, pre,
                  owner=None, flat=None, psize=None):
    """Plan a bucket on the host (dc_plan_flush) and flush it with the plan
    (dc_flush_bucket_planned).  owner / flat / psize are host arrays; their
    device copies are made here.  Returns the device tensors the launch reads."""
    import torch
    tiles, roots = dc.dc_plan_flush(W, dtype, col0, numel, tasks, len(tasks), owner, flat, psize, P,
                                    comms, len(comms))
    keep = [torch.from_numpy(tiles.view(np.uint8).copy()).cuda() if len(tiles) else None]
    d_own = torch.from_numpy(np.asarray(owner, np.int32)).cuda() if owner is not None else None
    d_flat = torch.from_numpy(np.asarray(flat, np.int64)).cuda() if flat is not None else None
    d_ps = torch.from_numpy(np.asarray(psize, np.int64)).cuda() if psize is not None else None
    keep += [d_own, d_flat, d_ps]
    dc.dc_flush_bucket_planned(W, dtype, x, ld_in, y, ld_out, col0, numel, d_tasks, len(tasks), d_own,
                               d_flat, d_ps, P, comms, len(comms), pre, keep[0], len(tiles), roots)
    return keep


def fused_flush_full_size(w, planned=True):
    """Per-rank gradient arenas [W, ld] holding each param at a 128-byte
    aligned position with the slab's values, grad-buffer arenas of the same
    layout for the holders, the executor's tables, and every bucket flushed."""
    import torch
    from gradient_reduction_amd import executor
    ex = executor.from_workload(w, reduce_to_owner=True)
    ex.build_owner_map()
    ex.fetch_metadata()
    eb = w.elem_bytes()
    pcol = np.zeros(w.P, np.int64)
    for bk in w.buckets:
        for t in bk.tasks:
            pcol[t.param] = bk.col + t.offset
    pad = 128 // eb
    poff = np.zeros(w.P, np.int64)
    pos = 0
    for p in range(w.P):
        poff[p] = pos
        pos = wl.round_up(pos + w.numel[p], pad)
    ld = wl.round_up(max(pos, 1), 64)
    say("full-size arenas", w.name, "ld", ld)
    d_in = empty_slab(w.dtype, w.W, ld, sentinel=False)
    stream = torch.cuda.current_stream().cuda_stream
    for p in range(w.P):
        if w.numel[p]:
            synth.fill_slab_device(w.dtype, w.value_seed, 0, w.scale, w.W, ld, w.numel[p],
                                   d_in.data_ptr() + int(poff[p]) * eb, stream, col0=int(pcol[p]))
    d_out = empty_slab(w.dtype, w.W, ld)
    hold = np.zeros((w.W, w.P), bool)
    for b, bk in enumerate(w.buckets):
        h = ex.holders(b)
        for k, t in enumerate(bk.tasks):
            hold[:, t.param] |= h[k]
    rows = np.arange(w.W, dtype=np.int64)[:, None] * ld
    in_addr = (d_in.data_ptr() + (rows + poff[None, :]) * eb).astype(np.uint64)
    out_addr = np.where(hold, d_out.data_ptr() + (rows + poff[None, :]) * eb, 0).astype(np.uint64)
    ex.register_buffers(in_addr, out_addr, planned=planned)
    for b in range(len(w.buckets)):
        ex.flush_buffers(b)
    torch.cuda.synchronize()
    return ex, d_out, ld, poff, pcol, hold
