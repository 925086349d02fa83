"""CPU oracle for the gradient-reduction path (numpy front end over liboracle.so).

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's CPU
baseline may import this package; the product (gradient_reduction_amd) never
does.  The C source (oracle.c) shares no code with the GPU library.

Every function works on raw bit patterns for bf16 (uint16 arrays) and on
float32 arrays for fp32, exactly as stored in a [rows, ld] slab.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

BF16 = 0
F32 = 1

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p


def load_library(path):
    """Open an oracle build at `path` and declare its signatures."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    L.or_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.or_bf16_to_f32.restype = ctypes.c_float
    L.or_f32_to_bf16.argtypes = [ctypes.c_float]
    L.or_f32_to_bf16.restype = ctypes.c_uint16
    L.or_f32_to_bf16_array.argtypes = [_vp, _vp, ctypes.c_int64]
    L.or_f32_to_bf16_array.restype = None
    L.or_partition_ids.argtypes = [ctypes.c_int32, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp,
                                       _vp, _vp, ctypes.c_int64]
    L.or_partition_ids.restype = ctypes.c_int64
    L.or_group_eligible.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp]
    L.or_group_eligible.restype = None
    L.or_owner_map.argtypes = [ctypes.c_int32, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp]
    L.or_owner_map.restype = None
    L.or_flush.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int64, _vp,
                               ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, _vp, _vp, _vp, _vp,
                               _vp, _vp, _vp, ctypes.c_int32]
    L.or_flush.restype = None
    L.or_flush_zero2.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int64, _vp,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _vp, _vp, ctypes.c_int32]
    L.or_flush_zero2.restype = None
    L.or_flush_buffers.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                   _vp, _vp, _vp, _vp, ctypes.c_int32]
    L.or_flush_buffers.restype = None
    L.or_relayout_map.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp,
                                  ctypes.c_int64, _vp, _vp]
    L.or_relayout_map.restype = ctypes.c_int64
    L.or_relayout_apply.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int64, _vp,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _vp]
    L.or_relayout_apply.restype = None
    L.or_reduce_scatter_v.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int64, _vp,
                                      ctypes.c_int64, _vp, ctypes.c_int32]
    L.or_reduce_scatter_v.restype = None
    L.or_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp, _vp, _vp, _vp, _vp, _vp]
    L.or_probe.restype = None
    L.or_reduce_scatter.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int64, _vp,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
    L.or_reduce_scatter.restype = None
    L.or_reduce_scatter_ring.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int64, _vp,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
    L.or_reduce_scatter_ring.restype = None
    L.or_ag_step_transfers.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp]
    L.or_ag_step_transfers.restype = ctypes.c_int32
    L.or_all_gather_step.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int64, _vp,
                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    L.or_all_gather_step.restype = ctypes.c_int32
    L.or_ring_ag_schedule.argtypes = [ctypes.c_int32, _vp, _vp]
    L.or_ring_ag_schedule.restype = None
    L.or_rd_ag_schedule.argtypes = [ctypes.c_int32, _vp, _vp, _vp]
    L.or_rd_ag_schedule.restype = ctypes.c_int32
    L.or_all_gather.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int64, _vp,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    L.or_all_gather.restype = ctypes.c_int32
    L.or_accumulate.argtypes = [ctypes.c_int32, _vp, ctypes.c_int64, _vp, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int32]
    L.or_accumulate.restype = None
    L.or_deferred_reduce.argtypes = [ctypes.c_int32, _vp, ctypes.c_int64, _vp, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int32]
    L.or_deferred_reduce.restype = None
    return L


def lib():
    global _lib
    if _lib is None:
        _lib = load_library(os.path.join(_HERE, "liboracle.so"))
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(_vp)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _slab(a, dtype):
    a = np.asarray(a)
    want = np.uint16 if dtype == BF16 else np.float32
    if a.dtype != want and not (dtype == F32 and a.dtype == np.uint32):
        raise TypeError(f"slab dtype {a.dtype} does not match {want}")
    if a.ndim != 2 or not a.flags.c_contiguous:
        raise ValueError("slab must be a C-contiguous [rows, ld] array")
    return a


# -- numbers ---------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (round to nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().or_f32_to_bf16_array(_p(x), _p(out), x.size)
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# -- partition lists and owner map -----------------------------------------

def partition_ids(numel, group_begin, group_parts):
    numel = _c(numel, np.int64)
    gb = _c(group_begin, np.int32)
    gp = _c(group_parts, np.int32)
    P, G = len(numel), len(gp)
    cap = P + int(np.sum(np.maximum(gp - 1, 0))) + 1
    flat = np.zeros(P, np.int64)
    ps = np.zeros(G, np.int64)
    off = np.zeros(P + 1, np.int32)
    pids = np.zeros(cap, np.int32)
    n = lib().or_partition_ids(P, _p(numel), G, _p(gb), _p(gp), _p(flat), _p(ps), _p(off),
                               _p(pids), cap)
    if n < 0:
        raise RuntimeError("pid capacity exceeded")
    return flat, ps, off, pids[:n].copy()


def group_eligible(W, comm_size, rank_to_global):
    cs = _c(comm_size, np.int32)
    r2g = _c(rank_to_global, np.int32).reshape(-1)
    G = len(cs)
    out = np.zeros(G, np.int32)
    lib().or_group_eligible(W, G, _p(cs), _p(r2g), _p(out))
    return out


def owner_map(pid_offsets, pids, group_begin, eligible):
    off = _c(pid_offsets, np.int32)
    pids = _c(pids, np.int32)
    if len(pids) == 0:
        pids = np.zeros(1, np.int32)
    gb = _c(group_begin, np.int32)
    el = _c(eligible, np.int32)
    P, G = len(off) - 1, len(el)
    owner = np.zeros(P, np.int32)
    counts = np.zeros(2 * G, np.int32)
    lib().or_owner_map(P, _p(off), _p(pids), G, _p(gb), _p(el), _p(owner), _p(counts))
    return owner, counts


# -- bucket flushes and the probe ------------------------------------------

def flush(W, dtype, slab_in, slab_out, bucket_col, t_off, t_numel, t_param, t_comm, owner,
          comm_size, comm_stride, pre_div):
    """In place on slab_out (which may be slab_in)."""
    slab_in = _slab(slab_in, dtype)
    slab_out = _slab(slab_out, dtype)
    t_off, t_numel = _c(t_off, np.int64), _c(t_numel, np.int64)
    t_param, t_comm = _c(t_param, np.int32), _c(t_comm, np.int32)
    cs, cst = _c(comm_size, np.int32), _c(comm_stride, np.int32)
    ow = None if owner is None else _c(owner, np.int32)
    lib().or_flush(W, dtype, _p(slab_in), slab_in.shape[1], _p(slab_out), slab_out.shape[1],
                   bucket_col, len(t_off), _p(t_off), _p(t_numel), _p(t_param), _p(t_comm),
                   _p(ow), _p(cs), _p(cst), pre_div)
    return slab_out


def flush_zero2(W, dtype, slab_in, slab_out, bucket_col, t_off, t_numel, t_param, t_comm,
                flat_offset, part_size, comm_size, comm_stride, pre_div):
    """ZeRO-2 flush, in place on slab_out.  part_size[p] = the partition size
    of param p's group, 0 for params that keep AllReduce."""
    slab_in = _slab(slab_in, dtype)
    slab_out = _slab(slab_out, dtype)
    t_off, t_numel = _c(t_off, np.int64), _c(t_numel, np.int64)
    t_param, t_comm = _c(t_param, np.int32), _c(t_comm, np.int32)
    fo, ps = _c(flat_offset, np.int64), _c(part_size, np.int64)
    cs, cst = _c(comm_size, np.int32), _c(comm_stride, np.int32)
    lib().or_flush_zero2(W, dtype, _p(slab_in), slab_in.shape[1], _p(slab_out), slab_out.shape[1],
                         bucket_col, len(t_off), _p(t_off), _p(t_numel), _p(t_param), _p(t_comm),
                         _p(fo), _p(ps), _p(cs), _p(cst), pre_div)
    return slab_out


def flush_buffers(W, dtype, in_arena, in_off, out_arena, out_off, t_numel, t_comm, comm_size,
                  comm_stride, pre_div):
    """Flush straight from per-rank gradient buffers into per-rank grad
    buffers: in_off / out_off are [n_tasks, W] element offsets into the flat
    arenas (out_off -1: that rank's buffer is empty)."""
    arr = np.uint16 if dtype == BF16 else np.float32
    assert in_arena.dtype == arr and out_arena.dtype == arr
    assert in_arena.flags.c_contiguous and out_arena.flags.c_contiguous
    n = len(t_numel)
    in_off = _c(np.asarray(in_off).reshape(n * W), np.int64)
    out_off = _c(np.asarray(out_off).reshape(n * W), np.int64)
    for t in range(n):
        for r in range(W):
            assert 0 <= in_off[t * W + r] and in_off[t * W + r] + t_numel[t] <= in_arena.size
            o = out_off[t * W + r]
            assert o == -1 or (0 <= o and o + t_numel[t] <= out_arena.size)
    lib().or_flush_buffers(W, dtype, _p(in_arena), _p(in_off), _p(out_arena), _p(out_off), n,
                           _p(_c(t_numel, np.int64)), _p(_c(t_comm, np.int32)),
                           _p(_c(comm_size, np.int32)), _p(_c(comm_stride, np.int32)), pre_div)
    return out_arena


def relayout_map(W, t_off, t_numel, t_param, t_comm, flat_offset, part_size, bucket_numel):
    """(dest[bucket_numel], seg_start[W+1]) of the by-destination relayout."""
    t_off, t_numel = _c(t_off, np.int64), _c(t_numel, np.int64)
    t_param, t_comm = _c(t_param, np.int32), _c(t_comm, np.int32)
    fo, ps = _c(flat_offset, np.int64), _c(part_size, np.int64)
    dest = np.zeros(max(bucket_numel, 1), np.int64)
    seg = np.zeros(W + 1, np.int64)
    lib().or_relayout_map(W, len(t_off), _p(t_off), _p(t_numel), _p(t_param), _p(t_comm), _p(fo),
                          _p(ps), bucket_numel, _p(dest), _p(seg))
    return dest[:bucket_numel], seg


def relayout_apply(W, dtype, slab_in, out, bucket_col, bucket_numel, dest):
    slab_in, out = _slab(slab_in, dtype), _slab(out, dtype)
    d = _c(dest, np.int64)
    lib().or_relayout_apply(W, dtype, _p(slab_in), slab_in.shape[1], _p(out), out.shape[1],
                            bucket_col, bucket_numel, _p(d))
    return out


def reduce_scatter_v(W, dtype, slab_in, out, seg_start, pre_div):
    slab_in, out = _slab(slab_in, dtype), _slab(out, dtype)
    seg = _c(seg_start, np.int64)
    lib().or_reduce_scatter_v(W, dtype, _p(slab_in), slab_in.shape[1], _p(out), out.shape[1],
                              _p(seg), pre_div)
    return out


def probe(W, t_numel, t_param, t_comm, owner, pid_offsets, pids, comm_size, comm_stride):
    t_numel = _c(t_numel, np.int64)
    t_param, t_comm = _c(t_param, np.int32), _c(t_comm, np.int32)
    ow = None if owner is None else _c(owner, np.int32)
    off, pids = _c(pid_offsets, np.int32), _c(pids, np.int32)
    if len(pids) == 0:
        pids = np.zeros(1, np.int32)
    cs, cst = _c(comm_size, np.int32), _c(comm_stride, np.int32)
    o64 = np.zeros(2, np.int64)
    o32 = np.zeros(2, np.int32)
    wr, kp, dc = (np.zeros(W, np.int64) for _ in range(3))
    lib().or_probe(W, len(t_numel), _p(t_numel), _p(t_param), _p(t_comm), _p(ow), _p(off),
                   _p(pids), _p(cs), _p(cst), _p(o64), _p(o32), _p(wr), _p(kp), _p(dc))
    return dict(tasks=int(o32[0]), owner_tasks=int(o32[1]), reduced_elems=int(o64[0]),
                owner_elems=int(o64[1]), written=wr, kept=kp, discarded=dc)


def probe_line(rank, flush_no, dtype, pr, pre_div):
    """The probe's one-line report for rank `rank` (kept/discarded of that
    rank; discarded as a share of the reduced elements)."""
    name = "BFloat16" if dtype == BF16 else "Float"
    red = pr["reduced_elems"]
    disc = 100.0 * pr["discarded"][rank] / red if red else 0.0
    oe = 100.0 * pr["owner_elems"] / red if red else 0.0
    return (f"[dc-probe][r{rank}] flushReduceBucket #{flush_no} dtype={name} "
            f"tasks={pr['tasks']} reduced_elems={red} kept_elems={int(pr['kept'][rank])} "
            f"discarded={disc:.1f}% pre_div={pre_div} owner_tasks={pr['owner_tasks']} "
            f"owner_elems={pr['owner_elems']} ({oe:.1f}%)")


def ratio_line(owners, P):
    return f"DeepCompile reduce_to_owner: {owners}/{P} gradients reduce to one rank"


# -- reduce-scatter and all-gather -----------------------------------------

def reduce_scatter(W, dtype, slab_in, out, M, pre_div):
    slab_in, out = _slab(slab_in, dtype), _slab(out, dtype)
    lib().or_reduce_scatter(W, dtype, _p(slab_in), slab_in.shape[1], _p(out), out.shape[1], M,
                            pre_div)
    return out


def reduce_scatter_ring(W, dtype, slab_in, out, M, pre_div):
    slab_in, out = _slab(slab_in, dtype), _slab(out, dtype)
    lib().or_reduce_scatter_ring(W, dtype, _p(slab_in), slab_in.shape[1], _p(out), out.shape[1],
                                 M, pre_div)
    return out


AG_RING, AG_BIDIR, AG_RD = 0, 1, 2


def ag_step_transfers(N, algo, step):
    """[(dst, src, chunk)] of one step, or None if the step does not exist."""
    rec = np.zeros((N * N, 3), np.int32)
    n = lib().or_ag_step_transfers(N, algo, step, _p(rec))
    return None if n < 0 else [tuple(int(v) for v in r) for r in rec[:n]]


def all_gather_step(W, dtype, shards, out, L, algo, step):
    shards, out = _slab(shards, dtype), _slab(out, dtype)
    return lib().or_all_gather_step(W, dtype, _p(shards), shards.shape[1], _p(out), out.shape[1],
                                    L, algo, step)


def ring_ag_schedule(N):
    order = np.zeros((N, N), np.int32)
    sends = np.zeros((max(N - 1, 0) * N, 4), np.int32)
    lib().or_ring_ag_schedule(N, _p(order), _p(sends) if N > 1 else None)
    return order, sends


def rd_ag_schedule(N):
    steps_max = max(1, N.bit_length())
    partner = np.zeros((steps_max, N), np.int32)
    recv = np.zeros(steps_max, np.int64)
    held = np.zeros(steps_max, np.int64)
    s = lib().or_rd_ag_schedule(N, _p(partner), _p(recv), _p(held))
    if s < 0:
        raise ValueError("recursive doubling needs a power-of-two node count")
    return partner[:s], recv[:s], held[:s]


def all_gather(W, dtype, shards, out, L, order, step=-1):
    shards, out = _slab(shards, dtype), _slab(out, dtype)
    lib().or_all_gather(W, dtype, _p(shards), shards.shape[1], _p(out), out.shape[1], L, order,
                        step)
    return out


# -- accumulation and the deferred reduce ----------------------------------

def accumulate(rows, x, acc, M, init):
    x, acc = _slab(x, F32), _slab(acc, F32)
    lib().or_accumulate(rows, _p(x), x.shape[1], _p(acc), acc.shape[1], M, init)
    return acc


def deferred_reduce(W, acc, out, M, out_rows):
    acc, out = _slab(acc, F32), _slab(out, F32)
    lib().or_deferred_reduce(W, _p(acc), acc.shape[1], _p(out), out.shape[1], M, out_rows)
    return out
