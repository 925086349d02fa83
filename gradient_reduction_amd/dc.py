"""Thin ctypes binding of libdc.so: the functions of include/dc.h, same names,
same arguments.

Marshalling only.  Device pointers may be given as torch tensors (their
data_ptr()) or ints; host arrays as numpy arrays or sequences; `stream` as a
torch stream, a raw hipStream_t int, or None for torch's current stream on the
current device.  Every function raises DCError when the library returns a
non-zero status.  There is no fallback: without libdc.so nothing runs.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdc.so")

DC_OK = 0
DC_ERR_NULL, DC_ERR_ARG, DC_ERR_SHAPE, DC_ERR_ALIGN = 1, 2, 3, 4
DC_ERR_DTYPE, DC_ERR_TASKS, DC_ERR_HIP, DC_ERR_UNSUPPORTED = 5, 6, 7, 8
DC_BF16, DC_F32 = 0, 1
DC_ORDER_RANK, DC_ORDER_RING = 0, 1
DC_SCHED_RING, DC_SCHED_BIDIR, DC_SCHED_RD = 0, 1, 2
DC_MAX_W, DC_MAX_GROUPS, DC_MAX_COMMS = 64, 64, 8

TASK_DTYPE = np.dtype([("offset", "<i8"), ("numel", "<i8"), ("param", "<i4"),
                       ("comm", "<i4"), ("reserved", "<i8")])
COMM_DTYPE = np.dtype([("size", "<i4"), ("stride", "<i4")])
PIECE_DTYPE = np.dtype([("src", "<i8"), ("dst", "<i8"), ("len", "<i8"), ("reserved", "<i8")])
TILE_DTYPE = np.dtype([("first", "<i4"), ("last", "<i4"), ("root", "<i4"), ("flags", "<i4")])


class dc_probe(ctypes.Structure):
    _fields_ = [("tasks", ctypes.c_int32), ("owner_tasks", ctypes.c_int32),
                ("pre_div", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("reduced_elems", ctypes.c_int64), ("owner_elems", ctypes.c_int64),
                ("written", ctypes.c_int64 * DC_MAX_W), ("kept", ctypes.c_int64 * DC_MAX_W),
                ("discarded", ctypes.c_int64 * DC_MAX_W)]


class DCError(RuntimeError):
    def __init__(self, code, fn, msg):
        super().__init__(f"{fn}: status {code}: {msg}")
        self.code = code


_lib = None
_i32, _i64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p

_SIGS = {
    "dc_version": ([], ctypes.c_char_p),
    "dc_strerror": ([_i32], ctypes.c_char_p),
    "dc_last_error": ([], ctypes.c_char_p),
    "dc_partition_ids": ([_i32, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp], _i32),
    "dc_build_owner_map": ([_i32, _i32, _vp, _vp, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp], _i32),
    "dc_validate_tasks": ([_i32, _vp, _i32, _i64, _i32, _vp, _i32], _i32),
    "dc_flush_bucket": ([_i32, _i32, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _i32, _vp, _i32, _vp,
                         _i32, _i32, _vp], _i32),
    "dc_flush_bucket_buffers": ([_i32, _i32, _i64, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _vp], _i32),
    "dc_validate_buffer_tasks": ([_i32, _i32, _vp, _i32, _i64, _vp, _i32, _vp, _vp], _i32),
    "dc_plan_flush_buffers": ([_i32, _i32, _i64, _vp, _i32, _vp, _i32, _vp, _i64, _vp], _i32),
    "dc_plan_flush_buffers_device": ([_i32, _i32, _i64, _vp, _i32, _vp, _i32, _vp, _i64, _vp, _vp],
                                     _i32),
    "dc_flush_bucket_buffers_planned": ([_i32, _i32, _i64, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _vp,
                                         _i64, _vp], _i32),
    "dc_flush_bucket_zero2": ([_i32, _i32, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _i32, _vp, _vp,
                               _i32, _vp, _i32, _i32, _vp], _i32),
    "dc_plan_flush": ([_i32, _i32, _i64, _i64, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _i64,
                       _vp, _vp], _i32),
    "dc_plan_flush_device": ([_i32, _i32, _i64, _i64, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _vp,
                              _i64, _vp, _vp, _vp], _i32),
    "dc_flush_bucket_planned": ([_i32, _i32, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _i32, _vp, _vp,
                                 _vp, _i32, _vp, _i32, _i32, _vp, _i64, _i64, _vp], _i32),
    "dc_probe_flush": ([_i32, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _vp], _i32),
    "dc_holders": ([_i32, _vp, _i32, _i32, _vp, _vp, _vp, _i32, _vp], _i32),
    "dc_param_part_size": ([_i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp], _i32),
    "dc_plan_relayout": ([_i32, _vp, _i32, _vp, _vp, _i32, _vp, _i32, _vp, _vp], _i32),
    "dc_relayout_bucket": ([_i32, _i32, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _i32, _i64, _vp],
                           _i32),
    "dc_plan_relayout_tiles": ([_i32, _i64, _i64, _vp, _i32, _i64, _vp, _i64, _vp], _i32),
    "dc_plan_relayout_tiles_device": ([_i32, _i64, _i64, _vp, _i32, _i64, _vp, _i64, _vp, _vp], _i32),
    "dc_relayout_bucket_planned": ([_i32, _i32, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _i32, _i64,
                                    _vp, _i64, _vp], _i32),
    "dc_reduce_scatter_v": ([_i32, _i32, _vp, _i64, _vp, _i64, _vp, _i32, _vp], _i32),
    "dc_reduce_scatter": ([_i32, _i32, _vp, _i64, _vp, _i64, _i64, _i32, _vp], _i32),
    "dc_reduce_scatter_ring": ([_i32, _i32, _vp, _i64, _vp, _i64, _i64, _i32, _vp], _i32),
    "dc_all_gather_step": ([_i32, _i32, _vp, _i64, _vp, _i64, _i64, _i32, _i32, _vp], _i32),
    "dc_all_gather": ([_i32, _i32, _vp, _i64, _vp, _i64, _i64, _i32, _i32, _vp], _i32),
    "dc_accumulate": ([_i32, _vp, _i64, _vp, _i64, _i64, _i32, _vp], _i32),
    "dc_deferred_reduce": ([_i32, _vp, _i64, _vp, _i64, _i64, _i32, _vp], _i32),
    "dc_accumulate_reduce": ([_i32, _vp, _i64, _vp, _i64, _i32, _i32, _vp, _i64, _i32, _i64, _vp],
                             _i32),
    "dc_round_bf16": ([_vp, _vp, _i64, _vp], _i32),
    "dc_stream_copy": ([_vp, _vp, _i64, _vp], _i32),
    "dc_stream_rows": ([_vp, _i64, _i32, _vp, _i64, _i32, _i64, _vp], _i32),
    "dc_stream_rows_shaped": ([_vp, _i64, _i32, _vp, _i64, _i32, _i64, _i32, _i32, _vp], _i32),
}


def lib():
    """The loaded libdc.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        # torch ships its own HIP runtime under the same soname as the system
        # one libdc is linked against; whichever is loaded first serves the
        # whole process, so load torch's first: the streams and memory handed
        # to libdc are torch's.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _dev(x):
    """Device pointer of a tensor / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _host(x, dtype):
    """Host pointer of a numpy array (converted to `dtype`) or sequence."""
    if x is None:
        return None, None
    a = np.ascontiguousarray(x, dtype=dtype)
    return a.ctypes.data_as(_vp), a


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, rc):
    if rc != DC_OK:
        raise DCError(rc, fn, lib().dc_last_error().decode())


def dc_version():
    return lib().dc_version().decode()


def dc_strerror(status):
    return lib().dc_strerror(status).decode()


def dc_last_error():
    return lib().dc_last_error().decode()


def dc_partition_ids(W, num_params, numel, num_groups, group_begin, group_parts, flat_offset,
                     part_size, pid_offsets, pids, pids_capacity, stream=None):
    gb, _a = _host(group_begin, np.int32)
    gp, _b = _host(group_parts, np.int32)
    _check("dc_partition_ids", lib().dc_partition_ids(
        W, num_params, _dev(numel), num_groups, gb, gp, _dev(flat_offset), _dev(part_size),
        _dev(pid_offsets), _dev(pids), pids_capacity, _stream(stream)))


def dc_build_owner_map(W, num_params, pid_offsets, pids, pids_capacity, num_groups, group_begin,
                       group_comm_size, group_rank_to_global, owner, counts, stream=None):
    gb, _a = _host(group_begin, np.int32)
    cs, _b = _host(group_comm_size, np.int32)
    rg, _c = _host(np.asarray(group_rank_to_global, np.int32).reshape(-1), np.int32)
    _check("dc_build_owner_map", lib().dc_build_owner_map(
        W, num_params, _dev(pid_offsets), _dev(pids), pids_capacity, num_groups, gb, cs, rg,
        _dev(owner), _dev(counts), _stream(stream)))


def dc_validate_tasks(W, tasks, num_tasks, bucket_numel, num_params, comms, num_comms):
    tp, _a = _host(tasks, TASK_DTYPE)
    cp, _b = _host(comms, COMM_DTYPE)
    _check("dc_validate_tasks", lib().dc_validate_tasks(W, tp, num_tasks, bucket_numel,
                                                        num_params, cp, num_comms))


def dc_flush_bucket(W, dtype, slab_in, ld_in, slab_out, ld_out, bucket_col, bucket_numel, tasks,
                    num_tasks, owner, num_params, comms, num_comms, pre_div, stream=None):
    cp, _a = _host(comms, COMM_DTYPE)
    _check("dc_flush_bucket", lib().dc_flush_bucket(
        W, dtype, _dev(slab_in), ld_in, _dev(slab_out), ld_out, bucket_col, bucket_numel,
        _dev(tasks), num_tasks, _dev(owner), num_params, cp, num_comms, pre_div,
        _stream(stream)))


def dc_flush_bucket_buffers(W, dtype, bucket_numel, tasks, num_tasks, in_ptrs, out_ptrs, comms,
                            num_comms, pre_div, stream=None):
    """tasks, in_ptrs, out_ptrs: device tensors (in_ptrs / out_ptrs int64
    [num_tasks * W] holding device addresses, 0 for an empty buffer)."""
    cp, _a = _host(comms, COMM_DTYPE)
    _check("dc_flush_bucket_buffers", lib().dc_flush_bucket_buffers(
        W, dtype, bucket_numel, _dev(tasks), num_tasks, _dev(in_ptrs), _dev(out_ptrs), cp, num_comms,
        pre_div, _stream(stream)))


def dc_plan_flush_buffers(W, dtype, bucket_numel, tasks, num_tasks, comms, num_comms):
    """Host only; returns the fused flush's dc_tile records (TILE_DTYPE)."""
    tp, _a = _host(tasks, TASK_DTYPE)
    cp, _b = _host(comms, COMM_DTYPE)
    n = ctypes.c_int64(0)
    _check("dc_plan_flush_buffers", lib().dc_plan_flush_buffers(
        W, dtype, bucket_numel, tp, num_tasks, cp, num_comms, None, 0, ctypes.byref(n)))
    tiles = np.zeros(max(n.value, 1), TILE_DTYPE)
    _check("dc_plan_flush_buffers", lib().dc_plan_flush_buffers(
        W, dtype, bucket_numel, tp, num_tasks, cp, num_comms, tiles.ctypes.data_as(_vp), n.value,
        ctypes.byref(n)))
    return tiles[:n.value].copy()


def dc_flush_bucket_buffers_planned(W, dtype, bucket_numel, tasks, num_tasks, in_ptrs, out_ptrs,
                                    comms, num_comms, pre_div, tiles, num_tiles, stream=None):
    cp, _a = _host(comms, COMM_DTYPE)
    _check("dc_flush_bucket_buffers_planned", lib().dc_flush_bucket_buffers_planned(
        W, dtype, bucket_numel, _dev(tasks), num_tasks, _dev(in_ptrs), _dev(out_ptrs), cp, num_comms,
        pre_div, _dev(tiles), num_tiles, _stream(stream)))


def dc_validate_buffer_tasks(W, dtype, tasks, num_tasks, bucket_numel, comms, num_comms, in_ptrs,
                             out_ptrs):
    """Host arrays: tasks (TASK_DTYPE), comms, in_ptrs / out_ptrs (uint64
    addresses, 0 = empty buffer)."""
    tp, _a = _host(tasks, TASK_DTYPE)
    cp, _b = _host(comms, COMM_DTYPE)
    ip, _c = _host(in_ptrs, np.uint64)
    op, _d = _host(out_ptrs, np.uint64)
    _check("dc_validate_buffer_tasks", lib().dc_validate_buffer_tasks(
        W, dtype, tp, num_tasks, bucket_numel, cp, num_comms, ip, op))


def dc_flush_bucket_zero2(W, dtype, slab_in, ld_in, slab_out, ld_out, bucket_col, bucket_numel,
                          tasks, num_tasks, flat_offset, part_size, num_params, comms, num_comms,
                          pre_div, stream=None):
    cp, _a = _host(comms, COMM_DTYPE)
    _check("dc_flush_bucket_zero2", lib().dc_flush_bucket_zero2(
        W, dtype, _dev(slab_in), ld_in, _dev(slab_out), ld_out, bucket_col, bucket_numel,
        _dev(tasks), num_tasks, _dev(flat_offset), _dev(part_size), num_params, cp, num_comms,
        pre_div, _stream(stream)))


def dc_probe_flush(W, dtype, tasks, num_tasks, owner, num_params, pid_offsets, pids, comms,
                   num_comms, pre_div):
    """Host-only; returns a dc_probe."""
    tp, _a = _host(tasks, TASK_DTYPE)
    op, _b = _host(owner, np.int32)
    po, _c = _host(pid_offsets, np.int32)
    pp, _d = _host(pids, np.int32) if pids is not None and len(pids) else (None, None)
    cp, _e = _host(comms, COMM_DTYPE)
    out = dc_probe()
    _check("dc_probe_flush", lib().dc_probe_flush(W, dtype, tp, num_tasks, op, num_params, po, pp,
                                                  cp, num_comms, pre_div, ctypes.byref(out)))
    return out


def dc_holders(W, tasks, num_tasks, num_params, pid_offsets, pids, comms, num_comms):
    """Host only; returns a [num_tasks, W] bool array."""
    tp, _a = _host(tasks, TASK_DTYPE)
    po, _b = _host(pid_offsets, np.int32)
    pp, _c = _host(pids, np.int32) if pids is not None and len(pids) else (None, None)
    cp, _d = _host(comms, COMM_DTYPE)
    out = np.zeros((max(num_tasks, 0), W), np.uint8)
    _check("dc_holders", lib().dc_holders(W, tp, num_tasks, num_params, po, pp, cp, num_comms,
                                          out.ctypes.data_as(_vp)))
    return out.astype(bool)


def dc_param_part_size(W, num_params, num_groups, group_begin, group_comm_size,
                       group_rank_to_global, part_size, param_part_size, stream=None):
    gb, _a = _host(group_begin, np.int32)
    cs, _b = _host(group_comm_size, np.int32)
    rg, _c = _host(np.asarray(group_rank_to_global, np.int32).reshape(-1), np.int32)
    _check("dc_param_part_size", lib().dc_param_part_size(
        W, num_params, num_groups, gb, cs, rg, _dev(part_size), _dev(param_part_size),
        _stream(stream)))


def dc_plan_flush(W, dtype, bucket_col, bucket_numel, tasks, num_tasks, owner, flat_offset,
                  part_size, num_params, comms, num_comms):
    """Host only; returns (dc_tile records as TILE_DTYPE, root tile count).
    Asks for the tile count first, then fills an array of that size."""
    tp, _a = _host(tasks, TASK_DTYPE)
    op, _b = _host(owner, np.int32)
    fo, _c = _host(flat_offset, np.int64)
    ps, _d = _host(part_size, np.int64)
    cp, _e = _host(comms, COMM_DTYPE)
    n, r = ctypes.c_int64(0), ctypes.c_int64(0)
    _check("dc_plan_flush", lib().dc_plan_flush(
        W, dtype, bucket_col, bucket_numel, tp, num_tasks, op, fo, ps, num_params, cp, num_comms,
        None, 0, ctypes.byref(n), None))
    tiles = np.zeros(max(n.value, 1), TILE_DTYPE)
    _check("dc_plan_flush", lib().dc_plan_flush(
        W, dtype, bucket_col, bucket_numel, tp, num_tasks, op, fo, ps, num_params, cp, num_comms,
        tiles.ctypes.data_as(_vp), n.value, ctypes.byref(n), ctypes.byref(r)))
    return tiles[:n.value].copy(), r.value


def dc_plan_flush_device(W, dtype, bucket_col, bucket_numel, tasks, num_tasks, owner, flat_offset,
                         part_size, num_params, comms, num_comms, tiles, capacity, root_tiles=None,
                         stream=None):
    """tasks, owner, flat_offset, part_size, tiles, root_tiles: device
    pointers (tensors or ints) or None.  Returns the tile count; with tiles
    None it only asks for it (nothing is launched, no stream is needed)."""
    cp, _a = _host(comms, COMM_DTYPE)
    n = ctypes.c_int64(0)
    s = None if tiles is None and stream is None else _stream(stream)
    _check("dc_plan_flush_device", lib().dc_plan_flush_device(
        W, dtype, bucket_col, bucket_numel, _dev(tasks), num_tasks, _dev(owner), _dev(flat_offset),
        _dev(part_size), num_params, cp, num_comms, _dev(tiles), capacity, ctypes.byref(n),
        _dev(root_tiles), s))
    return n.value


def dc_plan_flush_buffers_device(W, dtype, bucket_numel, tasks, num_tasks, comms, num_comms, tiles,
                                 capacity, stream=None):
    """tasks, tiles: device pointers (tensors or ints) or None.  Returns the
    tile count; with tiles None it only asks for it (nothing is launched)."""
    cp, _a = _host(comms, COMM_DTYPE)
    n = ctypes.c_int64(0)
    s = None if tiles is None and stream is None else _stream(stream)
    _check("dc_plan_flush_buffers_device", lib().dc_plan_flush_buffers_device(
        W, dtype, bucket_numel, _dev(tasks), num_tasks, cp, num_comms, _dev(tiles), capacity,
        ctypes.byref(n), s))
    return n.value


def dc_plan_relayout_tiles_device(dtype, bucket_col, bucket_numel, pieces, num_pieces, out_numel,
                                  tiles, tiles_capacity, stream=None):
    """pieces, tiles: device pointers (tensors or ints) or None.  Returns the
    tile count; with tiles None it only asks for it (nothing is launched)."""
    n = ctypes.c_int64(0)
    s = None if tiles is None and stream is None else _stream(stream)
    _check("dc_plan_relayout_tiles_device", lib().dc_plan_relayout_tiles_device(
        dtype, bucket_col, bucket_numel, _dev(pieces), num_pieces, out_numel, _dev(tiles),
        tiles_capacity, ctypes.byref(n), s))
    return n.value


def dc_flush_bucket_planned(W, dtype, slab_in, ld_in, slab_out, ld_out, bucket_col, bucket_numel,
                            tasks, num_tasks, owner, flat_offset, part_size, num_params, comms,
                            num_comms, pre_div, tiles, num_tiles, root_tiles, stream=None):
    cp, _a = _host(comms, COMM_DTYPE)
    _check("dc_flush_bucket_planned", lib().dc_flush_bucket_planned(
        W, dtype, _dev(slab_in), ld_in, _dev(slab_out), ld_out, bucket_col, bucket_numel,
        _dev(tasks), num_tasks, _dev(owner), _dev(flat_offset), _dev(part_size), num_params, cp,
        num_comms, pre_div, _dev(tiles), num_tiles, root_tiles, _stream(stream)))


def dc_plan_relayout(W, tasks, num_tasks, flat_offset, part_size, num_params):
    """Host only; returns (pieces array, seg_start array).  Asks for the piece
    count first, then fills an array of that size."""
    tp, _a = _host(tasks, TASK_DTYPE)
    fo, _b = _host(flat_offset, np.int64)
    ps, _c = _host(part_size, np.int64)
    seg = np.zeros(W + 1, np.int64)
    n = ctypes.c_int32(0)
    _check("dc_plan_relayout", lib().dc_plan_relayout(
        W, tp, num_tasks, fo, ps, num_params, None, 0, ctypes.byref(n), seg.ctypes.data_as(_vp)))
    pieces = np.zeros(max(n.value, 1), PIECE_DTYPE)
    _check("dc_plan_relayout", lib().dc_plan_relayout(
        W, tp, num_tasks, fo, ps, num_params, pieces.ctypes.data_as(_vp), n.value,
        ctypes.byref(n), seg.ctypes.data_as(_vp)))
    return pieces[:n.value].copy(), seg


def dc_relayout_bucket(W, dtype, slab_in, ld_in, out, ld_out, bucket_col, bucket_numel, pieces,
                       num_pieces, out_numel, stream=None):
    _check("dc_relayout_bucket", lib().dc_relayout_bucket(
        W, dtype, _dev(slab_in), ld_in, _dev(out), ld_out, bucket_col, bucket_numel, _dev(pieces),
        num_pieces, out_numel, _stream(stream)))


def dc_plan_relayout_tiles(dtype, bucket_col, bucket_numel, pieces, num_pieces, out_numel):
    """Host only; returns the int64 tile plan (size query first, then the
    fill)."""
    pp, _a = (None, None) if num_pieces == 0 else _host(pieces, PIECE_DTYPE)
    n = ctypes.c_int64(0)
    _check("dc_plan_relayout_tiles", lib().dc_plan_relayout_tiles(
        dtype, bucket_col, bucket_numel, pp, num_pieces, out_numel, None, 0, ctypes.byref(n)))
    tiles = np.zeros(max(n.value, 1), np.int64)
    _check("dc_plan_relayout_tiles", lib().dc_plan_relayout_tiles(
        dtype, bucket_col, bucket_numel, pp, num_pieces, out_numel, tiles.ctypes.data_as(_vp),
        n.value, ctypes.byref(n)))
    return tiles[:n.value].copy()


def dc_relayout_bucket_planned(W, dtype, slab_in, ld_in, out, ld_out, bucket_col, bucket_numel,
                               pieces, num_pieces, out_numel, tiles, num_tiles, stream=None):
    _check("dc_relayout_bucket_planned", lib().dc_relayout_bucket_planned(
        W, dtype, _dev(slab_in), ld_in, _dev(out), ld_out, bucket_col, bucket_numel, _dev(pieces),
        num_pieces, out_numel, _dev(tiles), num_tiles, _stream(stream)))


def dc_reduce_scatter_v(W, dtype, in_, ld_in, out, ld_out, seg_start, pre_div, stream=None):
    sp, _a = _host(seg_start, np.int64)
    _check("dc_reduce_scatter_v", lib().dc_reduce_scatter_v(W, dtype, _dev(in_), ld_in, _dev(out),
                                                            ld_out, sp, pre_div, _stream(stream)))


def dc_reduce_scatter(W, dtype, in_, ld_in, out, ld_out, M, pre_div, stream=None):
    _check("dc_reduce_scatter", lib().dc_reduce_scatter(W, dtype, _dev(in_), ld_in, _dev(out),
                                                        ld_out, M, pre_div, _stream(stream)))


def dc_reduce_scatter_ring(W, dtype, in_, ld_in, out, ld_out, M, pre_div, stream=None):
    _check("dc_reduce_scatter_ring", lib().dc_reduce_scatter_ring(
        W, dtype, _dev(in_), ld_in, _dev(out), ld_out, M, pre_div, _stream(stream)))


def dc_all_gather_step(W, dtype, in_, ld_in, out, ld_out, shard_numel, algo, step, stream=None):
    _check("dc_all_gather_step", lib().dc_all_gather_step(
        W, dtype, _dev(in_), ld_in, _dev(out), ld_out, shard_numel, algo, step, _stream(stream)))


def dc_all_gather(W, dtype, in_, ld_in, out, ld_out, shard_numel, order, step, stream=None):
    _check("dc_all_gather", lib().dc_all_gather(W, dtype, _dev(in_), ld_in, _dev(out), ld_out,
                                                shard_numel, order, step, _stream(stream)))


def dc_accumulate(rows, x, ld_x, acc, ld_acc, M, init, stream=None):
    _check("dc_accumulate", lib().dc_accumulate(rows, _dev(x), ld_x, _dev(acc), ld_acc, M, init,
                                                _stream(stream)))


def dc_deferred_reduce(W, acc, ld_acc, out, ld_out, M, out_rows, stream=None):
    _check("dc_deferred_reduce", lib().dc_deferred_reduce(W, _dev(acc), ld_acc, _dev(out), ld_out,
                                                          M, out_rows, _stream(stream)))


def dc_accumulate_reduce(W, x, ld_x, acc, ld_acc, init, keep_acc, out, ld_out, out_rows, M,
                         stream=None):
    _check("dc_accumulate_reduce", lib().dc_accumulate_reduce(
        W, _dev(x), ld_x, _dev(acc), ld_acc, init, keep_acc, _dev(out), ld_out, out_rows, M,
        _stream(stream)))


def dc_round_bf16(in_, out, n, stream=None):
    _check("dc_round_bf16", lib().dc_round_bf16(_dev(in_), _dev(out), n, _stream(stream)))


def dc_stream_copy(src, dst, nbytes, stream=None):
    _check("dc_stream_copy", lib().dc_stream_copy(_dev(src), _dev(dst), nbytes, _stream(stream)))


def dc_stream_rows(src, src_ld_vec, rows_read, dst, dst_ld_vec, rows_written, nvec, stream=None):
    _check("dc_stream_rows", lib().dc_stream_rows(_dev(src), src_ld_vec, rows_read, _dev(dst),
                                                  dst_ld_vec, rows_written, nvec, _stream(stream)))


def dc_stream_rows_shaped(src, src_ld_vec, rows_read, dst, dst_ld_vec, rows_written, nvec, group,
                          cap, stream=None):
    _check("dc_stream_rows_shaped", lib().dc_stream_rows_shaped(
        _dev(src), src_ld_vec, rows_read, _dev(dst), dst_ld_vec, rows_written, nvec, group, cap,
        _stream(stream)))


def tasks_array(tasks):
    """dc_task records from (offset, numel, param, comm) tuples."""
    a = np.zeros(len(tasks), TASK_DTYPE)
    for k, (off, n, p, c) in enumerate(tasks):
        a[k] = (off, n, p, c, 0)
    return a


def comms_array(comms):
    a = np.zeros(len(comms), COMM_DTYPE)
    for k, (size, stride) in enumerate(comms):
        a[k] = (size, stride)
    return a
