"""The C ABI on the host (no GPU): every symbol of include/dc.h is exported,
every argument check returns its documented code before any device work, and
the host-only probe and task check agree with the oracle."""
import ctypes
import os
import random
import re

import numpy as np
import pytest

import oracle
from gradient_reduction_amd import dc
from synth import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "dc.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dc_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert "dc_flush_bucket" in names and len(names) >= 14
    lib = ctypes.CDLL(dc.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(dc._SIGS), "binding and header disagree"


def test_task_record_layout():
    assert dc.TASK_DTYPE.itemsize == 32 and dc.COMM_DTYPE.itemsize == 8
    assert ctypes.sizeof(dc.dc_probe) == 4 * 4 + 2 * 8 + 3 * 64 * 8


def expect(code, fn, *args, **kw):
    with pytest.raises(dc.DCError) as e:
        fn(*args, **kw)
    assert e.value.code == code, str(e.value)
    assert dc.dc_last_error() != ""


FAKE = 1 << 40          # an aligned address nothing dereferences: every call below fails its checks first
TASK_PTR = FAKE + 4096


def test_flush_argument_checks():
    f = dc.dc_flush_bucket
    ok = dict(W=8, dtype=0, slab_in=FAKE, ld_in=64, slab_out=FAKE, ld_out=64, bucket_col=0,
              bucket_numel=64, tasks=TASK_PTR, num_tasks=1, owner=None, num_params=1,
              comms=[(8, 1)], num_comms=1, pre_div=1, stream=0)

    def call(**ch):
        a = dict(ok)
        a.update(ch)
        return f(**a)

    expect(dc.DC_ERR_ARG, call, W=0)
    expect(dc.DC_ERR_ARG, call, W=65)
    expect(dc.DC_ERR_DTYPE, call, dtype=2)
    expect(dc.DC_ERR_NULL, call, slab_in=None)
    expect(dc.DC_ERR_NULL, call, slab_out=None)
    expect(dc.DC_ERR_NULL, call, tasks=None)
    expect(dc.DC_ERR_ALIGN, call, slab_in=FAKE + 2, slab_out=FAKE + 4098)
    expect(dc.DC_ERR_ALIGN, call, ld_in=60, ld_out=60, bucket_numel=60)
    expect(dc.DC_ERR_SHAPE, call, bucket_col=10)
    expect(dc.DC_ERR_ARG, call, bucket_numel=-1)
    expect(dc.DC_ERR_ARG, call, pre_div=2)
    expect(dc.DC_ERR_ARG, call, comms=[(4, 1)])
    expect(dc.DC_ERR_ARG, call, comms=[(8, 1), (3, 1)], num_comms=2)
    expect(dc.DC_ERR_ARG, call, comms=[(8, 1), (4, 3)], num_comms=2)
    expect(dc.DC_ERR_ARG, call, comms=[(8, 1)] * 9, num_comms=9)
    expect(dc.DC_ERR_ARG, call, ld_out=128)                        # in place with different ld
    expect(dc.DC_ERR_ARG, call, slab_out=FAKE + 64)                # partial overlap
    # sizes whose products would overflow int64 are refused before any arithmetic
    big = (1 << 62) + 64
    expect(dc.DC_ERR_SHAPE, call, ld_in=big, ld_out=big, slab_out=FAKE << 1)
    expect(dc.DC_ERR_SHAPE, call, bucket_col=(1 << 63) - 8)
    expect(dc.DC_ERR_SHAPE, call, bucket_numel=(1 << 44) + 8)


def test_other_argument_checks():
    expect(dc.DC_ERR_SHAPE, dc.dc_reduce_scatter, 8, 0, FAKE, 64, FAKE << 1, 64, 60, 0, stream=0)
    expect(dc.DC_ERR_ARG, dc.dc_reduce_scatter, 8, 0, FAKE, 64, FAKE + 64, 64, 64, 0, stream=0)
    expect(dc.DC_ERR_SHAPE, dc.dc_reduce_scatter, 8, 0, FAKE, 64, FAKE << 1, 0, 64, 0, stream=0)
    expect(dc.DC_ERR_ARG, dc.dc_all_gather, 4, 1, FAKE, 64, FAKE << 1, 256, 64, 2, -1, stream=0)
    expect(dc.DC_ERR_ARG, dc.dc_all_gather, 4, 1, FAKE, 64, FAKE << 1, 256, 64, 0, 4, stream=0)
    expect(dc.DC_ERR_SHAPE, dc.dc_all_gather, 4, 1, FAKE, 64, FAKE << 1, 200, 64, 0, -1, stream=0)
    rr = dc.dc_reduce_scatter_ring
    expect(dc.DC_ERR_SHAPE, rr, 8, 0, FAKE, 64, FAKE << 1, 64, 60, 0, stream=0)
    expect(dc.DC_ERR_ARG, rr, 8, 0, FAKE, 64, FAKE + 64, 64, 64, 0, stream=0)
    expect(dc.DC_ERR_ARG, rr, 8, 0, FAKE, 64, FAKE << 1, 64, 64, 2, stream=0)
    st = dc.dc_all_gather_step
    expect(dc.DC_ERR_ARG, st, 4, 1, FAKE, 64, FAKE << 1, 256, 64, 3, 1, stream=0)
    expect(dc.DC_ERR_ARG, st, 4, 1, FAKE, 64, FAKE << 1, 256, 64, dc.DC_SCHED_RING, 4, stream=0)
    expect(dc.DC_ERR_ARG, st, 4, 1, FAKE, 64, FAKE << 1, 256, 64, dc.DC_SCHED_BIDIR, 3, stream=0)
    expect(dc.DC_ERR_ARG, st, 5, 1, FAKE, 64, FAKE << 1, 320, 64, dc.DC_SCHED_BIDIR, 3, stream=0)
    expect(dc.DC_ERR_ARG, st, 6, 1, FAKE, 64, FAKE << 1, 384, 64, dc.DC_SCHED_RD, 1, stream=0)
    expect(dc.DC_ERR_ARG, st, 8, 1, FAKE, 64, FAKE << 1, 512, 64, dc.DC_SCHED_RD, 4, stream=0)
    expect(dc.DC_ERR_ARG, st, 4, 1, FAKE, 64, FAKE << 1, 256, 64, dc.DC_SCHED_RING, -1, stream=0)
    expect(dc.DC_ERR_SHAPE, st, 4, 1, FAKE, 64, FAKE << 1, 200, 64, dc.DC_SCHED_RING, 0, stream=0)
    expect(dc.DC_ERR_ARG, dc.dc_accumulate, 0, FAKE, 64, FAKE << 1, 64, 64, 0, stream=0)
    expect(dc.DC_ERR_ARG, dc.dc_accumulate, 2, FAKE, 64, FAKE, 128, 64, 0, stream=0)
    expect(dc.DC_ERR_ALIGN, dc.dc_accumulate, 2, FAKE, 66, FAKE << 1, 64, 64, 0, stream=0)
    expect(dc.DC_ERR_ARG, dc.dc_deferred_reduce, 4, FAKE, 64, FAKE << 1, 64, 64, 2, stream=0)
    expect(dc.DC_ERR_ARG, dc.dc_deferred_reduce, 4, FAKE, 64, FAKE + 128, 64, 64, 1, stream=0)
    expect(dc.DC_ERR_SHAPE, dc.dc_stream_copy, FAKE, FAKE << 1, 100, stream=0)
    ar = dc.dc_accumulate_reduce
    expect(dc.DC_ERR_ARG, ar, 4, FAKE, 64, FAKE << 1, 64, 0, 0, FAKE << 2, 64, 2, 64, stream=0)
    expect(dc.DC_ERR_ARG, ar, 4, FAKE, 64, FAKE << 1, 64, 2, 0, FAKE << 2, 64, 1, 64, stream=0)
    expect(dc.DC_ERR_ARG, ar, 4, FAKE, 64, FAKE << 1, 64, 0, 1, FAKE << 1, 64, 4, 64, stream=0)
    expect(dc.DC_ERR_ARG, ar, 4, FAKE, 64, FAKE << 1, 64, 0, 0, FAKE + 256, 64, 1, 64, stream=0)
    expect(dc.DC_ERR_ALIGN, ar, 4, FAKE, 62, FAKE << 1, 64, 0, 0, FAKE << 2, 64, 1, 60, stream=0)
    expect(dc.DC_ERR_UNSUPPORTED, dc.dc_stream_rows, FAKE, 64, 3, FAKE << 1, 64, 1, 64, stream=0)
    expect(dc.DC_ERR_UNSUPPORTED, dc.dc_stream_rows, FAKE, 64, 8, FAKE << 1, 64, 2, 64, stream=0)
    expect(dc.DC_ERR_SHAPE, dc.dc_stream_rows, FAKE, 32, 8, FAKE << 1, 64, 1, 64, stream=0)
    # the plain reference takes W rows to 1 or W; the shaped one also 1 to many and 8 to 4
    expect(dc.DC_ERR_UNSUPPORTED, dc.dc_stream_rows, FAKE, 64, 1, FAKE << 1, 64, 8, 64, stream=0)
    expect(dc.DC_ERR_UNSUPPORTED, dc.dc_stream_rows, FAKE, 64, 8, FAKE << 1, 64, 4, 64, stream=0)
    sh = dc.dc_stream_rows_shaped
    expect(dc.DC_ERR_UNSUPPORTED, sh, FAKE, 64, 2, FAKE << 1, 64, 1, 64, 1, 0, stream=0)
    expect(dc.DC_ERR_UNSUPPORTED, sh, FAKE, 64, 1, FAKE << 1, 64, 2, 64, 1, 0, stream=0)
    expect(dc.DC_ERR_UNSUPPORTED, sh, FAKE, 64, 4, FAKE << 1, 64, 2, 64, 1, 0, stream=0)
    expect(dc.DC_ERR_UNSUPPORTED, sh, FAKE, 64, 8, FAKE << 1, 64, 1, 64, 3, 0, stream=0)
    expect(dc.DC_ERR_ARG, sh, FAKE, 64, 8, FAKE << 1, 64, 1, 64, 1, 65, stream=0)
    expect(dc.DC_ERR_SHAPE, sh, FAKE, 32, 1, FAKE << 1, 64, 8, 64, 1, 0, stream=0)
    expect(dc.DC_ERR_ARG, sh, FAKE, 64, 8, FAKE + 1024, 64, 4, 64, 2, 8, stream=0)
    expect(dc.DC_ERR_ARG, dc.dc_stream_rows, FAKE, 64, 8, FAKE + 1024, 64, 1, 64, stream=0)
    expect(dc.DC_ERR_ARG, dc.dc_stream_copy, FAKE, FAKE + 16, 64, stream=0)
    huge = 1 << 60
    expect(dc.DC_ERR_SHAPE, dc.dc_all_gather, 8, 0, FAKE, huge, FAKE << 1, huge, huge, 0, -1, stream=0)
    expect(dc.DC_ERR_SHAPE, dc.dc_all_gather_step, 8, 0, FAKE, huge, FAKE << 1, huge, huge,
           dc.DC_SCHED_RING, 1, stream=0)
    expect(dc.DC_ERR_SHAPE, dc.dc_accumulate, 65535, FAKE, huge, FAKE << 1, huge, 64, 0, stream=0)
    expect(dc.DC_ERR_SHAPE, dc.dc_reduce_scatter, 8, 0, FAKE, huge, FAKE << 1, huge, huge, 0, stream=0)
    expect(dc.DC_ERR_SHAPE, dc.dc_stream_copy, FAKE, FAKE << 1, huge, stream=0)
    expect(dc.DC_ERR_SHAPE, dc.dc_stream_rows, FAKE, huge, 8, FAKE << 1, 64, 1, 64, stream=0)
    expect(dc.DC_ERR_SHAPE, dc.dc_partition_ids, 4, 3, FAKE, 1, [0, 2], [4], FAKE, FAKE, FAKE,
           FAKE, 10, stream=0)
    expect(dc.DC_ERR_SHAPE, dc.dc_partition_ids, 4, 3, FAKE, 1, [0, 3], [4], FAKE, FAKE, FAKE,
           FAKE, 5, stream=0)
    expect(dc.DC_ERR_ARG, dc.dc_partition_ids, 4, 3, FAKE, 1, [0, 3], [0], FAKE, FAKE, FAKE,
           FAKE, 10, stream=0)
    expect(dc.DC_ERR_ARG, dc.dc_build_owner_map, 4, 3, FAKE, FAKE, 10, 0, [0], [4], [0, 1, 2, 3],
           FAKE, FAKE, stream=0)


def test_validate_tasks():
    comms = [(8, 1), (4, 1)]
    good = dc.tasks_array([(0, 5, 0, 0), (5, 0, 1, 1), (5, 7, 2, 1)])
    dc.dc_validate_tasks(8, good, 3, 12, 3, comms, 2)
    for bad, n in ((dc.tasks_array([(1, 5, 0, 0)]), 6), (dc.tasks_array([(0, 5, 0, 0), (4, 1, 1, 0)]), 6),
                   (dc.tasks_array([(0, 5, 3, 0)]), 5), (dc.tasks_array([(0, 5, 0, 2)]), 5),
                   (dc.tasks_array([(0, -1, 0, 0)]), -1), (dc.tasks_array([(0, 5, 0, 0)]), 6)):
        expect(dc.DC_ERR_TASKS, dc.dc_validate_tasks, 8, bad, len(bad), n, 3, comms, 2)


def test_probe_matches_oracle_on_workloads():
    """dc_probe_flush is host code: compare it with the oracle's probe on the
    synthetic workloads and random ones (owner path on and off)."""
    ws = [wl.tiny_flush(), wl.owner_flush_w8(), wl.owner_flush_w8_layered(), wl.mixed_flush_w16()]
    rng = random.Random(3)
    for k in range(5):
        W = rng.choice([2, 4, 8, 16])
        sizes = [rng.randint(0, 500) for _ in range(200)]
        ws.append(wl.custom_flush(f"r{k}", W, 0, sizes, group_begin=[0, 120, 200],
                                  group_comm=[0, 1], comms=[wl.Comm(W, 1), wl.Comm(W // 2, 2)],
                                  capacity=3000))
    for w in ws:
        flat, ps, off, pids = oracle.partition_ids(w.numel, w.group_begin, w.group_parts())
        comm_sizes = [w.comms[c].size for c in w.group_comm]
        elig = oracle.group_eligible(w.W, comm_sizes, w.group_rank_to_global())
        owner, _ = oracle.owner_map(off, pids, w.group_begin, elig)
        comms = [(c.size, c.stride) for c in w.comms]
        for own in (None, owner):
            for bk in w.buckets:
                t = dc.tasks_array([(x.offset, x.numel, x.param, x.comm) for x in bk.tasks])
                pr = dc.dc_probe_flush(w.W, w.dtype, t, len(t), own, w.P, off, pids, comms,
                                       len(comms), w.pre_div)
                want = oracle.probe(w.W, t["numel"], t["param"], t["comm"], own, off, pids,
                                    [c[0] for c in comms], [c[1] for c in comms])
                assert pr.reduced_elems == want["reduced_elems"]
                assert (pr.owner_tasks, pr.owner_elems) == (want["owner_tasks"], want["owner_elems"])
                assert list(pr.kept)[:w.W] == list(want["kept"])
                assert list(pr.written)[:w.W] == list(want["written"])
                assert list(pr.discarded)[:w.W] == list(want["discarded"])


def _dest_from_pieces(pieces, n):
    dest = np.full(n, -1, np.int64)
    for pc in pieces:
        dest[pc["src"]:pc["src"] + pc["len"]] = np.arange(pc["dst"], pc["dst"] + pc["len"])
    return dest


def test_plan_relayout_matches_oracle():
    """The host relayout planner against the oracle's element-by-element
    relayout map, on the synthetic workloads and random ones."""
    ws = [wl.tiny_flush(), wl.owner_flush_w8(), wl.owner_flush_w8_layered(), wl.mixed_flush_w16()]
    rng = random.Random(4)
    for k in range(6):
        W = rng.choice([2, 3, 4, 8])
        sizes = [rng.randint(0, 300) for _ in range(150)]
        ws.append(wl.custom_flush(f"r{k}", W, 0, sizes, group_begin=[0, 90, 150],
                                  group_comm=[0, 0], comms=[wl.Comm(W, 1)], capacity=2500))
    for w in ws:
        flat, ps, off, pids = oracle.partition_ids(w.numel, w.group_begin, w.group_parts())
        comm_sizes = [w.comms[c].size for c in w.group_comm]
        elig = oracle.group_eligible(w.W, comm_sizes, w.group_rank_to_global())
        psize = np.zeros(w.P, np.int64)
        for g in range(w.G):
            if elig[g]:
                psize[w.group_begin[g]:w.group_begin[g + 1]] = ps[g]
        for bk in w.buckets[:8]:
            t = dc.tasks_array([(x.offset, x.numel, x.param, x.comm) for x in bk.tasks])
            pieces, seg = dc.dc_plan_relayout(w.W, t, len(t), flat, psize, w.P)
            assert np.all(np.diff(pieces["dst"]) > 0) if len(pieces) > 1 else True
            dest, oseg = oracle.relayout_map(w.W, t["offset"], t["numel"], t["param"], t["comm"],
                                             flat, psize, bk.numel)
            assert np.array_equal(seg, oseg), w.name
            assert np.array_equal(_dest_from_pieces(pieces, bk.numel), dest), w.name


def test_plan_relayout_errors():
    t = dc.tasks_array([(0, 10, 0, 0), (10, 10, 1, 0)])
    # partition index past W
    expect(dc.DC_ERR_TASKS, dc.dc_plan_relayout, 2, t, 2, [0, 10], [4, 4], 2)
    # too few slots
    seg = np.zeros(3, np.int64)
    n = ctypes.c_int32(0)
    rc = dc.lib().dc_plan_relayout(2, t.ctypes.data_as(ctypes.c_void_p), 2,
                                   np.array([0, 10], np.int64).ctypes.data_as(ctypes.c_void_p),
                                   np.array([10, 10], np.int64).ctypes.data_as(ctypes.c_void_p), 2,
                                   np.zeros(1, dc.PIECE_DTYPE).ctypes.data_as(ctypes.c_void_p), 1,
                                   ctypes.byref(n), seg.ctypes.data_as(ctypes.c_void_p))
    assert rc == dc.DC_ERR_SHAPE and n.value == 2


def test_flush_buffers_argument_checks():
    f = dc.dc_flush_bucket_buffers
    expect(dc.DC_ERR_NULL, f, 4, 0, 64, None, 1, FAKE, FAKE, [(4, 1)], 1, 0, stream=0)
    expect(dc.DC_ERR_NULL, f, 4, 0, 64, TASK_PTR, 1, None, FAKE, [(4, 1)], 1, 0, stream=0)
    expect(dc.DC_ERR_ARG, f, 4, 0, -1, TASK_PTR, 1, FAKE, FAKE, [(4, 1)], 1, 0, stream=0)
    expect(dc.DC_ERR_ARG, f, 4, 0, 64, TASK_PTR, 1, FAKE, FAKE, [(4, 1)], 1, 3, stream=0)
    expect(dc.DC_ERR_ARG, f, 4, 0, 64, TASK_PTR, 1, FAKE, FAKE, [(2, 1)], 1, 0, stream=0)
    expect(dc.DC_ERR_DTYPE, f, 4, 7, 64, TASK_PTR, 1, FAKE, FAKE, [(4, 1)], 1, 0, stream=0)


def _buffer_tables(W, numel, gap_in=64, gap_out=64):
    """Disjoint fake addresses: in buffers then out buffers, 16-byte aligned."""
    n = len(numel)
    tin = np.zeros((n, W), np.uint64)
    tout = np.zeros((n, W), np.uint64)
    pos = FAKE
    for t in range(n):
        for r in range(W):
            tin[t, r] = pos
            pos += numel[t] * 2 + gap_in
    for t in range(n):
        for r in range(W):
            tout[t, r] = pos
            pos += numel[t] * 2 + gap_out
    return tin, tout


def test_validate_buffer_tasks():
    W = 4
    numel = [10, 0, 7]
    tasks = dc.tasks_array([(0, 10, 0, 0), (10, 0, 1, 0), (16, 7, 2, 1)])
    comms = [(4, 1), (2, 1)]
    tin, tout = _buffer_tables(W, numel)
    v = dc.dc_validate_buffer_tasks
    v(W, 0, tasks, 3, 23, comms, 2, tin.ravel(), tout.ravel())
    # empty buffers and the in-place pair are fine
    t2 = tout.copy()
    t2[0, 1:] = 0
    t2[2] = tin[2]
    v(W, 0, tasks, 3, 23, comms, 2, tin.ravel(), t2.ravel())
    # ranks may share one input buffer (identical gradients on every rank)
    ti = tin.copy()
    ti[0, :] = tin[0, 0]
    v(W, 0, tasks, 3, 23, comms, 2, ti.ravel(), tout.ravel())
    # failures
    bad = dc.tasks_array([(0, 10, 0, 0), (10, 0, 1, 0), (9, 7, 2, 1)])
    expect(dc.DC_ERR_TASKS, v, W, 0, bad, 3, 23, comms, 2, tin.ravel(), tout.ravel())
    expect(dc.DC_ERR_TASKS, v, W, 0, tasks, 3, 22, comms, 2, tin.ravel(), tout.ravel())
    bad = dc.tasks_array([(0, 10, 0, 0), (10, 0, 1, 0), (16, 7, 2, 2)])
    expect(dc.DC_ERR_TASKS, v, W, 0, bad, 3, 23, comms, 2, tin.ravel(), tout.ravel())
    t3 = tin.copy()
    t3[2, 3] = 0
    expect(dc.DC_ERR_TASKS, v, W, 0, tasks, 3, 23, comms, 2, t3.ravel(), tout.ravel())
    t4 = tout.copy()
    t4[2, 1] = tout[2, 0] + 2        # two outputs overlap
    expect(dc.DC_ERR_TASKS, v, W, 0, tasks, 3, 23, comms, 2, tin.ravel(), t4.ravel())
    t5 = tout.copy()
    t5[0, 2] = tin[0, 3] + 4         # an output inside another rank's input
    expect(dc.DC_ERR_TASKS, v, W, 0, tasks, 3, 23, comms, 2, tin.ravel(), t5.ravel())
    t6 = tout.copy()
    t6[0, 2] = tin[0, 2] + 2         # shifted in place: overlaps its own input
    expect(dc.DC_ERR_TASKS, v, W, 0, tasks, 3, 23, comms, 2, tin.ravel(), t6.ravel())
    # packed back to back for 2-byte elements: fine in bf16, overlapping in fp32
    pin, pout = _buffer_tables(W, numel, 0, 0)
    v(W, 0, tasks, 3, 23, comms, 2, pin.ravel(), pout.ravel())
    expect(dc.DC_ERR_TASKS, v, W, 1, tasks, 3, 23, comms, 2, pin.ravel(), pout.ravel())


def _host_executor(w):
    """An executor built on the CPU, its partition lists set from the oracle
    (the device kernels that build them need a GPU)."""
    from gradient_reduction_amd import executor
    ex = executor.from_workload(w, reduce_to_owner=True, device="cpu")
    flat, ps, off, pids = oracle.partition_ids(w.numel, w.group_begin, w.group_parts())
    comm_sizes = [w.comms[c].size for c in w.group_comm]
    elig = oracle.group_eligible(w.W, comm_sizes, w.group_rank_to_global())
    owner, _ = oracle.owner_map(off, pids, w.group_begin, elig)
    ex.h_owner, ex.h_pid_off, ex.h_pids = owner, off, pids
    return ex


def test_holders_match_oracle():
    """dc_holders against the holder sets written out from the oracle's
    partition lists (rank r holds a param when its partition -- its group
    rank in every block of a sub-communicator -- is in the param's list),
    and the kept counts they give against the oracle's probe; the executor
    hands the same mask to the fused flush."""
    ws = [wl.tiny_flush(), wl.mixed_flush_w16(),
          wl.custom_flush("h", 8, 0, [1000, 3, 77, 4096, 5000, 12, 900, 64], group_begin=[0, 5, 8],
                          group_comm=[0, 1], comms=[wl.Comm(8, 1), wl.Comm(4, 2)], capacity=3000)]
    for w in ws:
        flat, ps, off, pids = oracle.partition_ids(w.numel, w.group_begin, w.group_parts())
        comm_sizes = [w.comms[c].size for c in w.group_comm]
        elig = oracle.group_eligible(w.W, comm_sizes, w.group_rank_to_global())
        owner, _ = oracle.owner_map(off, pids, w.group_begin, elig)
        comms = [(c.size, c.stride) for c in w.comms]
        ex = _host_executor(w)
        for b, bk in enumerate(w.buckets):
            t = dc.tasks_array([(x.offset, x.numel, x.param, x.comm) for x in bk.tasks])
            got = dc.dc_holders(w.W, t, len(t), w.P, off, pids, comms, len(comms))
            want = np.zeros((len(t), w.W), bool)
            for k, x in enumerate(bk.tasks):
                c, st = w.comms[x.comm].size, w.comms[x.comm].stride
                for q in pids[off[x.param]:off[x.param + 1]]:
                    for blk in w.comms[x.comm].blocks(w.W):
                        want[k, blk[int(q)]] = True
            assert np.array_equal(got, want), (w.name, b)
            assert np.array_equal(ex.holders(b), want)
            pr = oracle.probe(w.W, t["numel"], t["param"], t["comm"], owner, off, pids,
                              [c for c, _ in comms], [s for _, s in comms])
            kept = (got * t["numel"][:, None]).sum(axis=0)
            assert list(kept) == list(pr["kept"]), (w.name, b)


def test_holders_argument_checks():
    t = dc.tasks_array([(0, 10, 0, 0), (10, 10, 1, 0)])
    off = np.array([0, 1, 3], np.int32)
    pids = np.array([0, 1, 2], np.int32)
    expect(dc.DC_ERR_TASKS, dc.dc_holders, 4, t, 2, 1, off, pids, [(4, 1)], 1)      # param 1 >= 1
    bad = np.array([0, 1, 2, 9], np.int32)
    expect(dc.DC_ERR_TASKS, dc.dc_holders, 4, t, 2, 2, off, bad[[0, 3, 1]], [(4, 1)], 1)  # pid 9
    expect(dc.DC_ERR_ARG, dc.dc_holders, 4, t, 2, 2, off, pids, [(3, 1)], 1)        # comm 0 != W
    assert dc.dc_holders(4, t, 2, 2, off, pids, [(4, 1)], 1).tolist() == [
        [True, False, False, False], [False, True, True, False]]


def test_header_is_plain_c(tmp_path):
    """include/dc.h is a C header: a C99 translation unit that includes it and
    names its types and constants compiles with -pedantic -Werror."""
    import subprocess
    src = tmp_path / "h.c"
    src.write_text('#include "dc.h"\n'
                   "int f(void) {\n"
                   "  dc_task t = {0, 0, 0, 0, 0}; dc_comm c = {1, 1}; dc_probe p; dc_piece q;\n"
                   "  (void)t; (void)c; (void)p; (void)q;\n"
                   "  return DC_OK + DC_BF16 + DC_F32 + DC_MAX_W + DC_SCHED_RD;\n"
                   "}\n")
    r = subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-c",
                        "-I", os.path.join(ROOT, "include"), str(src), "-o",
                        str(tmp_path / "h.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def _brute_plan(W, dtype, col0, numel, tasks, owner, flat, psize):
    """The tile records as the header defines them, from a per-column task
    index: tile b covers vectors [v0 + 64 b, v0 + 64 (b + 1)) clipped to the
    bucket's last vector; records XCD-major."""
    E = 8 if dtype == wl.DT_BF16 else 4
    first_v = col0 // E
    v0 = first_v - first_v % 64
    v_end = -(-(col0 + numel) // E)
    count = -(-(v_end - v0) // 64) if numel > 0 else 0
    tid = np.repeat(np.arange(len(tasks)), tasks["numel"])          # task of each bucket column
    out = np.zeros(count, dc.TILE_DTYPE)
    for b in range(count):
        f_lo = (v0 + 64 * b) * E - col0
        f_hi = (v0 + min(64 * (b + 1), v_end - v0)) * E - col0
        ids = tid[max(f_lo, 0):min(f_hi, numel)]
        first, last = (int(ids.min()), int(ids.max())) if len(ids) else (0, -1)
        root, flags = -1, 0
        whole = first == last and f_lo >= 0 and f_hi <= numel
        if whole:
            k = first
            p, c = int(tasks["param"][k]), int(tasks["comm"][k])
            if c == 0 and flat is not None and psize[p] > 0:
                a = int(flat[p]) - int(tasks["offset"][k])
                q0, q1 = (a + f_lo) // int(psize[p]), (a + f_hi - 1) // int(psize[p])
                if q0 == q1 and 0 <= q0 < W:
                    root = q0
                else:
                    whole = False
            elif c == 0 and owner is not None and 0 <= owner[p] < W:
                root = int(owner[p])
            flags = 1 | (c << 8) if whole else 0
            root = root if whole else -1
        out[b] = (first, last, root, flags)
    # XCD-major: tile b's record at (b mod 8) floor(n/8) + min(b mod 8, n mod 8) + floor(b/8)
    b = np.arange(count)
    r, q, rem = b % 8, count // 8, count % 8
    slot = r * q + np.minimum(r, rem) + b // 8
    assert np.array_equal(np.sort(slot), b)
    placed = np.zeros_like(out)
    placed[slot] = out
    return placed


def test_plan_flush_matches_definition():
    """dc_plan_flush (host code) against the tile records the header
    defines, built from a per-column task index: small and random workloads
    with every bucket-start residue, owner map on and off, and ZeRO-2."""
    ws = [wl.tiny_flush()]
    rng = random.Random(8)
    for k in range(8):
        W = rng.choice([1, 2, 3, 4, 8, 16])
        dtype = rng.choice([wl.DT_BF16, wl.DT_F32])
        sizes = [rng.choice([0, 1, 7, 8, 9, 500, 1023, 1024, 1025, 4000, 9000]) for _ in range(120)]
        ws.append(wl.custom_flush(f"r{k}", W, dtype, sizes, group_begin=[0, 70, 120],
                                  group_comm=[0, 1 if W > 1 else 0],
                                  comms=[wl.Comm(W, 1), wl.Comm(1, W) if W > 1 else wl.Comm(1, 1)],
                                  capacity=rng.choice([3000, 20_000, 10 ** 6])))
    for w in ws:
        flat, ps, off, pids = oracle.partition_ids(w.numel, w.group_begin, w.group_parts())
        comm_sizes = [w.comms[c].size for c in w.group_comm]
        elig = oracle.group_eligible(w.W, comm_sizes, w.group_rank_to_global())
        owner, _ = oracle.owner_map(off, pids, w.group_begin, elig)
        psize = np.zeros(w.P, np.int64)
        for g in range(w.G):
            if elig[g]:
                psize[w.group_begin[g]:w.group_begin[g + 1]] = ps[g]
        comms = [(c.size, c.stride) for c in w.comms]
        for bk in w.buckets[:10]:
            t = dc.tasks_array([(x.offset, x.numel, x.param, x.comm) for x in bk.tasks])
            for col0 in (bk.col, bk.col + rng.randint(1, 15)):
                for own, fl, pz in ((None, None, None), (owner, None, None), (None, flat, psize)):
                    got, roots = dc.dc_plan_flush(w.W, w.dtype, col0, bk.numel, t, len(t), own, fl,
                                                  pz, w.P, comms, len(comms))
                    want = _brute_plan(w.W, w.dtype, col0, bk.numel, t, own, fl, pz)
                    assert np.array_equal(got, want), (w.name, col0, own is None, fl is None)
                    assert roots == int(np.sum(want["root"] >= 0))


def test_plan_flush_headline_tiles_all_whole():
    """On the 402.8M-parameter W=8 bf16 layout every tile lies inside one task
    (tensors and buckets fall on 1024-element steps), and the roots are the
    owners the oracle's owner map names."""
    w = wl.owner_flush_w8()
    _, _, off, pids = oracle.partition_ids(w.numel, w.group_begin, w.group_parts())
    elig = oracle.group_eligible(w.W, [w.comms[c].size for c in w.group_comm], w.group_rank_to_global())
    owner, _ = oracle.owner_map(off, pids, w.group_begin, elig)
    comms = [(c.size, c.stride) for c in w.comms]
    total = 0
    for bk in w.buckets:
        t = dc.tasks_array([(x.offset, x.numel, x.param, x.comm) for x in bk.tasks])
        got, roots = dc.dc_plan_flush(w.W, w.dtype, bk.col, bk.numel, t, len(t), owner, None, None,
                                      w.P, comms, len(comms))
        assert roots == int(np.sum(got["root"] >= 0))
        total += len(got)
        assert np.all(got["flags"] == 1) and np.all(got["first"] == got["last"])
        assert np.array_equal(got["root"], owner[t["param"][got["first"]]])
    assert total * 64 * 8 == sum(bk.numel for bk in w.buckets)


def test_plan_flush_argument_checks():
    t = dc.tasks_array([(0, 10, 0, 0), (10, 10, 1, 0)])
    comms = [(8, 1)]
    expect(dc.DC_ERR_DTYPE, dc.dc_plan_flush, 8, 3, 0, 20, t, 2, None, None, None, 2, comms, 1)
    expect(dc.DC_ERR_TASKS, dc.dc_plan_flush, 8, 0, 0, 21, t, 2, None, None, None, 2, comms, 1)
    expect(dc.DC_ERR_ARG, dc.dc_plan_flush, 8, 0, -1, 20, t, 2, None, None, None, 2, comms, 1)
    expect(dc.DC_ERR_NULL, dc.dc_plan_flush, 8, 0, 0, 20, t, 2, None, [0, 10], None, 2, comms, 1)
    expect(dc.DC_ERR_ARG, dc.dc_plan_flush, 8, 0, 0, 20, t, 2, [0, 1], [0, 10], [3, 3], 2, comms, 1)
    expect(dc.DC_ERR_SHAPE, dc.dc_plan_flush, 8, 0, (1 << 44) + 8, 20, t, 2, None, None, None, 2, comms, 1)
    # too few slots, and the size query
    n = ctypes.c_int64(0)
    big = dc.tasks_array([(0, 5000, 0, 0)])
    args = (8, 0, 0, 5000, big.ctypes.data_as(ctypes.c_void_p), 1, None, None, None, 1,
            dc.comms_array(comms).ctypes.data_as(ctypes.c_void_p), 1)
    # 625 vectors: 10 tiles of 64
    assert dc.lib().dc_plan_flush(*args, None, 0, ctypes.byref(n), None) == dc.DC_OK and n.value == 10
    rc = dc.lib().dc_plan_flush(*args, np.zeros(4, dc.TILE_DTYPE).ctypes.data_as(ctypes.c_void_p), 4,
                                ctypes.byref(n), None)
    assert rc == dc.DC_ERR_SHAPE
    assert dc.TILE_DTYPE.itemsize == 16


def test_plan_flush_device_argument_checks():
    """dc_plan_flush_device's checks, all before any launch: the size query
    launches nothing and needs no stream."""
    f = dc.dc_plan_flush_device
    comms = [(8, 1)]
    ok = dict(W=8, dtype=0, bucket_col=0, bucket_numel=5000, tasks=TASK_PTR, num_tasks=1,
              owner=None, flat_offset=None, part_size=None, num_params=1, comms=comms,
              num_comms=1, tiles=FAKE, capacity=4, stream=0)
    # 625 vectors: 10 tiles of 64; the size query answers without a launch
    assert f(**dict(ok, tiles=None, capacity=0)) == 10
    assert f(**dict(ok, bucket_col=8, tiles=None, capacity=0)) == 10
    assert f(**dict(ok, bucket_numel=0, tiles=None, capacity=0)) == 0
    for code, kw in [(dc.DC_ERR_ARG, dict(W=0)), (dc.DC_ERR_ARG, dict(W=65)),
                     (dc.DC_ERR_DTYPE, dict(dtype=2)),
                     (dc.DC_ERR_ARG, dict(comms=[(4, 1)])), (dc.DC_ERR_NULL, dict(comms=None)),
                     (dc.DC_ERR_ARG, dict(bucket_col=-1)), (dc.DC_ERR_ARG, dict(bucket_numel=-5)),
                     (dc.DC_ERR_SHAPE, dict(bucket_numel=(1 << 44) + 8)),
                     (dc.DC_ERR_ARG, dict(num_tasks=-1)), (dc.DC_ERR_ARG, dict(num_params=-1)),
                     (dc.DC_ERR_NULL, dict(flat_offset=FAKE)),
                     (dc.DC_ERR_NULL, dict(part_size=FAKE)),
                     (dc.DC_ERR_ARG, dict(owner=FAKE, flat_offset=FAKE, part_size=FAKE)),
                     (dc.DC_ERR_SHAPE, dict(capacity=9)),
                     (dc.DC_ERR_NULL, dict(tasks=None, capacity=10))]:
        expect(code, f, **dict(ok, **kw))
    # a NULL count pointer
    cp = dc.comms_array(comms)
    assert dc.lib().dc_plan_flush_device(8, 0, 0, 5000, None, 0, None, None, None, 1,
                                         cp.ctypes.data_as(ctypes.c_void_p), 1, None, 0, None, None,
                                         None) == dc.DC_ERR_NULL


def test_plan_device_variants_argument_checks():
    """The fused-flush and relayout device planners' checks, all before any
    launch; their size queries launch nothing."""
    f = dc.dc_plan_flush_buffers_device
    ok = dict(W=8, dtype=0, bucket_numel=5000, tasks=TASK_PTR, num_tasks=2, comms=[(8, 1)],
              num_comms=1, tiles=FAKE, capacity=2, stream=0)
    # 625 slots of 8: 10 tiles of 64; no tasks, no tiles
    assert f(**dict(ok, tiles=None, capacity=0)) == 10
    assert f(**dict(ok, num_tasks=0, tiles=None, capacity=0)) == 0
    for code, kw in [(dc.DC_ERR_ARG, dict(W=0)), (dc.DC_ERR_DTYPE, dict(dtype=9)),
                     (dc.DC_ERR_ARG, dict(comms=[(4, 1)])), (dc.DC_ERR_ARG, dict(bucket_numel=-1)),
                     (dc.DC_ERR_ARG, dict(num_tasks=-2)),
                     (dc.DC_ERR_SHAPE, dict(bucket_numel=(1 << 44) + 8)),
                     (dc.DC_ERR_SHAPE, dict(capacity=9)),
                     (dc.DC_ERR_NULL, dict(tasks=None, capacity=10))]:
        expect(code, f, **dict(ok, **kw))
    g = dc.dc_plan_relayout_tiles_device
    ok = dict(dtype=1, bucket_col=0, bucket_numel=4096, pieces=TASK_PTR, num_pieces=3,
              out_numel=4096, tiles=FAKE, tiles_capacity=2, stream=0)
    # 1024 vectors of 4: 16 tiles of 64
    assert g(**dict(ok, tiles=None, tiles_capacity=0)) == 16
    assert g(**dict(ok, out_numel=0, tiles=None, tiles_capacity=0)) == 0
    for code, kw in [(dc.DC_ERR_DTYPE, dict(dtype=4)), (dc.DC_ERR_ARG, dict(bucket_col=-1)),
                     (dc.DC_ERR_ARG, dict(out_numel=-1)), (dc.DC_ERR_ARG, dict(num_pieces=-1)),
                     (dc.DC_ERR_SHAPE, dict(out_numel=(1 << 44) + 4)),
                     (dc.DC_ERR_SHAPE, dict(tiles_capacity=15)),
                     (dc.DC_ERR_NULL, dict(pieces=None, tiles_capacity=16))]:
        expect(code, g, **dict(ok, **kw))


def test_flush_planned_argument_checks():
    f = dc.dc_flush_bucket_planned
    ok = dict(W=8, dtype=0, slab_in=FAKE, ld_in=2048, slab_out=FAKE, ld_out=2048, bucket_col=0,
              bucket_numel=2048, tasks=TASK_PTR, num_tasks=1, owner=None, flat_offset=None,
              part_size=None, num_params=1, comms=[(8, 1)], num_comms=1, pre_div=1,
              tiles=TASK_PTR + 4096, num_tiles=4, root_tiles=0, stream=0)

    def call(**ch):
        a = dict(ok)
        a.update(ch)
        return f(**a)

    expect(dc.DC_ERR_SHAPE, call, num_tiles=3)                     # 2048 bf16 columns: 4 tiles
    expect(dc.DC_ERR_SHAPE, call, num_tiles=0)
    expect(dc.DC_ERR_SHAPE, call, bucket_col=8, ld_in=4096, ld_out=4096)   # starts mid-tile: 5 tiles
    expect(dc.DC_ERR_NULL, call, tiles=None)
    expect(dc.DC_ERR_NULL, call, tiles=None, num_tiles=0)             # a bucket with tiles needs a plan
    expect(dc.DC_ERR_ARG, call, num_tiles=-1)
    expect(dc.DC_ERR_ARG, call, root_tiles=5)
    expect(dc.DC_ERR_ARG, call, root_tiles=-1)
    expect(dc.DC_ERR_NULL, call, flat_offset=FAKE)
    expect(dc.DC_ERR_ARG, call, flat_offset=FAKE, part_size=FAKE, owner=FAKE)
    expect(dc.DC_ERR_ARG, call, W=0)
    expect(dc.DC_ERR_NULL, call, slab_in=None)
    expect(dc.DC_ERR_ARG, call, pre_div=2)


def _brute_plan_buffers(dtype, numel, tasks):
    """The fused flush's tile records as the header defines them, from each
    tile's coordinate range, XCD-major."""
    E = 8 if dtype == wl.DT_BF16 else 4
    nslots = -(-numel // E)
    count = -(-nslots // 64) if len(tasks) else 0
    off = tasks["offset"].astype(np.int64)
    out = np.zeros(count, dc.TILE_DTYPE)
    for b in range(count):
        lo, s1 = 64 * b * E, min(64 * (b + 1), nslots)
        hi = min(s1 * E, numel)
        first = max(int(np.searchsorted(off, lo, side="right")) - 1, 0)
        last = int(np.searchsorted(off, hi, side="left")) - 1
        t = tasks[first]
        whole = (last == first and t["comm"] == 0 and t["offset"] % E == 0 and t["offset"] <= lo
                 and s1 * E <= t["offset"] + t["numel"])
        out[b] = (first, last, -1, 1 if whole else 0)
    b = np.arange(count)
    slot = (b % 8) * (count // 8) + np.minimum(b % 8, count % 8) + b // 8
    placed = np.zeros_like(out)
    placed[slot] = out
    return placed


def buffer_plan_cases(seed, count=30):
    """Seeded buffer-coordinate task tables: (W, dtype, bucket_numel, tasks,
    comms), with gaps, empty tasks and offsets on and off slot boundaries."""
    rng = random.Random(seed)
    cases = []
    for _ in range(count):
        W = rng.choice([2, 4, 6, 8, 16])
        dtype = rng.choice([wl.DT_BF16, wl.DT_F32])
        E = 8 if dtype == wl.DT_BF16 else 4
        comms = [(W, 1), (W // 2, 2)]
        rows, pos = [], rng.randint(0, 20)
        for i in range(rng.randint(1, 60)):
            n = rng.choice([0, 1, 7, 8, 63, 64, 500, 1024, 1025, 3000, 20_000])
            rows.append((pos, n, i, rng.choice([0, 0, 0, 1])))
            pos += n + rng.choice([0, 0, 1, 5, 64, 3000])
            if rng.random() < 0.5:
                pos = -(-pos // (4 * E)) * 4 * E
        numel = rows[-1][0] + rows[-1][1] + rng.choice([0, 3, 100])
        cases.append((W, dtype, numel, dc.tasks_array(rows), comms))
    return cases


def test_plan_flush_buffers_matches_definition():
    for k, (W, dtype, numel, t, comms) in enumerate(buffer_plan_cases(12)):
        got = dc.dc_plan_flush_buffers(W, dtype, numel, t, len(t), comms, len(comms))
        want = _brute_plan_buffers(dtype, numel, t)
        assert np.array_equal(got, want), k


def test_plan_flush_buffers_argument_checks():
    comms = [(8, 1)]
    bad = dc.tasks_array([(0, 10, 0, 0), (5, 10, 1, 0)])           # overlapping
    expect(dc.DC_ERR_TASKS, dc.dc_plan_flush_buffers, 8, 0, 20, bad, 2, comms, 1)
    expect(dc.DC_ERR_TASKS, dc.dc_plan_flush_buffers, 8, 0, 12, dc.tasks_array([(0, 13, 0, 0)]), 1,
           comms, 1)
    expect(dc.DC_ERR_TASKS, dc.dc_plan_flush_buffers, 8, 0, 20, dc.tasks_array([(0, 10, 0, 3)]), 1,
           comms, 1)
    expect(dc.DC_ERR_DTYPE, dc.dc_plan_flush_buffers, 8, 5, 20, dc.tasks_array([(0, 10, 0, 0)]), 1,
           comms, 1)
    f = dc.dc_flush_bucket_buffers_planned
    ok = dict(W=8, dtype=0, bucket_numel=2048, tasks=TASK_PTR, num_tasks=1, in_ptrs=FAKE,
              out_ptrs=FAKE, comms=comms, num_comms=1, pre_div=1, tiles=TASK_PTR + 4096,
              num_tiles=4, stream=0)      # 2048 bf16 coordinates: 256 slots, 4 tiles

    def call(**ch):
        a = dict(ok)
        a.update(ch)
        return f(**a)

    expect(dc.DC_ERR_SHAPE, call, num_tiles=3)
    expect(dc.DC_ERR_SHAPE, call, num_tiles=2)
    expect(dc.DC_ERR_NULL, call, tiles=None)
    expect(dc.DC_ERR_NULL, call, in_ptrs=None)
    expect(dc.DC_ERR_ARG, call, pre_div=3)
    expect(dc.DC_ERR_ARG, call, W=0)


def _xcd_major(recs):
    """Records in tile order placed XCD-major (tile b at (b mod 8)
    floor(n/8) + min(b mod 8, n mod 8) + floor(b/8))."""
    n = len(recs)
    b = np.arange(n)
    r, q, rem = b % 8, n // 8, n % 8
    out = np.zeros_like(recs)
    out[r * q + np.minimum(r, rem) + b // 8] = recs
    return out


def _brute_relayout_tiles(dtype, bucket_col, bucket_numel, pieces, out_numel):
    """The relayout tile records as the header defines them, from a
    per-column piece index: tile t covers relaid columns [t*64E, (t+1)*64E);
    it gets the slab vector its source starts at when all of its columns lie
    in [0, out_numel) and in one piece whose source run starts on a vector
    and stays in the bucket, else -1."""
    E = 8 if dtype == wl.DT_BF16 else 4
    span = 64 * E
    n = -(-(-(-out_numel // E)) // 64)
    # a column belongs to the last piece starting at or before it, if that
    # piece reaches it
    cols = np.arange(n * span)
    dst = pieces["dst"].astype(np.int64)
    last = np.searchsorted(dst, cols, side="right") - 1
    pid = np.full(n * span, -1, np.int64)
    has = last >= 0
    ends = dst + pieces["len"].astype(np.int64)
    inside = np.zeros(n * span, bool)
    inside[has] = cols[has] < ends[last[has]]
    pid[inside] = last[inside]
    recs = np.full(n, -1, np.int64)
    for t in range(n):
        d0 = t * span
        ids = pid[d0:d0 + span]
        if d0 + span > out_numel or ids[0] < 0 or np.any(ids != ids[0]):
            continue
        pc = pieces[int(ids[0])]
        src0 = int(pc["src"]) + d0 - int(pc["dst"])
        if src0 >= 0 and src0 + span <= bucket_numel and (bucket_col + src0) % E == 0:
            recs[t] = (bucket_col + src0) // E
    return _xcd_major(recs)


def relayout_tile_cases(seed):
    """(dtype, bucket_col, bucket_numel, pieces, out_numel): the relayout
    planner's pieces of small and random workloads at several bucket-start
    residues, and random piece tables with unaligned sources, gaps, empty
    pieces and pieces starting inside earlier ones."""
    rng = random.Random(seed)
    cases = []
    ws = [wl.tiny_flush()]
    for k in range(5):
        W = rng.choice([2, 4, 8])
        dt = rng.choice([wl.DT_BF16, wl.DT_F32])
        sizes = [rng.choice([0, 3, 64, 700, 2048, 4096, 9000]) for _ in range(60)]
        ws.append(wl.custom_flush(f"t{k}", W, dt, sizes, group_begin=[0, 40, 60], group_comm=[0, 0],
                                  comms=[wl.Comm(W, 1)], capacity=40_000))
    for w in ws:
        flat, ps, off, pids = oracle.partition_ids(w.numel, w.group_begin, w.group_parts())
        psize = np.zeros(w.P, np.int64)
        for g in range(w.G):
            psize[w.group_begin[g]:w.group_begin[g + 1]] = ps[g]
        for bk in w.buckets:
            t = dc.tasks_array([(x.offset, x.numel, x.param, x.comm) for x in bk.tasks])
            pieces, seg = dc.dc_plan_relayout(w.W, t, len(t), flat, psize, w.P)
            for shift in (0, 1, 8):
                cases.append((w.dtype, bk.col + shift, bk.numel, pieces, int(seg[-1])))
    for k in range(60):
        dt = rng.choice([wl.DT_BF16, wl.DT_F32])
        numel = rng.randint(0, 20_000)
        dst, pcs = 0, []
        overlap = k >= 40          # later pieces may start inside earlier ones
        for _ in range(rng.randint(0, 12)):
            dst += rng.choice([0, 0, 1, 8, 300])
            ln = rng.choice([0, 5, 512, 1024, 3000])
            src = rng.randint(-4, numel) if rng.random() < 0.2 else rng.choice([0, 8, 512, 1000])
            pcs.append((src, dst, ln, 0))
            dst += rng.choice([0, 100, ln // 2]) if overlap else ln
        pieces = np.array(pcs, dc.PIECE_DTYPE) if pcs else np.zeros(0, dc.PIECE_DTYPE)
        cases.append((dt, rng.choice([0, 3, 64, 4096]), numel, pieces, dst + rng.choice([0, 7, 600])))
    return cases


def test_plan_relayout_tiles_matches_definition():
    """dc_plan_relayout_tiles (host code) against the records the header
    defines, on relayout_tile_cases."""
    whole = 0
    for dt, col, numel, pieces, out_numel in relayout_tile_cases(12):
        got = dc.dc_plan_relayout_tiles(dt, col, numel, pieces, len(pieces), out_numel)
        want = _brute_relayout_tiles(dt, col, numel, pieces, out_numel)
        assert np.array_equal(got, want), (dt, col, numel, out_numel)
        whole += int(np.sum(got >= 0))
    assert whole > 100        # the cases reach the straight copy, not only the search


def test_plan_relayout_tiles_argument_checks():
    pcs = np.array([(0, 0, 600, 0), (600, 600, 600, 0)], dc.PIECE_DTYPE)
    assert len(dc.dc_plan_relayout_tiles(0, 0, 1200, pcs, 2, 1200)) == 3
    assert len(dc.dc_plan_relayout_tiles(1, 0, 1200, pcs, 2, 1200)) == 5
    assert len(dc.dc_plan_relayout_tiles(0, 0, 0, None, 0, 0)) == 0
    bad = pcs.copy()
    bad[1]["dst"] = 0
    bad[0]["dst"] = 600
    expect(dc.DC_ERR_ARG, dc.dc_plan_relayout_tiles, 0, 0, 1200, bad, 2, 1200)   # out of dst order
    bad = pcs.copy()
    bad[0]["len"] = -1
    expect(dc.DC_ERR_ARG, dc.dc_plan_relayout_tiles, 0, 0, 1200, bad, 2, 1200)
    expect(dc.DC_ERR_ARG, dc.dc_plan_relayout_tiles, 0, -1, 1200, pcs, 2, 1200)
    expect(dc.DC_ERR_DTYPE, dc.dc_plan_relayout_tiles, 5, 0, 1200, pcs, 2, 1200)
    n = ctypes.c_int64(0)
    rc = dc.lib().dc_plan_relayout_tiles(0, 0, 1200, pcs.ctypes.data_as(ctypes.c_void_p), 2, 1200,
                                         np.zeros(2, np.int64).ctypes.data_as(ctypes.c_void_p), 2,
                                         ctypes.byref(n))
    assert rc == dc.DC_ERR_SHAPE and n.value == 3
    rc = dc.lib().dc_plan_relayout_tiles(0, 0, 1200, pcs.ctypes.data_as(ctypes.c_void_p), 2, 1200,
                                         None, 0, None)
    assert rc == dc.DC_ERR_NULL
    rc = dc.lib().dc_plan_relayout_tiles(0, 0, 1200, None, 2, 1200, None, 0, ctypes.byref(n))
    assert rc == dc.DC_ERR_NULL


def test_relayout_planned_argument_checks():
    f = dc.dc_relayout_bucket_planned
    ok = dict(W=8, dtype=0, slab_in=FAKE, ld_in=2048, out=FAKE + (1 << 30), ld_out=2048,
              bucket_col=0, bucket_numel=2048, pieces=TASK_PTR, num_pieces=1, out_numel=2048,
              tiles=TASK_PTR + 4096, num_tiles=4, stream=0)

    def call(**ch):
        a = dict(ok)
        a.update(ch)
        return f(**a)

    expect(dc.DC_ERR_SHAPE, call, num_tiles=3)               # 2048 bf16 columns: 4 tiles
    expect(dc.DC_ERR_SHAPE, call, dtype=1, num_tiles=4)      # fp32: 8 tiles
    expect(dc.DC_ERR_NULL, call, tiles=None)
    expect(dc.DC_ERR_NULL, call, pieces=None)
    expect(dc.DC_ERR_ARG, call, W=0)
    expect(dc.DC_ERR_ARG, call, bucket_col=-1)
    expect(dc.DC_ERR_NULL, call, slab_in=None)
    expect(dc.DC_ERR_ARG, call, out=FAKE)                    # overlaps slab_in
    expect(dc.DC_ERR_SHAPE, call, ld_out=1024)               # out_numel past ld_out
