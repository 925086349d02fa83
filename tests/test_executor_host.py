"""Host logic of the executor, on the CPU: the fused flush's pointer tables
(per-rank addresses, split params, empty buffers, coordinates); the device
kernels are not run (the holder sets come from dc_holders, tested in
test_abi.py; the ZeRO-2 partition sizes from a kernel, tested on the GPU)."""
import numpy as np
import pytest

import oracle
from gradient_reduction_amd import dc, executor
from synth import workloads as wl
from tests import gpu_util as U


def _cpu_executor(W, dtype, numel, buckets, group_begin=None, group_parts=None):
    P = len(numel)
    gb = group_begin or [0, P]
    G = len(gb) - 1
    parts = group_parts or [W] * G
    ex = executor.Zero1FlushExecutor(
        W, dtype, numel, gb, parts, [W] * G, [list(range(W))] * G, [(W, 1)], buckets, 1,
        reduce_to_owner=True, device="cpu")
    flat, ps, off, pids = oracle.partition_ids(numel, gb, parts)
    elig = oracle.group_eligible(W, [W] * G, [list(range(W))] * G)
    owner, _ = oracle.owner_map(off, pids, gb, elig)
    ex.h_owner, ex.h_pid_off, ex.h_pids = owner, off, pids
    return ex


def test_register_buffers_tables_split_param():
    """Param 1 is split over two buckets: its second task's pointers start
    where the first task ended; a rank without a buffer gets 0; task
    coordinates sit on 128-byte steps; the extent is the last task's end."""
    W, dtype = 4, dc.DC_BF16
    numel = [100, 5000, 37]
    buckets = [executor.BucketSpec(0, 3100, [(0, 100, 0, 0), (100, 3000, 1, 0)]),
               executor.BucketSpec(3100, 2037, [(0, 2000, 1, 0), (2000, 37, 2, 0)])]
    ex = _cpu_executor(W, dtype, numel, buckets)
    base_in = 1 << 40
    in_addr = np.array([[base_in + (r << 30) + p * 65536 for p in range(3)] for r in range(W)],
                       np.uint64)
    out_addr = np.zeros((W, 3), np.uint64)
    out_addr[1, 1] = (1 << 41) + 4096          # only rank 1 keeps param 1
    out_addr[:, 0] = (1 << 42) + np.arange(W, dtype=np.uint64) * 4096
    ex.register_buffers(in_addr, out_addr)
    ti = ex.d_bin.numpy().view(np.uint64).reshape(-1, W)
    to = ex.d_bout.numpy().view(np.uint64).reshape(-1, W)
    tasks = ex.d_btasks.numpy().view(dc.TASK_DTYPE)
    # bucket 0: tasks 0, 1; bucket 1: tasks 2, 3
    assert list(ex.buf_begin) == [0, 2, 4]
    for r in range(W):
        assert ti[0, r] == in_addr[r, 0]
        assert ti[1, r] == in_addr[r, 1]
        assert ti[2, r] == in_addr[r, 1] + 3000 * 2         # continues after 3000 elements
        assert ti[3, r] == in_addr[r, 2]
    assert to[1].tolist() == [0, int(out_addr[1, 1]), 0, 0]
    assert to[2].tolist() == [0, int(out_addr[1, 1]) + 6000, 0, 0]
    assert to[3].tolist() == [0, 0, 0, 0]
    step = 128 // 2
    assert all(int(o) % step == 0 for o in tasks["offset"])
    assert list(tasks["numel"]) == [100, 3000, 2000, 37]
    assert ex.buf_extent == [int(tasks["offset"][1]) + 3000, int(tasks["offset"][3]) + 37]


def test_register_buffers_rejects_overlap():
    W = 2
    numel = [64, 64]
    buckets = [executor.BucketSpec(0, 128, [(0, 64, 0, 0), (64, 64, 1, 0)])]
    ex = _cpu_executor(W, dc.DC_F32, numel, buckets)
    in_addr = np.array([[1 << 40, (1 << 40) + 4096], [(1 << 40) + 8192, (1 << 40) + 12288]], np.uint64)
    out_addr = in_addr.copy()
    out_addr[1, 0] = in_addr[0, 0] + 16          # rank 1's output inside rank 0's input
    with pytest.raises(dc.DCError) as e:
        ex.register_buffers(in_addr, out_addr)
    assert e.value.code == dc.DC_ERR_TASKS




def test_deferred_reducer_rejects_short_stride():
    """DeferredReducer checks its accumulator's stride before allocating."""
    from gradient_reduction_amd.deferred import DeferredReducer
    with pytest.raises(ValueError):
        DeferredReducer(4, 100, ld=64)
