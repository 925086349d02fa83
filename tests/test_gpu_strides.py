"""GPU parity with every slab at a row stride of its own (through the C ABI).

The other parity tests give input and output slabs one stride, so a kernel
that addressed an output row with the input's stride (or the reverse) would
pass them.  Here the strides of the inputs and outputs all differ, both
larger and smaller than each other, and the results are compared with the
oracle bit for bit, sentinels included: bucket flush (fast W = 8 path and
run-time W = 5 path, owner and AllReduce, both dtypes), ZeRO-2 flush,
accumulate, deferred reduce and the fused accumulate-reduce.
"""
import numpy as np
import pytest

import oracle
from gradient_reduction_amd import dc
from synth import workloads as wl
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dc.lib()
    yield
    torch.cuda.synchronize()


def _bucket(W, sizes, col0):
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(int).tolist()
    return offs, col0, int(sum(sizes))


FLUSH_CASES = [(8, wl.DT_BF16, True, 1, 64), (8, wl.DT_BF16, False, 1, 128),
               (8, wl.DT_F32, True, 0, 192), (5, wl.DT_BF16, True, 1, 64),
               (5, wl.DT_F32, False, 0, 256), (16, wl.DT_F32, True, 0, 64)]


@pytest.mark.parametrize("planned", [False, True], ids=["searched", "planned"])
@pytest.mark.parametrize("W,dtype,owner,pre,extra", FLUSH_CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("out_wider", [True, False], ids=["out-wider", "in-wider"])
def test_flush_distinct_strides(W, dtype, owner, pre, extra, out_wider, planned):
    import torch
    sizes = [3000, 1, 17, 8191, 0, 640, 4097, 9]
    offs, col0, numel = _bucket(W, sizes, 13)
    P = len(sizes)
    base = wl.round_up(col0 + numel, 64)
    ld_in, ld_out = (base, base + extra) if out_wider else (base + extra, base)
    U.say("flush strides", W, dtype, owner, pre, ld_in, ld_out)
    scale = wl.sigma_scale(1e-2)
    x = U.gen_slab(dtype, W, ld_in, ld_in, 501, 0, scale)
    y = U.empty_slab(dtype, W, ld_out)
    own = np.array([(3 * p) % W if p % 3 else -1 for p in range(P)], np.int32)
    tasks = dc.tasks_array([(offs[k], sizes[k], k, 0) for k in range(P)])
    d_tasks = torch.from_numpy(tasks.view(np.uint8).copy()).cuda()
    d_own = torch.from_numpy(own).cuda() if owner else None
    if planned:
        keep = U.planned_flush(W, dtype, x, ld_in, y, ld_out, col0, numel, tasks, d_tasks, P,
                               [(W, 1)], pre, owner=own if owner else None)
    else:
        dc.dc_flush_bucket(W, dtype, x, ld_in, y, ld_out, col0, numel, d_tasks, P, d_own, P,
                           [(W, 1)], 1, pre)
    torch.cuda.synchronize()
    hin = U.host_slab(dtype, W, ld_in, ld_in, 501, 0, scale)
    hout = np.zeros((W, ld_out), hin.dtype)
    U.bits(hout, dtype)[:] = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
    oracle.flush(W, dtype, hin, hout, col0, offs, sizes, list(range(P)), [0] * P,
                 own if owner else None, [W], [1], pre)
    assert np.array_equal(U.bits(U.to_host(y, dtype), dtype), U.bits(hout, dtype))


@pytest.mark.parametrize("planned", [False, True], ids=["searched", "planned"])
@pytest.mark.parametrize("W,dtype", [(8, wl.DT_BF16), (4, wl.DT_F32), (6, wl.DT_BF16)])
def test_flush_zero2_distinct_strides(W, dtype, planned):
    import torch
    sizes = [5000, 77, 12001, 3, 2500]
    offs, col0, numel = _bucket(W, sizes, 5)
    P = len(sizes)
    flat = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)
    S = -(-int(sum(sizes)) // W)
    psize = np.full(P, S, np.int64)
    base = wl.round_up(col0 + numel, 64)
    ld_in, ld_out = base + 128, base + 64
    U.say("zero2 strides", W, dtype, ld_in, ld_out)
    scale = wl.sigma_scale(1e-2)
    x = U.gen_slab(dtype, W, ld_in, ld_in, 502, 0, scale)
    y = U.empty_slab(dtype, W, ld_out)
    tasks = dc.tasks_array([(offs[k], sizes[k], k, 0) for k in range(P)])
    d_tasks = torch.from_numpy(tasks.view(np.uint8).copy()).cuda()
    if planned:
        keep = U.planned_flush(W, dtype, x, ld_in, y, ld_out, col0, numel, tasks, d_tasks, P,
                               [(W, 1)], 1, flat=flat, psize=psize)
    else:
        dc.dc_flush_bucket_zero2(W, dtype, x, ld_in, y, ld_out, col0, numel, d_tasks, P,
                                 torch.from_numpy(flat).cuda(), torch.from_numpy(psize).cuda(), P,
                                 [(W, 1)], 1, 1)
    torch.cuda.synchronize()
    hin = U.host_slab(dtype, W, ld_in, ld_in, 502, 0, scale)
    hout = np.zeros((W, ld_out), hin.dtype)
    U.bits(hout, dtype)[:] = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
    oracle.flush_zero2(W, dtype, hin, hout, col0, offs, sizes, list(range(P)), [0] * P, flat, psize,
                       [W], [1], 1)
    assert np.array_equal(U.bits(U.to_host(y, dtype), dtype), U.bits(hout, dtype))


@pytest.mark.parametrize("rows,M,init", [(4, 10_003, 0), (4, 10_003, 1), (1, 777, 0)])
def test_accumulate_distinct_strides(rows, M, init):
    import torch
    base = wl.round_up(M, 64)
    ld_x, ld_acc = base + 192, base + 64
    scale = wl.sigma_scale(1e-3)
    x = U.gen_slab(wl.DT_F32, rows, ld_x, ld_x, 511, 0, scale).view(torch.float32)
    acc = U.gen_slab(wl.DT_F32, rows, ld_acc, ld_acc, 512, 0, scale).view(torch.float32)
    hx = U.host_slab(wl.DT_F32, rows, ld_x, ld_x, 511, 0, scale)
    hacc = U.host_slab(wl.DT_F32, rows, ld_acc, ld_acc, 512, 0, scale)
    dc.dc_accumulate(rows, x, ld_x, acc, ld_acc, M, init)
    torch.cuda.synchronize()
    oracle.accumulate(rows, hx, hacc, M, init)
    assert np.array_equal(acc.cpu().numpy().view(np.uint32), hacc.view(np.uint32))


@pytest.mark.parametrize("W,out_rows", [(4, 4), (4, 1), (8, 8), (3, 1)])
def test_deferred_reduce_distinct_strides(W, out_rows):
    import torch
    M = 9_001
    base = wl.round_up(M, 64)
    ld_acc, ld_out = base + 64, base + 256
    scale = wl.sigma_scale(1e-3)
    acc = U.gen_slab(wl.DT_F32, W, ld_acc, ld_acc, 521, 0, scale).view(torch.float32)
    hacc = U.host_slab(wl.DT_F32, W, ld_acc, ld_acc, 521, 0, scale)
    out = U.empty_slab(wl.DT_F32, out_rows, ld_out).view(torch.float32)
    hout = np.full((out_rows, ld_out), np.uint32(U.SENTINEL32)).view(np.float32)
    dc.dc_deferred_reduce(W, acc, ld_acc, out, ld_out, M, out_rows)
    torch.cuda.synchronize()
    oracle.deferred_reduce(W, hacc, hout, M, out_rows)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), hout.view(np.uint32))


@pytest.mark.parametrize("W,init,keep,out_rows", [(4, 0, 1, 4), (4, 1, 0, 1), (8, 0, 1, 1)])
def test_accumulate_reduce_distinct_strides(W, init, keep, out_rows):
    import torch
    M = 6_007
    base = wl.round_up(M, 64)
    ld_x, ld_acc, ld_out = base + 128, base, base + 320
    scale = wl.sigma_scale(1e-3)
    x = U.gen_slab(wl.DT_F32, W, ld_x, ld_x, 531, 0, scale).view(torch.float32)
    acc = U.gen_slab(wl.DT_F32, W, ld_acc, ld_acc, 532, 0, scale).view(torch.float32)
    hx = U.host_slab(wl.DT_F32, W, ld_x, ld_x, 531, 0, scale)
    hacc = U.host_slab(wl.DT_F32, W, ld_acc, ld_acc, 532, 0, scale)
    out = U.empty_slab(wl.DT_F32, out_rows, ld_out).view(torch.float32)
    dc.dc_accumulate_reduce(W, x, ld_x, acc, ld_acc, init, keep, out, ld_out, out_rows, M)
    torch.cuda.synchronize()
    a2 = hacc.copy()
    oracle.accumulate(W, hx, a2, M, init)
    want = np.full((out_rows, ld_out), np.uint32(U.SENTINEL32)).view(np.float32)
    oracle.deferred_reduce(W, a2, want, M, out_rows)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))
    wacc = a2 if keep else hacc
    assert np.array_equal(acc.cpu().numpy().view(np.uint32), wacc.view(np.uint32))
