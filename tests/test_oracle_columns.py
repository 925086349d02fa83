"""The oracle's column-block driver (oracle/columns.py) writes exactly what
one whole call of the oracle writes: flushes in every mode (owner,
AllReduce, ZeRO-2, a sub-communicator), in place and out of place, the
deferred path and its status quo, the reduce-scatter.  Blocks are made small
here so that tasks and shards are cut into many of them."""
import numpy as np
import pytest

import oracle
from oracle import columns as OC
import synth
from synth import workloads as wl

SENT16, SENT32 = 0x7E7E, 0x7E7E7E7E


def _whole(w, owner, zero2, init):
    """The oracle over the whole slab in one call per bucket."""
    ld = w.ld
    hin = synth.fill_slab(w.dtype, w.value_seed, 0, w.scale, w.W, ld, w.total)
    if w.dtype == wl.DT_F32:
        hin = hin.view(np.float32)
    if init == "input":
        hout = hin.copy()
    else:
        hout = np.zeros_like(hin)
        hout.view(np.uint16 if w.dtype == wl.DT_BF16 else np.uint32)[:] = init
    cs = [c.size for c in w.comms]
    cst = [c.stride for c in w.comms]
    for bk in w.buckets:
        args = (w.W, w.dtype, hin, hout, bk.col, [t.offset for t in bk.tasks],
                [t.numel for t in bk.tasks], [t.param for t in bk.tasks],
                [t.comm for t in bk.tasks])
        if zero2 is None:
            oracle.flush(*args, owner, cs, cst, w.pre_div)
        else:
            oracle.flush_zero2(*args, zero2[0], zero2[1], cs, cst, w.pre_div)
    return hout


def _small_mixed():
    """W = 16 fp32, three groups, the last on four 4-rank sub-communicators."""
    rng = np.random.default_rng(5)
    numel = [int(v) for v in rng.integers(1, 9000, 60)] + [0, 1, 7]
    P = len(numel)
    return wl.custom_flush("mixed_small", 16, wl.DT_F32, numel,
                           group_begin=[0, P // 3, 2 * P // 3, P], group_comm=[0, 0, 1],
                           comms=[wl.Comm(16, 1), wl.Comm(4, 1)], capacity=60000, pre_div=0,
                           sigma=1e-3, value_seed=9)


CASES = [("tiny", "owner", SENT16), ("tiny", "allreduce", SENT16), ("tiny", "zero2", "input"),
         ("mixed", "owner", "input"), ("mixed", "allreduce", SENT32), ("mixed", "zero2", SENT32)]


@pytest.mark.parametrize("wname,mode,init", CASES)
def test_flush_blocks_equal_one_call(wname, mode, init):
    w = wl.tiny_flush() if wname == "tiny" else _small_mixed()
    owner = OC.owner_of(w) if mode == "owner" else None
    zero2 = OC.zero2_tables(w) if mode == "zero2" else None
    want = _whole(w, owner, zero2, init)
    for b, bk in enumerate(w.buckets):
        got = OC.flush_bucket(w, b, owner=owner, zero2=zero2, init=init, block=1000)
        exp = want[:, bk.col:bk.col + bk.numel]
        assert np.array_equal(got.view(np.uint8), np.ascontiguousarray(exp).view(np.uint8)), b


def test_zero2_blocks_cross_partition_boundaries():
    """A block of a straddling param starts inside the param: its flat
    position must carry the block's offset.  The driver gets it right, and
    the same blocks with the offset dropped land in other partitions (so the
    check above would catch that slip)."""
    w = wl.custom_flush("z2", 4, wl.DT_BF16, [5000, 7001, 3000], capacity=10 ** 6, pre_div=1)
    flat, psize = OC.zero2_tables(w)
    assert psize[0] > 0
    want = _whole(w, None, (flat, psize), SENT16)
    got = OC.flush_bucket(w, 0, zero2=(flat, psize), init=SENT16, block=333)
    assert np.array_equal(got, want[:, :w.total])
    blocks = OC.task_blocks(OC.bucket_tasks(w.buckets[0]), 333)
    hin = OC.host_rows(w.dtype, w.value_seed, 0, w.scale, w.W, 0, w.total)
    slip = np.full_like(hin, SENT16)
    oracle.flush_zero2(w.W, w.dtype, hin, slip, 0, [b[0] for b in blocks], [b[1] for b in blocks],
                       [b[2] for b in blocks], [b[3] for b in blocks], flat, psize, [w.W], [1],
                       w.pre_div)
    assert not np.array_equal(slip[:, :w.total], want[:, :w.total])


def test_deferred_columns_equal_one_call():
    W, K, n = 4, 3, 70000
    scale = wl.sigma_scale(1e-3)

    def so(k, r):
        return wl.microbatch_stream(k, W, r)
    acc, D, A = OC.deferred_columns(W, 3, scale, K, so, 1000, n, block=1 << 12)
    xs = [OC.host_rows(wl.DT_F32, 3, 0, scale, W, 1000, n, stream_of=lambda r, k=k: so(k, r))
          for k in range(K)]
    a = np.zeros((W, n), np.float32)
    q = np.zeros((1, n), np.float32)
    for k, x in enumerate(xs):
        x = np.ascontiguousarray(x[:, :n])
        oracle.accumulate(W, x, a, n, 1 if k == 0 else 0)
        g = np.zeros((1, n), np.float32)
        oracle.deferred_reduce(W, x, g, n, 1)
        oracle.accumulate(1, g, q, n, 1 if k == 0 else 0)
    d = np.zeros((1, n), np.float32)
    oracle.deferred_reduce(W, a, d, n, 1)
    assert np.array_equal(acc.view(np.uint32), a.view(np.uint32))
    assert np.array_equal(D.view(np.uint32), d[0].view(np.uint32))
    assert np.array_equal(A.view(np.uint32), q[0].view(np.uint32))


@pytest.mark.parametrize("W,dtype,pre", [(8, wl.DT_BF16, 0), (4, wl.DT_F32, 1)])
def test_reduce_scatter_columns_equal_one_call(W, dtype, pre):
    M = W * 5003
    hin = OC.host_rows(dtype, 4, 0, wl.sigma_scale(1e-2), W, 0, M)
    got = OC.reduce_scatter_columns(W, dtype, np.ascontiguousarray(hin[:, :M]), M, pre, block=700)
    want = np.zeros((W, M // W), hin.dtype)
    oracle.reduce_scatter(W, dtype, np.ascontiguousarray(hin[:, :M]), want, M, pre)
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))
