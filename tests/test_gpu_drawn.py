"""GPU: the slab collectives and the deferred path on hypothesis-drawn shapes
(derandomized, so every run draws the same cases): W from 1 to 64, both
dtypes, shard lengths and column counts from empty to several tiles with
ragged tails, padded row strides, pre-division on and off.  Every output
element against the oracle, bit for bit."""
import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from gradient_reduction_amd import dc
from synth import workloads as wl
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

SET = settings(max_examples=120, deadline=None, derandomize=True)
SCALE = wl.sigma_scale(1e-2)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dc.lib()
    yield
    torch.cuda.synchronize()


def _host_sentinel(dtype, rows, ld):
    a = np.zeros((rows, ld), np.uint16 if dtype == wl.DT_BF16 else np.float32)
    U.bits(a, dtype)[:] = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
    return a


def _same(dev, host, dtype):
    return np.array_equal(U.bits(U.to_host(dev, dtype), dtype), U.bits(host, dtype))


@st.composite
def collective_shapes(draw):
    W = draw(st.sampled_from([1, 2, 3, 4, 5, 7, 8, 12, 16, 33, 64]))
    dtype = draw(st.sampled_from([wl.DT_BF16, wl.DT_F32]))
    L = draw(st.one_of(st.integers(0, 70), st.integers(0, 3000), st.sampled_from([64, 512, 1024])))
    pad_in = draw(st.sampled_from([0, 8, 64, 8000]))
    pad_sh = draw(st.sampled_from([0, 8, 24]))
    pre = draw(st.integers(0, 1))
    seed = draw(st.integers(0, 1000))
    return W, dtype, L, pad_in, pad_sh, pre, seed


def test_reduce_scatter_and_all_gather_on_drawn_shapes():
    """dc_reduce_scatter, then dc_all_gather of its shards in rank and in
    ring order ([AG] eq:ag-semantic-output, Ring AllGather)."""
    import torch

    @SET
    @given(collective_shapes())
    def run(shape):
        W, dtype, L, pad_in, pad_sh, pre, seed = shape
        M = W * L
        ld = wl.round_up(max(M, 1), 8) + pad_in
        ld_sh = wl.round_up(max(L, 1), 8) + pad_sh
        x = U.gen_slab(dtype, W, ld, M, seed, 0, SCALE)
        hin = U.host_slab(dtype, W, ld, M, seed, 0, SCALE)
        sh = U.empty_slab(dtype, W, ld_sh)
        dc.dc_reduce_scatter(W, dtype, x, ld, sh, ld_sh, M, pre)
        want_sh = _host_sentinel(dtype, W, ld_sh)
        oracle.reduce_scatter(W, dtype, hin, want_sh, M, pre)
        torch.cuda.synchronize()
        assert _same(sh, want_sh, dtype), ("reduce-scatter", shape)
        for order in (dc.DC_ORDER_RANK, dc.DC_ORDER_RING):
            out = U.empty_slab(dtype, W, ld)
            dc.dc_all_gather(W, dtype, sh, ld_sh, out, ld, L, order, -1)
            want = _host_sentinel(dtype, W, ld)
            oracle.all_gather(W, dtype, want_sh, want, L, order)
            torch.cuda.synchronize()
            assert _same(out, want, dtype), ("all-gather", order, shape)

    U.say("reduce-scatter / all-gather on drawn shapes")
    run()


@st.composite
def deferred_shapes(draw):
    W = draw(st.sampled_from([1, 2, 3, 4, 8, 16]))
    M = draw(st.one_of(st.integers(0, 100), st.integers(0, 5000)))
    K = draw(st.integers(1, 4))
    out_rows = draw(st.sampled_from([1, W]))
    pad = draw(st.sampled_from([0, 4, 12, 400]))
    seed = draw(st.integers(0, 1000))
    return W, M, K, out_rows, pad, seed


def test_accumulate_and_deferred_reduce_on_drawn_shapes():
    """K replica-local accumulates from a zero start, then the deferred
    cross-replica reduce ([MT] What): the accumulators and the reduced rows."""
    import torch

    @SET
    @given(deferred_shapes())
    def run(shape):
        W, M, K, out_rows, pad, seed = shape
        ld = wl.round_up(max(M, 1), 4) + pad
        acc = U.empty_slab(wl.DT_F32, W, ld)
        h_acc = _host_sentinel(wl.DT_F32, W, ld)
        for k in range(K):
            x = U.gen_slab(wl.DT_F32, W, ld, M, seed, k * W, SCALE)
            hx = U.host_slab(wl.DT_F32, W, ld, M, seed, k * W, SCALE)
            dc.dc_accumulate(W, x, ld, acc, ld, M, 1 if k == 0 else 0)
            oracle.accumulate(W, hx, h_acc, M, 1 if k == 0 else 0)
        out = U.empty_slab(wl.DT_F32, out_rows, ld)
        dc.dc_deferred_reduce(W, acc, ld, out, ld, M, out_rows)
        h_out = _host_sentinel(wl.DT_F32, out_rows, ld)
        oracle.deferred_reduce(W, h_acc, h_out, M, out_rows)
        torch.cuda.synchronize()
        assert _same(acc, h_acc, wl.DT_F32), ("accumulators", shape)
        assert _same(out, h_out, wl.DT_F32), ("deferred reduce", shape)

    U.say("accumulate / deferred reduce on drawn shapes")
    run()


def test_ring_reduce_scatter_and_all_gather_steps_on_drawn_shapes():
    """The ring-order reduce-scatter (shard s folded in the order s, s+1, ...),
    and every step of the ring, bidirectional-ring and (at powers of two)
    recursive-doubling all-gather schedules replayed one launch per step, the
    output checked after each step ([AG] Ring AllGather, eq:ag-bidir-ring,
    Recursive Doubling AllGather)."""
    import torch

    @SET
    @given(collective_shapes())
    def run(shape):
        W, dtype, L, pad_in, pad_sh, pre, seed = shape
        M = W * L
        ld = wl.round_up(max(M, 1), 8) + pad_in
        ld_sh = wl.round_up(max(L, 1), 8) + pad_sh
        x = U.gen_slab(dtype, W, ld, M, seed, 0, SCALE)
        hin = U.host_slab(dtype, W, ld, M, seed, 0, SCALE)
        sh = U.empty_slab(dtype, W, ld_sh)
        dc.dc_reduce_scatter_ring(W, dtype, x, ld, sh, ld_sh, M, pre)
        want_sh = _host_sentinel(dtype, W, ld_sh)
        oracle.reduce_scatter_ring(W, dtype, hin, want_sh, M, pre)
        torch.cuda.synchronize()
        assert _same(sh, want_sh, dtype), ("ring reduce-scatter", shape)
        algos = [dc.DC_SCHED_RING, dc.DC_SCHED_BIDIR]
        if W & (W - 1) == 0:
            algos.append(dc.DC_SCHED_RD)
        steps = {dc.DC_SCHED_RING: W - 1, dc.DC_SCHED_BIDIR: W // 2,
                 dc.DC_SCHED_RD: W.bit_length() - 1}
        for algo in algos:
            out = U.empty_slab(dtype, W, ld)
            want = _host_sentinel(dtype, W, ld)
            for s in range(steps[algo] + 1):
                dc.dc_all_gather_step(W, dtype, sh, ld_sh, out, ld, L, algo, s)
                oracle.all_gather_step(W, dtype, want_sh, want, L, algo, s)
                torch.cuda.synchronize()
                assert _same(out, want, dtype), ("all-gather step", algo, s, shape)

    U.say("ring reduce-scatter / all-gather steps on drawn shapes")
    run()


def test_fused_accumulate_reduce_on_drawn_shapes():
    """The last accumulate fused into the deferred reduce, keeping the
    accumulator or not, against the oracle's accumulate then reduce."""
    import torch

    @SET
    @given(deferred_shapes(), st.integers(0, 1), st.integers(0, 1))
    def run(shape, init, keep):
        W, M, K, out_rows, pad, seed = shape
        ld = wl.round_up(max(M, 1), 4) + pad
        acc = U.gen_slab(wl.DT_F32, W, ld, M, seed + 1, 0, SCALE)
        h_acc = U.host_slab(wl.DT_F32, W, ld, M, seed + 1, 0, SCALE)
        x = U.gen_slab(wl.DT_F32, W, ld, M, seed, 7 * W, SCALE)
        hx = U.host_slab(wl.DT_F32, W, ld, M, seed, 7 * W, SCALE)
        out = U.empty_slab(wl.DT_F32, out_rows, ld)
        dc.dc_accumulate_reduce(W, x, ld, acc, ld, init, keep, out, ld, out_rows, M)
        h_acc2 = h_acc.copy()
        oracle.accumulate(W, hx, h_acc2, M, init)
        h_out = _host_sentinel(wl.DT_F32, out_rows, ld)
        oracle.deferred_reduce(W, h_acc2, h_out, M, out_rows)
        torch.cuda.synchronize()
        assert _same(out, h_out, wl.DT_F32), ("fused reduce", shape, init, keep)
        assert _same(acc, h_acc2 if keep else h_acc, wl.DT_F32), ("accumulator", shape, init, keep)

    U.say("fused accumulate-reduce on drawn shapes")
    run()


@st.composite
def relayout_workloads(draw):
    W = draw(st.sampled_from([1, 2, 3, 4, 5, 8, 16]))
    dtype = draw(st.sampled_from([wl.DT_BF16, wl.DT_F32]))
    sizes = draw(st.lists(st.one_of(st.integers(0, 20), st.integers(0, 3000),
                                    st.sampled_from([64, 1024, 4096])), min_size=1, max_size=40))
    split = draw(st.integers(0, len(sizes)))
    capacity = draw(st.sampled_from([500, 5000, 20_000, 10 ** 6]))
    pre = draw(st.integers(0, 1))
    seed = draw(st.integers(0, 1000))
    return wl.custom_flush("drawn", W, dtype, sizes, group_begin=[0, split, len(sizes)],
                           group_comm=[0, 0], comms=[wl.Comm(W, 1)], capacity=capacity,
                           pre_div=pre, value_seed=seed)


def test_relayout_and_reduce_scatter_v_on_drawn_workloads():
    """Every bucket of drawn workloads (two parameter groups, buckets of any
    start residue, empty and one-element tensors) relaid by destination rank,
    searched and from its tile plan, then reduced by reduce-scatter-v: the
    relaid slab and the shards against the oracle's relayout map and
    reduce-scatter-v ([DS] "Describe alternatives")."""
    from tests import test_gpu_relayout as TR

    @settings(max_examples=60, deadline=None, derandomize=True)
    @given(relayout_workloads(), st.booleans())
    def run(w, planned):
        ld = w.ld
        x = U.gen_slab(w.dtype, w.W, ld, w.total, w.value_seed, 0, w.scale)
        hx = U.host_slab(w.dtype, w.W, ld, w.total, w.value_seed, 0, w.scale)
        sent = U.SENTINEL16 if w.dtype == wl.DT_BF16 else U.SENTINEL32
        for b, bk in enumerate(w.buckets):
            relaid, shards, seg, pieces, flat, psize = TR.run_bucket(w, b, x, ld, planned=planned)
            dest, oseg = oracle.relayout_map(w.W, [k.offset for k in bk.tasks],
                                             [k.numel for k in bk.tasks], [k.param for k in bk.tasks],
                                             [k.comm for k in bk.tasks], flat, psize, bk.numel)
            assert np.array_equal(seg, oseg)
            hr = np.zeros_like(relaid)
            U.bits(hr, w.dtype)[:] = sent
            oracle.relayout_apply(w.W, w.dtype, hx, hr, bk.col, bk.numel, dest)
            assert np.array_equal(U.bits(relaid, w.dtype), U.bits(hr, w.dtype)), (b, planned)
            hs = np.zeros_like(shards)
            U.bits(hs, w.dtype)[:] = sent
            oracle.reduce_scatter_v(w.W, w.dtype, hr, hs, oseg, w.pre_div)
            assert np.array_equal(U.bits(shards, w.dtype), U.bits(hs, w.dtype)), (b, planned)

    U.say("relayout + reduce-scatter-v on drawn workloads")
    run()


def test_fused_flush_on_drawn_layouts():
    """The flush with copy-in and copy-out fused in, on drawn task sizes,
    holder sets, buffer placements (aligned or not, packed or padded task
    coordinates, in place or not), searched and planned, W from 1 to 64 with
    sub-communicators: every element of every buffer against the oracle's
    or_flush_buffers ([DS] problem statement: copy-in and copy-out around
    the bucket)."""
    from tests import test_gpu_flush_buffers as FB

    sizes = st.lists(st.one_of(st.integers(0, 20), st.integers(0, 5000),
                               st.sampled_from([64, 1000, 4099, 8197])), min_size=1, max_size=16)

    @settings(max_examples=80, deadline=None, derandomize=True)
    @given(st.sampled_from(FB.CASES), sizes, st.integers(0, 10 ** 6),
           st.sampled_from([(True, True), (True, False), (False, True)]), st.booleans(),
           st.booleans())
    def run(case, numel, seed, aligned_padded, inplace, planned):
        W, dtype, pre, comms = case
        FB.run_case(W, dtype, pre, comms, numel, seed, aligned_padded[0], aligned_padded[1], inplace,
                    planned=planned)

    run()


@st.composite
def flush_workloads(draw):
    W = draw(st.sampled_from([1, 2, 3, 4, 6, 8, 12, 16, 32, 64]))
    dtype = draw(st.sampled_from([wl.DT_BF16, wl.DT_F32]))
    sizes = draw(st.lists(st.one_of(st.integers(0, 20), st.integers(0, 4000),
                                    st.sampled_from([512, 1024, 4096, 9000])), min_size=1, max_size=50))
    P = len(sizes)
    a = draw(st.integers(0, P))
    b = draw(st.integers(a, P))
    comms = [wl.Comm(W, 1)]
    divs = [c for c in range(1, W) if W % c == 0]
    group_comm = [0, 0, 0]
    if divs and draw(st.booleans()):
        c = draw(st.sampled_from(divs))
        comms.append(wl.Comm(c, draw(st.sampled_from([1, W // c]))))
        group_comm[2] = 1
    return wl.custom_flush("drawn", W, dtype, sizes, group_begin=[0, a, b, P], group_comm=group_comm,
                           comms=comms, capacity=draw(st.sampled_from([700, 6000, 40_000, 10 ** 6])),
                           pre_div=draw(st.integers(0, 1)), value_seed=draw(st.integers(0, 1000)),
                           arrival=draw(st.permutations(list(range(P)))))


def test_owner_map_flush_and_probe_on_drawn_workloads():
    """Drawn workloads -- three parameter groups (one possibly on a
    sub-communicator), empty and one-element tensors, any arrival order and
    bucket capacity -- through the executor: partition lists, owner map and
    counts, the flush of every bucket (AllReduce, reduce-to-owner or ZeRO-2;
    searched, host-planned or device-planned) and the probe records, all
    against the oracle ([DS] Design points, problem statement)."""
    from tests import test_gpu_flush as F

    @settings(max_examples=60, deadline=None, derandomize=True)
    @given(flush_workloads(), st.sampled_from(["allreduce", "owner", "zero2"]),
           st.sampled_from([False, True, "device"]))
    def run(w, mode, planned):
        F.test_partition_ids_and_owner_map(w)
        F.flush_case(w, mode == "owner", zero2=mode == "zero2", planned=planned)

    run()
