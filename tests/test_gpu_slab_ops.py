"""GPU parity for reduce-scatter, all-gather (rank and ring order, step
replay), replica-local accumulation and the deferred reduce, through the C
ABI, against the CPU oracle.  Bit-exact, except the deferred-vs-per-micro-
batch comparison, which is two different summation orders and is held to
5e-5 * sum|x| per element."""
import numpy as np
import pytest

import oracle
import synth
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


RS_CASES = [(8, wl.DT_BF16, 8 * 5000, 0), (8, wl.DT_BF16, 8 * 4097, 1), (4, wl.DT_F32, 4 * 9999, 1),
            (3, wl.DT_BF16, 3 * 2001, 1), (16, wl.DT_F32, 16 * 1024, 0), (5, wl.DT_F32, 5 * 333, 0),
            (1, wl.DT_BF16, 800, 1), (2, wl.DT_BF16, 0, 0), (64, wl.DT_BF16, 64 * 1001, 1),
            (64, wl.DT_F32, 64 * 512, 0)]


@pytest.mark.parametrize("W,dtype,M,pre", RS_CASES, ids=lambda v: str(v))
def test_reduce_scatter_then_all_gather(W, dtype, M, pre):
    import torch
    U.say("rs/ag", W, dtype, M, pre)
    L = M // W
    ld_in = max(64, wl.round_up(M, 64))
    ld_sh = max(64, wl.round_up(L, 64))
    scale = wl.sigma_scale(1e-2)
    x = U.gen_slab(dtype, W, ld_in, M, 4, 0, scale)
    sh = U.empty_slab(dtype, W, ld_sh)
    dc.dc_reduce_scatter(W, dtype, x, ld_in, sh, ld_sh, M, pre)
    outs = {}
    for order in (dc.DC_ORDER_RANK, dc.DC_ORDER_RING):
        o = U.empty_slab(dtype, W, ld_in)
        dc.dc_all_gather(W, dtype, sh, ld_sh, o, ld_in, L, order, -1)
        outs[order] = o
    torch.cuda.synchronize()
    hx = U.host_slab(dtype, W, ld_in, M, 4, 0, scale)
    hsh = np.zeros((W, ld_sh), hx.dtype)
    U.bits(hsh, dtype)[:] = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
    oracle.reduce_scatter(W, dtype, hx, hsh, M, pre)
    assert np.array_equal(U.bits(U.to_host(sh, dtype), dtype), U.bits(hsh, dtype))
    for order, o in outs.items():
        ho = np.zeros((W, ld_in), hx.dtype)
        U.bits(ho, dtype)[:] = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
        oracle.all_gather(W, dtype, hsh, ho, L, order)
        assert np.array_equal(U.bits(U.to_host(o, dtype), dtype), U.bits(ho, dtype)), order


@pytest.mark.parametrize("W,dtype,L", [(4, wl.DT_BF16, 1000), (8, wl.DT_F32, 333), (5, wl.DT_BF16, 77)])
def test_all_gather_ring_step_replay(W, dtype, L):
    """Replaying the ring one step at a time rebuilds the full ring layout,
    and after step s exactly positions 0..s are written."""
    import torch
    ld_sh = wl.round_up(L, 64)
    ld = wl.round_up(W * L, 64)
    sh = U.gen_slab(dtype, W, ld_sh, L, 6, 0, wl.sigma_scale(1e-2))
    full = U.empty_slab(dtype, W, ld)
    dc.dc_all_gather(W, dtype, sh, ld_sh, full, ld, L, dc.DC_ORDER_RING, -1)
    part = U.empty_slab(dtype, W, ld)
    hsh = U.host_slab(dtype, W, ld_sh, L, 6, 0, wl.sigma_scale(1e-2))
    for s in range(W):
        dc.dc_all_gather(W, dtype, sh, ld_sh, part, ld, L, dc.DC_ORDER_RING, s)
        torch.cuda.synchronize()
        ho = np.zeros((W, ld), hsh.dtype)
        U.bits(ho, dtype)[:] = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
        for q in range(s + 1):
            oracle.all_gather(W, dtype, hsh, ho, L, 1, q)
        assert np.array_equal(U.bits(U.to_host(part, dtype), dtype), U.bits(ho, dtype)), s
    assert torch.equal(part, full)
    # rank order, chunk by chunk
    rk = U.empty_slab(dtype, W, ld)
    for s in range(W):
        dc.dc_all_gather(W, dtype, sh, ld_sh, rk, ld, L, dc.DC_ORDER_RANK, s)
    full_rank = U.empty_slab(dtype, W, ld)
    dc.dc_all_gather(W, dtype, sh, ld_sh, full_rank, ld, L, dc.DC_ORDER_RANK, -1)
    torch.cuda.synchronize()
    assert torch.equal(rk, full_rank)


def _as_f64(a, dtype):
    if dtype == wl.DT_BF16:
        return oracle.bf16_to_f32(a.view(np.uint16)).astype(np.float64)
    return a.astype(np.float64)


RING_CASES = RS_CASES + [(8, wl.DT_BF16, 8 * 1001, 1), (4, wl.DT_F32, 4 * 1001, 0),
                         (7, wl.DT_F32, 7 * 4096, 1), (64, wl.DT_BF16, 64 * 64, 1)]


@pytest.mark.parametrize("W,dtype,M,pre", RING_CASES, ids=lambda v: str(v))
def test_reduce_scatter_ring(W, dtype, M, pre):
    """Ring-order reduce-scatter bit-exact against the oracle's simulated
    ring; the distance to the rank-order shards is reported, not bounded
    beyond the fold error bound (both are correct sums in different orders)."""
    import torch
    U.say("ring rs", W, dtype, M, pre)
    L = M // W
    ld_in = max(64, wl.round_up(M, 64))
    ld_sh = max(64, wl.round_up(L, 64))
    scale = wl.sigma_scale(1e-2)
    x = U.gen_slab(dtype, W, ld_in, M, 14, 0, scale)
    sh = U.empty_slab(dtype, W, ld_sh)
    dc.dc_reduce_scatter_ring(W, dtype, x, ld_in, sh, ld_sh, M, pre)
    rk = U.empty_slab(dtype, W, ld_sh)
    dc.dc_reduce_scatter(W, dtype, x, ld_in, rk, ld_sh, M, pre)
    torch.cuda.synchronize()
    hx = U.host_slab(dtype, W, ld_in, M, 14, 0, scale)
    hsh = np.zeros((W, ld_sh), hx.dtype)
    U.bits(hsh, dtype)[:] = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
    oracle.reduce_scatter_ring(W, dtype, hx, hsh, M, pre)
    got = U.to_host(sh, dtype)
    assert np.array_equal(U.bits(got, dtype), U.bits(hsh, dtype))
    if L:
        a = _as_f64(got[:, :L], dtype)
        b = _as_f64(U.to_host(rk, dtype)[:, :L], dtype)
        U.say("  ring vs rank order: max |diff| / max |x| =",
              float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30)))


def test_reduce_scatter_ring_7b_layer_full_size():
    """The 7B-layer workload at full size, ring order, on sampled columns:
    the sampled columns of every shard are gathered into a small slab whose
    chunk s holds shard s's samples, so the oracle's ring folds them starting
    at the same rank."""
    import torch
    w = wl.rs_ag_w8()
    W, M, dtype = w.W, w.M, w.dtype
    L = M // W
    U.say("ring rs full size", M)
    x = U.gen_slab(dtype, W, w.ld, M, w.value_seed, 0, w.scale)
    ld_sh = wl.round_up(L, 64)
    sh = U.empty_slab(dtype, W, ld_sh)
    dc.dc_reduce_scatter_ring(W, dtype, x, w.ld, sh, ld_sh, M, 1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    ks = np.unique(np.concatenate([[0, 7, 8, L - 1], rng.integers(0, L, 2000)]))
    n = len(ks)
    got = sh[:, torch.from_numpy(ks).cuda()].cpu().numpy().view(np.uint16)
    cols = np.concatenate([s * L + ks for s in range(W)])
    slab = np.stack([synth.gather(dtype, w.value_seed, r, w.scale, cols) for r in range(W)])
    out = np.zeros((W, n), np.uint16)
    oracle.reduce_scatter_ring(W, dtype, slab, out, W * n, 1)
    assert np.array_equal(got, out)


AGS_CASES = [(W, dtype, L, algo) for (W, dtype, L) in
             [(4, wl.DT_BF16, 1000), (8, wl.DT_F32, 333), (5, wl.DT_BF16, 77), (16, wl.DT_BF16, 2048),
              (1, wl.DT_F32, 64), (2, wl.DT_BF16, 9), (3, wl.DT_F32, 0), (64, wl.DT_BF16, 100),
              (32, wl.DT_F32, 33)]
             for algo in (dc.DC_SCHED_RING, dc.DC_SCHED_BIDIR, dc.DC_SCHED_RD)
             if algo != dc.DC_SCHED_RD or W & (W - 1) == 0]


@pytest.mark.parametrize("W,dtype,L,algo", AGS_CASES, ids=lambda v: str(v))
def test_all_gather_step_schedules(W, dtype, L, algo):
    """Every step of the ring, bidirectional-ring and recursive-doubling
    schedules against the oracle's step executor (bit-exact, including the
    chunks not yet delivered, which keep the sentinel); the finished buffer
    is the rank-order gather."""
    import torch
    U.say("ag step", W, dtype, L, algo)
    ld_sh = max(64, wl.round_up(L, 64))
    ld = max(64, wl.round_up(W * L, 64))
    scale = wl.sigma_scale(1e-2)
    sh = U.gen_slab(dtype, W, ld_sh, L, 16, 0, scale)
    hsh = U.host_slab(dtype, W, ld_sh, L, 16, 0, scale)
    out = U.empty_slab(dtype, W, ld)
    ho = np.zeros((W, ld), hsh.dtype)
    U.bits(ho, dtype)[:] = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
    steps = {dc.DC_SCHED_RING: W - 1, dc.DC_SCHED_BIDIR: W // 2,
             dc.DC_SCHED_RD: W.bit_length() - 1}[algo]
    compare_every = W <= 16
    for s in range(steps + 1):
        dc.dc_all_gather_step(W, dtype, sh, ld_sh, out, ld, L, algo, s)
        oracle.all_gather_step(W, dtype, hsh, ho, L, algo, s)
        if compare_every or s == steps:
            torch.cuda.synchronize()
            assert np.array_equal(U.bits(U.to_host(out, dtype), dtype), U.bits(ho, dtype)), s
    rank = U.empty_slab(dtype, W, ld)
    dc.dc_all_gather(W, dtype, sh, ld_sh, rank, ld, L, dc.DC_ORDER_RANK, -1)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :W * L], rank[:, :W * L])


RING_AR_CASES = [(8, wl.DT_BF16, 1000, 0), (8, wl.DT_BF16, 1000, 1), (4, wl.DT_F32, 333, 0),
                 (5, wl.DT_BF16, 77, 1), (16, wl.DT_F32, 2048, 0), (2, wl.DT_BF16, 9, 0),
                 (1, wl.DT_F32, 64, 1), (64, wl.DT_BF16, 100, 0)]


@pytest.mark.parametrize("W,dtype,L,pre", RING_AR_CASES, ids=lambda v: str(v))
def test_ring_allreduce_composition(W, dtype, L, pre):
    """A ring AllReduce on one GPU: the ring-order reduce-scatter followed by
    every step of the ring all-gather schedule.  Bit-exact against the
    oracle's ring reduce-scatter and step executor; every row of the result
    holds the same vector; against the rank-order AllReduce of the flush it
    differs only within the error bound of two fp32 summation orders (plus
    one bf16 rounding of each side)."""
    import torch
    U.say("ring allreduce", W, dtype, L, pre)
    M = W * L
    ld = max(64, wl.round_up(M, 64))
    ld_sh = max(64, wl.round_up(L, 64))
    scale = wl.sigma_scale(1e-2)
    x = U.gen_slab(dtype, W, ld, M, 21, 0, scale)
    hx = U.host_slab(dtype, W, ld, M, 21, 0, scale)
    sh = U.empty_slab(dtype, W, ld_sh)
    out = U.empty_slab(dtype, W, ld)
    dc.dc_reduce_scatter_ring(W, dtype, x, ld, sh, ld_sh, M, pre)
    for s in range(W):
        dc.dc_all_gather_step(W, dtype, sh, ld_sh, out, ld, L, dc.DC_SCHED_RING, s)
    ar = U.empty_slab(dtype, W, ld)
    if M:
        tasks = dc.tasks_array([(0, M, 0, 0)])
        d_tasks = torch.from_numpy(tasks.view(np.uint8).copy()).cuda()
        dc.dc_flush_bucket(W, dtype, x, ld, ar, ld, 0, M, d_tasks, 1, None, 1, [(W, 1)], 1, pre)
    torch.cuda.synchronize()

    hsh = np.zeros((W, ld_sh), hx.dtype)
    oracle.reduce_scatter_ring(W, dtype, hx, hsh, M, pre)
    ho = np.zeros((W, ld), hx.dtype)
    U.bits(ho, dtype)[:] = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
    for s in range(W):
        oracle.all_gather_step(W, dtype, hsh, ho, L, oracle.AG_RING, s)
    got = U.to_host(out, dtype)
    assert np.array_equal(U.bits(got, dtype)[:, :M], U.bits(ho, dtype)[:, :M])
    for i in range(1, W):
        assert np.array_equal(U.bits(got, dtype)[i, :M], U.bits(got, dtype)[0, :M]), i
    if M and not pre:
        a = _as_f64(got[0, :M], dtype)
        b = _as_f64(U.to_host(ar, dtype)[0, :M], dtype)
        mag = np.sum(np.abs(_as_f64(hx[:, :M], dtype)), axis=0)
        tol = 2.0 * (W - 1) * 2.0 ** -24 * mag * 1.01
        if dtype == wl.DT_BF16:
            tol = tol + 2.0 ** -8 * (np.abs(a) + np.abs(b)) * 1.01
        assert np.all(np.abs(a - b) <= tol)
        U.say("  ring vs rank order: elements that differ", int(np.count_nonzero(a != b)), "of", M)


def test_reduce_scatter_all_gather_7b_layer_full_size():
    """The 7B-layer workload at full size (M = 202,383,360, W = 8): shards on
    sampled columns against the oracle, then AllReduce = ReduceScatter +
    AllGather checked against the flush's AllReduce of the same slab."""
    import torch
    w = wl.rs_ag_w8()
    W, M, dtype = w.W, w.M, w.dtype
    L = M // W
    U.say("rs/ag full size", M)
    x = U.gen_slab(dtype, W, w.ld, M, w.value_seed, 0, w.scale)
    ld_sh = wl.round_up(L, 64)
    sh = U.empty_slab(dtype, W, ld_sh)
    dc.dc_reduce_scatter(W, dtype, x, w.ld, sh, ld_sh, M, 0)
    full = U.empty_slab(dtype, W, w.ld)
    dc.dc_all_gather(W, dtype, sh, ld_sh, full, w.ld, L, dc.DC_ORDER_RANK, -1)
    ar = U.empty_slab(dtype, W, w.ld)
    tasks = dc.tasks_array([(0, M, 0, 0)])
    d_tasks = torch.from_numpy(tasks.view(np.uint8).copy()).cuda()
    dc.dc_flush_bucket(W, dtype, x, w.ld, ar, w.ld, 0, M, d_tasks, 1, None, 1, [(W, 1)], 1, 0)
    torch.cuda.synchronize()
    assert torch.equal(full[:, :M], ar[:, :M])
    rng = np.random.default_rng(1)
    ks = np.unique(np.concatenate([[0, L - 1], rng.integers(0, L, 3000)]))
    got = sh[:, torch.from_numpy(ks).cuda()].cpu().numpy().view(np.uint16)
    for s in range(W):
        cols = s * L + ks
        rows = np.stack([synth.gather(dtype, w.value_seed, r, w.scale, cols) for r in range(W)])
        ld = wl.round_up(len(ks) * W, 8)
        slab = np.zeros((W, ld), np.uint16)
        slab[:, :len(ks)] = rows
        out = np.zeros((1, ld), np.uint16)
        # the shard sums of these columns: a one-task flush of the gathered columns
        tmp = np.zeros((W, ld), np.uint16)
        oracle.flush(W, dtype, slab, tmp, 0, [0], [len(ks)], [0], [0], None, [W], [1], 0)
        out[0] = tmp[0]
        assert np.array_equal(got[s], out[0, :len(ks)]), s


@pytest.mark.parametrize("rows,M,init,alias", [(4, 1001, 1, False), (4, 1001, 0, False),
                                               (3, 4096, 0, True), (1, 7, 1, False),
                                               (4, 0, 0, False)])
def test_accumulate(rows, M, init, alias):
    import torch
    ld = wl.round_up(max(M, 1), 64)
    scale = wl.sigma_scale(1e-3)
    x = U.gen_slab(wl.DT_F32, rows, ld, M, 11, 0, scale).view(torch.float32)
    acc = U.gen_slab(wl.DT_F32, rows, ld, M, 12, 0, scale).view(torch.float32)
    hx = U.host_slab(wl.DT_F32, rows, ld, M, 11, 0, scale)
    hacc = U.host_slab(wl.DT_F32, rows, ld, M, 12, 0, scale)
    if M:
        x[0, 0] = -0.0
        hx[0, 0] = -0.0
    if alias:
        dc.dc_accumulate(rows, acc, ld, acc, ld, M, init)
        oracle.accumulate(rows, hacc, hacc, M, init)
    else:
        dc.dc_accumulate(rows, x, ld, acc, ld, M, init)
        oracle.accumulate(rows, hx, hacc, M, init)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().view(np.uint32), hacc.view(np.uint32))


@pytest.mark.parametrize("W,M,out_rows,alias", [(4, 1003, 1, False), (4, 1003, 4, False),
                                                (3, 500, 3, False), (16, 4096, 1, False),
                                                (4, 2048, 4, True), (8, 5, 1, False),
                                                (64, 999, 1, False), (64, 256, 64, False)])
def test_deferred_reduce(W, M, out_rows, alias):
    import torch
    ld = wl.round_up(M, 64)
    scale = wl.sigma_scale(1e-3)
    acc = U.gen_slab(wl.DT_F32, W, ld, M, 13, 0, scale).view(torch.float32)
    hacc = U.host_slab(wl.DT_F32, W, ld, M, 13, 0, scale)
    out = acc if alias else U.empty_slab(wl.DT_F32, out_rows, ld).view(torch.float32)
    hout = hacc if alias else np.full((out_rows, ld), np.uint32(U.SENTINEL32)).view(np.float32)
    dc.dc_deferred_reduce(W, acc, ld, out, ld, M, out_rows)
    oracle.deferred_reduce(W, hacc, hout, M, out_rows)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), hout.view(np.uint32))


@pytest.mark.parametrize("K", [1, 4, 8])
def test_deferred_ga_qwen3_full_size(K):
    """qwen3-0.6b tree, W = 4 replicas, K micro-batches generated on the
    device.  Deferred path (K accumulates, one reduce) against the status quo
    (per micro-batch reduce, then accumulate): bit-exact against the oracle on
    sampled columns for both paths, and D within 5e-5 * sum|x| of A on every
    column (bit-exact at K = 1)."""
    import torch
    w = wl.deferred_ga_w4(K)
    W, M, ld = w.W, w.M, w.ld
    U.say("deferred full size", K, M)
    acc = torch.empty((W, ld), dtype=torch.float32, device="cuda")
    A = torch.empty((1, ld), dtype=torch.float32, device="cuda")
    g = torch.empty((1, ld), dtype=torch.float32, device="cuda")
    S = torch.zeros((M,), dtype=torch.float64, device="cuda")
    x = torch.empty((W, ld), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for k in range(K):
        synth.fill_slab_device(wl.DT_F32, w.value_seed, wl.microbatch_stream(k, W, 0), w.scale, W,
                               ld, M, x.data_ptr(), stream)
        xf = x.view(torch.float32)
        dc.dc_accumulate(W, xf, ld, acc, ld, M, 1 if k == 0 else 0)
        dc.dc_deferred_reduce(W, xf, ld, g, ld, M, 1)
        dc.dc_accumulate(1, g, ld, A, ld, M, 1 if k == 0 else 0)
        S += xf[:, :M].abs().double().sum(dim=0)
    D = torch.empty((W, ld), dtype=torch.float32, device="cuda")
    dc.dc_deferred_reduce(W, acc, ld, D, ld, M, W)
    torch.cuda.synchronize()
    for i in range(1, W):
        assert torch.equal(D[i, :M], D[0, :M])
    err = (D[0, :M].double() - A[0, :M].double()).abs()
    assert bool((err <= 5e-5 * S).all()), float((err / S.clamp_min(1e-300)).max())
    if K == 1:
        assert torch.equal(D[0, :M], A[0, :M])
    rng = np.random.default_rng(K)
    cols = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 4000)]))
    xs = []
    for k in range(K):
        xs.append(np.stack([synth.gather(wl.DT_F32, w.value_seed, wl.microbatch_stream(k, W, r),
                                         w.scale, cols) for r in range(W)]).view(np.float32))
    n = len(cols)
    hacc = np.zeros((W, n), np.float32)
    hA = np.zeros((1, n), np.float32)
    for k, xk in enumerate(xs):
        oracle.accumulate(W, np.ascontiguousarray(xk), hacc, n, 1 if k == 0 else 0)
        hg = np.zeros((1, n), np.float32)
        oracle.deferred_reduce(W, np.ascontiguousarray(xk), hg, n, 1)
        oracle.accumulate(1, hg, hA, n, 1 if k == 0 else 0)
    hD = np.zeros((1, n), np.float32)
    oracle.deferred_reduce(W, hacc, hD, n, 1)
    tc = torch.from_numpy(cols).cuda()
    assert np.array_equal(D[0, tc].cpu().numpy().view(np.uint32), hD[0].view(np.uint32))
    assert np.array_equal(A[0, tc].cpu().numpy().view(np.uint32), hA[0].view(np.uint32))


@pytest.mark.parametrize("R,NW", [(4, 1), (8, 8), (16, 1)])
def test_stream_rows_reference(R, NW):
    """The access-mix reference kernel stores the xor of the R rows."""
    import torch
    nvec = 1000
    ld = wl.round_up(nvec * 4, 64)
    x = U.gen_slab(wl.DT_F32, R, ld, ld, 21, 0, wl.sigma_scale(1e-3))
    y = U.empty_slab(wl.DT_F32, R, ld)
    dc.dc_stream_rows(x, ld // 4, R, y, ld // 4, NW, nvec)
    torch.cuda.synchronize()
    hx = x.cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(hx[:, :nvec * 4], axis=0)
    got = y.cpu().numpy().view(np.uint32)
    for r in range(NW):
        assert np.array_equal(got[r, :nvec * 4], want)
    assert np.all(got[NW:, :] == U.SENTINEL32) and np.all(got[:, nvec * 4:] == U.SENTINEL32)


@pytest.mark.parametrize("R,NW", [(4, 1), (8, 8), (16, 16), (1, 8), (1, 16), (8, 1), (8, 4)])
@pytest.mark.parametrize("group,cap", [(1, 0), (2, 8), (4, 6)])
def test_stream_rows_shaped_reference(R, NW, group, cap):
    """The shaped access-mix reference (every launch shape the bench sweeps,
    one row read to every row written included) stores the xor of the R rows
    in NW rows, over full runs of 64 vectors and a ragged tail."""
    import torch
    nvec = 64 * group * 7 + 37
    ld = wl.round_up(nvec * 4, 64)
    x = U.gen_slab(wl.DT_F32, R, ld, ld, 23, 0, wl.sigma_scale(1e-3))
    rows = max(NW, 2)
    y = U.empty_slab(wl.DT_F32, rows, ld)
    dc.dc_stream_rows_shaped(x, ld // 4, R, y, ld // 4, NW, nvec, group, cap)
    torch.cuda.synchronize()
    hx = x.cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(hx[:, :nvec * 4], axis=0)
    got = y.cpu().numpy().view(np.uint32)
    for r in range(NW):
        assert np.array_equal(got[r, :nvec * 4], want), r
    assert np.all(got[NW:, :] == U.SENTINEL32) and np.all(got[:, nvec * 4:] == U.SENTINEL32)


AR_CASES = [(4, 1003, 0, 1, 4, "none"), (4, 1003, 1, 0, 1, "none"), (3, 517, 0, 0, 3, "out=acc"),
            (16, 4100, 0, 1, 1, "none"), (8, 2048, 1, 1, 8, "x=acc"), (5, 33, 0, 1, 5, "none"),
            (4, 0, 0, 0, 1, "none")]


@pytest.mark.parametrize("W,M,init,keep,out_rows,alias", AR_CASES, ids=lambda v: str(v))
def test_accumulate_reduce_equals_two_steps(W, M, init, keep, out_rows, alias):
    """The fused last-micro-batch kernel against the oracle's accumulate
    followed by its deferred reduce: bit-exact outputs and accumulator."""
    import torch
    ld = wl.round_up(max(M, 1), 64)
    scale = wl.sigma_scale(1e-3)
    x = U.gen_slab(wl.DT_F32, W, ld, M, 31, 0, scale).view(torch.float32)
    acc = U.gen_slab(wl.DT_F32, W, ld, M, 32, 0, scale).view(torch.float32)
    hx = U.host_slab(wl.DT_F32, W, ld, M, 31, 0, scale)
    hacc = U.host_slab(wl.DT_F32, W, ld, M, 32, 0, scale)
    if alias == "x=acc":
        x, hx = acc, hacc
    out = acc if alias == "out=acc" else U.empty_slab(wl.DT_F32, out_rows, ld).view(torch.float32)
    dc.dc_accumulate_reduce(W, x, ld, acc, ld, init, keep, out, ld, out_rows, M)
    torch.cuda.synchronize()
    a2 = hacc.copy()
    oracle.accumulate(W, hx.copy() if alias == "x=acc" else hx, a2, M, init)
    want = np.full((out_rows, ld), np.uint32(U.SENTINEL32)).view(np.float32)
    oracle.deferred_reduce(W, a2, want, M, out_rows)
    got = out.cpu().numpy()
    if alias == "out=acc":
        assert np.array_equal(got[:out_rows, :M].view(np.uint32), want[:, :M].view(np.uint32))
    else:
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        wacc = a2 if keep else hacc
        assert np.array_equal(acc.cpu().numpy().view(np.uint32), wacc.view(np.uint32))


def test_all_gather_schedules_7b_layer_full_size():
    """The 7B-layer slab (W = 8, L = 25,297,920 bf16): every schedule's
    finished buffer equals the one-shot rank-order gather bit for bit, and
    after step 1 of the ring exactly two chunks per node are placed (the
    rest keep the sentinel)."""
    import torch
    w = wl.rs_ag_w8()
    W, M, dtype = w.W, w.M, w.dtype
    L = M // W
    U.say("ag schedules full size", M)
    x = U.gen_slab(dtype, W, w.ld, M, w.value_seed, 0, w.scale)
    ld_sh = wl.round_up(L, 64)
    sh = U.empty_slab(dtype, W, ld_sh)
    dc.dc_reduce_scatter(W, dtype, x, w.ld, sh, ld_sh, M, 1)
    del x
    want = U.empty_slab(dtype, W, w.ld)
    dc.dc_all_gather(W, dtype, sh, ld_sh, want, w.ld, L, dc.DC_ORDER_RANK, -1)
    steps = {dc.DC_SCHED_RING: W - 1, dc.DC_SCHED_BIDIR: W // 2, dc.DC_SCHED_RD: 3}
    for algo, S in steps.items():
        out = U.empty_slab(dtype, W, w.ld)
        for s in range(S + 1):
            dc.dc_all_gather_step(W, dtype, sh, ld_sh, out, w.ld, L, algo, s)
            if algo == dc.DC_SCHED_RING and s == 1:
                torch.cuda.synchronize()
                for i in range(W):
                    for c in range(W):
                        blk = out[i, c * L:(c + 1) * L]
                        placed = c in (i, (i - 1) % W)
                        if placed:
                            assert torch.equal(blk, want[i, c * L:(c + 1) * L]), (i, c)
                        else:
                            assert bool((blk == U.SENTINEL16).all()), (i, c)
        torch.cuda.synchronize()
        assert torch.equal(out[:, :M], want[:, :M]), algo
        del out


def test_accumulator_lifetime_restore_and_round_trip():
    """MaxText PR, accumulator lifetime, on the GPU kernels: a reduced total
    restored onto replica 0 (zeros elsewhere) reduces back to itself; a
    mid-step save / restore / continue sequence matches the oracle's same
    sequence bit for bit and stays within the 5e-5 * sum|x| gate of the
    uninterrupted step."""
    import torch
    W, K, M = 4, 8, 5001
    ld = wl.round_up(M, 64)
    scale = wl.sigma_scale(1e-3)
    xs = [U.gen_slab(wl.DT_F32, W, ld, M, 81, wl.microbatch_stream(k, W, 0), scale).view(torch.float32)
          for k in range(K)]
    hxs = [U.host_slab(wl.DT_F32, W, ld, M, 81, wl.microbatch_stream(k, W, 0), scale) for k in range(K)]

    def gpu_deferred(chunks, acc=None):
        acc = torch.zeros((W, ld), dtype=torch.float32, device="cuda") if acc is None else acc
        for x in chunks:
            dc.dc_accumulate(W, x, ld, acc, ld, M, 0)
        D = torch.empty((1, ld), dtype=torch.float32, device="cuda")
        dc.dc_deferred_reduce(W, acc, ld, D, ld, M, 1)
        return D, acc

    def host_deferred(chunks, acc=None):
        acc = np.zeros((W, ld), np.float32) if acc is None else acc
        for x in chunks:
            oracle.accumulate(W, x, acc, M, 0)
        D = np.zeros((1, ld), np.float32)
        oracle.deferred_reduce(W, acc, D, M, 1)
        return D, acc

    D_full, _ = gpu_deferred(xs)
    D_save, _ = gpu_deferred(xs[:3])
    acc = torch.zeros((W, ld), dtype=torch.float32, device="cuda")
    acc[0, :M] = D_save[0, :M]
    D_rt, _ = gpu_deferred(xs[3:], acc)
    # restore alone: the saved total reduces back to itself
    acc2 = torch.zeros((W, ld), dtype=torch.float32, device="cuda")
    acc2[0, :M] = D_save[0, :M]
    D_back = torch.empty((1, ld), dtype=torch.float32, device="cuda")
    dc.dc_deferred_reduce(W, acc2, ld, D_back, ld, M, 1)
    torch.cuda.synchronize()
    h_full, _ = host_deferred(hxs)
    h_save, _ = host_deferred(hxs[:3])
    hacc = np.zeros((W, ld), np.float32)
    hacc[0, :M] = h_save[0, :M]
    h_rt, _ = host_deferred(hxs[3:], hacc)
    assert np.array_equal(D_full[0, :M].cpu().numpy().view(np.uint32), h_full[0, :M].view(np.uint32))
    assert np.array_equal(D_rt[0, :M].cpu().numpy().view(np.uint32), h_rt[0, :M].view(np.uint32))
    saved = D_save[0, :M].cpu().numpy()
    want_back = np.where(saved == 0, np.float32(0.0), saved)
    assert np.array_equal(D_back[0, :M].cpu().numpy().view(np.uint32), want_back.view(np.uint32))
    S = sum(np.abs(x[:, :M].astype(np.float64)).sum(axis=0) for x in hxs)
    err = np.abs(D_rt[0, :M].cpu().numpy().astype(np.float64) - D_full[0, :M].cpu().numpy())
    assert np.all(err <= 5e-5 * S)


@pytest.mark.parametrize("W,out_rows", [(4, 1), (4, 4), (3, 3), (8, 1)])
def test_deferred_reducer_steps_and_lifetime(W, out_rows):
    """gradient_reduction_amd.deferred.DeferredReducer ([MT] What, accumulator
    lifetime): a step of K micro-batches reduced at update() equals the
    oracle's accumulate-then-reduce bit for bit; the fused last micro-batch
    gives the same; a second step starts from zero; and a state saved after
    two micro-batches, restored into a fresh reducer, finishes the step with
    the uninterrupted step's result."""
    import torch
    from gradient_reduction_amd.deferred import DeferredReducer
    M, K = 5000 + W, 4
    ld = wl.round_up(M, 64)
    scale = wl.sigma_scale(1e-2)
    xs = [U.gen_slab(wl.DT_F32, W, ld, M, 900 + W, k * W, scale) for k in range(K)]
    hxs = [U.host_slab(wl.DT_F32, W, ld, M, 900 + W, k * W, scale) for k in range(K)]
    h_acc = np.zeros((W, ld), np.float32)
    for k in range(K):
        oracle.accumulate(W, hxs[k], h_acc, M, 1 if k == 0 else 0)
    want = np.zeros((out_rows, ld), np.float32)
    oracle.deferred_reduce(W, h_acc, want, M, out_rows)
    U.say("deferred reducer", W, out_rows)

    def bits(t):
        return t.cpu().numpy()[:, :M].view(np.uint32)

    red = DeferredReducer(W, M, ld)
    for step in range(2):                 # the second step must start from zero
        for k in range(K):
            red.accumulate(xs[k], ld)
        out = torch.zeros((out_rows, ld), dtype=torch.float32, device="cuda")
        red.reduce(out, ld, out_rows)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), want[:, :M].view(np.uint32)), step
    for k in range(K - 1):                # the last micro-batch fused into the reduce
        red.accumulate(xs[k], ld)
    out = torch.zeros((out_rows, ld), dtype=torch.float32, device="cuda")
    red.reduce(out, ld, out_rows, last=xs[K - 1], ld_last=ld, keep_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), want[:, :M].view(np.uint32))
    assert np.array_equal(bits(red.acc), h_acc[:, :M].view(np.uint32))
    red.accumulate(xs[0], ld)             # save mid-step, restore elsewhere, finish
    red.accumulate(xs[1], ld)
    state = red.state_dict()
    other = DeferredReducer(W, M, ld)
    other.load_state_dict(state)
    for k in range(2, K):
        other.accumulate(xs[k], ld)
    out = torch.zeros((out_rows, ld), dtype=torch.float32, device="cuda")
    other.reduce(out, ld, out_rows)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), want[:, :M].view(np.uint32))
    with pytest.raises(RuntimeError):
        other.reduce(out, ld, out_rows)   # a new step has no micro-batch yet
