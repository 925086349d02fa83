"""GPU parity of the flush with copy-in and copy-out fused in
(dc_flush_bucket_buffers) against the oracle's or_flush_buffers: every
element of every output buffer bit-exact, and every element outside the
buffers that exist (empty buffers, gaps) left as it was.

Small cases place each rank's buffers at random positions of one arena, with
16-byte aligned and unaligned starts and packed or vector-padded task
coordinates, so both the vector and the element paths run; the full-size
cases run the W=8 402.8M-element bf16 and W=16 1.2e9-element fp32 workloads
through the executor and check sampled elements."""
import random

import numpy as np
import pytest

import oracle
import synth
from gradient_reduction_amd import dc, executor
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


def _place(rng, sizes, step):
    """Disjoint offsets in shuffled order; step > 1 rounds every start up to a
    multiple of step, step == 1 leaves random 0-3 element gaps."""
    order = list(range(len(sizes)))
    rng.shuffle(order)
    off = [0] * len(sizes)
    pos = rng.randint(0, 3)
    for k in order:
        if step > 1:
            pos = -(-pos // step) * step
        off[k] = pos
        pos += sizes[k] + rng.randint(0, 3)
    return off, pos + 1


def _dev_ptrs(base, offs, eb, mask=None):
    import torch
    a = np.asarray(offs, np.int64) * eb + base
    if mask is not None:
        a = np.where(mask, a, 0)
    return torch.from_numpy(a.ravel().astype(np.int64)).cuda()


CASES = [
    (4, wl.DT_BF16, 1, [(4, 1), (2, 1), (2, 2)]),
    (8, wl.DT_F32, 0, [(8, 1), (4, 1), (2, 4)]),
    (8, wl.DT_BF16, 1, [(8, 1), (4, 1), (2, 4)]),
    (6, wl.DT_F32, 1, [(6, 1), (3, 1), (2, 3)]),
    (16, wl.DT_BF16, 0, [(16, 1), (8, 2)]),
    (3, wl.DT_BF16, 1, [(3, 1)]),
    (2, wl.DT_BF16, 1, [(2, 1)]),
    (1, wl.DT_F32, 1, [(1, 1)]),
    (32, wl.DT_BF16, 1, [(32, 1), (8, 4)]),
    (64, wl.DT_F32, 0, [(64, 1), (16, 1)]),
]
NUMEL = [0, 1, 7, 8, 9, 64, 1000, 4099, 5000, 3, 8197, 16]


def run_case(W, dtype, pre, comms, numel, seed, aligned, padded, inplace, planned=False,
             stale=False):
    """stale: plan with random records instead of the planner's; then only
    the contract is checked: nothing outside the holders' buffers is written
    and the inputs are unchanged."""
    import torch
    rng = random.Random(seed)
    n = len(numel)
    E = 8 if dtype == wl.DT_BF16 else 4
    eb = 2 if dtype == wl.DT_BF16 else 4
    cs, cst = [c for c, _ in comms], [s for _, s in comms]
    t_comm = [rng.randrange(len(comms)) for _ in range(n)]
    for k in range(0, n, 3):
        t_comm[k] = 0
    hold = np.array([[rng.random() < 0.4 for _ in range(W)] for _ in range(n)])
    hold[min(2, n - 1)] = True
    hold[min(3, n - 1)] = False
    if n > 4:
        hold[4] = [r == W - 1 for r in range(W)]
    in_off, in_size = _place(rng, [numel[t] for t in range(n) for _ in range(W)], E if aligned else 1)
    in_off = np.array(in_off, np.int64).reshape(n, W)
    scale = wl.sigma_scale(1e-2)
    ld_in = wl.round_up(in_size, 64)
    d_in = U.gen_slab(dtype, 1, ld_in, in_size, seed, 0, scale)
    h_in = U.host_slab(dtype, 1, ld_in, in_size, seed, 0, scale)[0].copy()
    if inplace:
        out_off = np.where(hold, in_off, -1)
        d_out, h_out = d_in, h_in
    else:
        held = [(t, r) for t in range(n) for r in range(W) if hold[t, r]]
        o_off, out_size = _place(rng, [numel[t] for t, _ in held], E if aligned else 1)
        out_off = np.full((n, W), -1, np.int64)
        for (t, r), o in zip(held, o_off):
            out_off[t, r] = o
        ld_out = wl.round_up(out_size, 64)
        d_out = U.empty_slab(dtype, 1, ld_out)
        h_out = np.zeros(ld_out, h_in.dtype)
        U.bits(h_out, dtype)[:] = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
    pos, rows = 0, []
    for t in range(n):
        rows.append((pos, numel[t], t, t_comm[t]))
        pos += numel[t]
        if padded:
            pos = -(-pos // E) * E
    extent = rows[-1][0] + rows[-1][1]
    tasks = dc.tasks_array(rows)
    d_tasks = torch.from_numpy(tasks.view(np.uint8).copy()).cuda()
    p_in = _dev_ptrs(d_in.data_ptr(), in_off, eb)
    p_out = _dev_ptrs(d_out.data_ptr(), np.maximum(out_off, 0), eb, out_off >= 0)
    dc.dc_validate_buffer_tasks(W, dtype, tasks, n, extent, comms, len(comms),
                                p_in.cpu().numpy().view(np.uint64), p_out.cpu().numpy().view(np.uint64))
    U.say("flush buffers", W, dtype, pre, n, "aligned" if aligned else "unaligned",
          "padded" if padded else "packed", "in place" if inplace else "", "planned" if planned else "")
    if planned:
        tiles = dc.dc_plan_flush_buffers(W, dtype, extent, tasks, n, comms, len(comms))
        if stale:
            tiles["first"] = [rng.randint(-3, n + 3) for _ in range(len(tiles))]
            tiles["last"] = [rng.randint(-3, n + 3) for _ in range(len(tiles))]
            tiles["root"] = [rng.randint(-3, W + 3) for _ in range(len(tiles))]
            tiles["flags"] = [rng.randint(0, 1) | (rng.randint(0, 4) << 8) for _ in range(len(tiles))]
        d_tiles = torch.from_numpy(tiles.view(np.uint8).copy()).cuda() if len(tiles) else None
        dc.dc_flush_bucket_buffers_planned(W, dtype, extent, d_tasks, n, p_in, p_out, comms, len(comms),
                                           pre, d_tiles, len(tiles))
    else:
        dc.dc_flush_bucket_buffers(W, dtype, extent, d_tasks, n, p_in, p_out, comms, len(comms), pre)
    torch.cuda.synchronize()
    if stale:
        got = U.bits(U.to_host(d_out, dtype)[0], dtype)
        legit = np.zeros(len(got), bool)
        for t in range(n):
            for r in range(W):
                if out_off[t, r] >= 0:
                    legit[out_off[t, r]:out_off[t, r] + numel[t]] = True
        sent = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
        assert np.all(got[~legit] == sent), "a stale plan wrote outside the holders' buffers"
        assert np.array_equal(U.bits(U.to_host(d_in, dtype)[0], dtype), U.bits(h_in, dtype))
        return
    oracle.flush_buffers(W, dtype, h_in, in_off, h_out, out_off, numel, t_comm, cs, cst, pre)
    got = U.to_host(d_out, dtype)[0]
    assert np.array_equal(U.bits(got, dtype), U.bits(h_out, dtype))


@pytest.mark.parametrize("W,dtype,pre,comms", CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("aligned,padded", [(True, True), (True, False), (False, True)],
                         ids=["aligned-padded", "aligned-packed", "unaligned"])
@pytest.mark.parametrize("planned", [False, True], ids=["searched", "planned"])
def test_flush_buffers_small(W, dtype, pre, comms, aligned, padded, planned):
    run_case(W, dtype, pre, comms, NUMEL, 100 + W, aligned, padded, inplace=False, planned=planned)


@pytest.mark.parametrize("W,dtype,pre,comms", CASES[:4], ids=lambda v: str(v))
@pytest.mark.parametrize("planned", [False, True], ids=["searched", "planned"])
def test_flush_buffers_in_place(W, dtype, pre, comms, planned):
    run_case(W, dtype, pre, comms, NUMEL, 200 + W, True, True, inplace=True, planned=planned)


@pytest.mark.parametrize("W,dtype,pre,comms", CASES, ids=lambda v: str(v))
def test_flush_buffers_stale_plan_stays_in_buffers(W, dtype, pre, comms):
    """A plan of random records (the kernel reads the plan without checking
    it on the host): sums may be wrong, but nothing outside the holders'
    grad buffers is written and the inputs are left as they were."""
    for aligned, padded in ((True, True), (False, True)):
        run_case(W, dtype, pre, comms, NUMEL, 300 + W, aligned, padded, inplace=False, planned=True,
                 stale=True)


def test_flush_buffers_many_tiny_tasks():
    """Hundreds of tasks inside one launch tile: the per-tile task staging
    runs several rounds."""
    rng = random.Random(5)
    numel = [rng.randint(0, 9) for _ in range(700)]
    for planned in (False, True):
        run_case(8, wl.DT_BF16, 1, [(8, 1), (4, 1)], numel, 301, True, True, inplace=False,
                 planned=planned)
        run_case(6, wl.DT_F32, 0, [(6, 1), (2, 3)], numel, 302, False, False, inplace=False,
                 planned=planned)


def test_flush_buffers_empty():
    import torch
    dc.dc_flush_bucket_buffers(4, 0, 0, None, 0, None, None, [(4, 1)], 1, 0)
    t = torch.from_numpy(dc.tasks_array([(0, 0, 0, 0)]).view(np.uint8).copy()).cuda()
    z = torch.zeros(4, dtype=torch.int64, device="cuda")
    dc.dc_flush_bucket_buffers(4, 0, 0, t, 1, z, z, [(4, 1)], 1, 0)
    torch.cuda.synchronize()


def _check_sampled(w, d_out, ld, poff, pcol, hold):
    import torch
    cols = U.sample_columns(w)
    order = np.argsort(pcol)
    starts = pcol[order]
    k = np.searchsorted(starts, cols, side="right") - 1
    params = order[k]
    e = cols - pcol[params]
    assert np.all((e >= 0) & (e < np.asarray(w.numel)[params]))
    want = U.oracle_sampled_flush(w, cols, None)
    idx = torch.from_numpy((poff[params] + e).astype(np.int64)).cuda()
    got = U.to_host(d_out[:, idx], w.dtype)
    H = hold[:, params]
    wb, gb = U.bits(want, w.dtype), U.bits(got, w.dtype)
    assert np.array_equal(gb[H], wb[H]), "holder buffers differ from the oracle"
    sent = U.SENTINEL16 if w.dtype == wl.DT_BF16 else U.SENTINEL32
    assert np.all(gb[~H] == sent), "a rank without a buffer was written"
    U.say("  checked", int(H.sum()), "holder elements,", int((~H).sum()), "untouched")


@pytest.mark.parametrize("planned", [True, False], ids=["planned", "searched"])
def test_flush_buffers_owner_w8_full_size(planned):
    w = wl.owner_flush_w8()
    ex, d_out, ld, poff, pcol, hold = U.fused_flush_full_size(w, planned)
    _check_sampled(w, d_out, ld, poff, pcol, hold)


def test_flush_buffers_mixed_w16_full_size():
    import torch
    free, _ = torch.cuda.mem_get_info()
    w = wl.mixed_flush_w16()
    need = 2.2 * w.W * w.total * w.elem_bytes()
    if free < need:
        pytest.skip(f"needs {need / 1e9:.0f} GB of device memory, {free / 1e9:.0f} GB free")
    ex, d_out, ld, poff, pcol, hold = U.fused_flush_full_size(w)
    _check_sampled(w, d_out, ld, poff, pcol, hold)


@pytest.mark.parametrize("planned", [True, "device"], ids=["host-plans", "device-plans"])
def test_flush_buffers_split_params_via_executor(planned):
    """Params split over buckets through the executor: each task's slice
    continues where the param's previous task ended, in the input buffers and
    in the holders' grad buffers; the whole output arena matches the oracle
    (sentinel wherever no holder keeps a buffer).  The plans are built on the
    host or on the device (the same records, compared here)."""
    import torch
    W, dtype, pre = 4, wl.DT_BF16, 1
    numel = [100, 5000, 37, 777, 4096]
    buckets = [executor.BucketSpec(0, 3100, [(0, 100, 0, 0), (100, 3000, 1, 0)]),
               executor.BucketSpec(3100, 2814, [(0, 2000, 1, 0), (2000, 37, 2, 0), (2037, 777, 3, 0)]),
               executor.BucketSpec(5914, 1000, [(0, 1000, 4, 0)]),
               executor.BucketSpec(6914, 3096, [(0, 3096, 4, 0)])]
    ex = executor.Zero1FlushExecutor(W, dtype, numel, [0, 5], [W], [W], [list(range(W))], [(W, 1)],
                                     buckets, pre, reduce_to_owner=True)
    ex.build_owner_map()
    ex.fetch_metadata()
    eb = 2
    pad = 64
    poff, pos = [], 0
    for n in numel:
        poff.append(pos)
        pos = wl.round_up(pos + n, pad)
    ld = wl.round_up(pos, 64)
    scale = wl.sigma_scale(1e-2)
    x = U.gen_slab(dtype, W, ld, ld, 71, 0, scale)
    hx = U.host_slab(dtype, W, ld, ld, 71, 0, scale)
    y = U.empty_slab(dtype, W, ld)
    hold = np.zeros((W, len(numel)), bool)
    for b, bk in enumerate(buckets):
        h = ex.holders(b)
        for k, t in enumerate(bk.tasks):
            hold[:, t[2]] |= h[k]
    rows = np.arange(W, dtype=np.int64)[:, None] * ld
    po = np.array(poff, np.int64)[None, :]
    in_addr = (x.data_ptr() + (rows + po) * eb).astype(np.uint64)
    out_addr = np.where(hold, y.data_ptr() + (rows + po) * eb, 0).astype(np.uint64)
    ex.register_buffers(in_addr, out_addr, planned=planned)
    if planned == "device":
        dev_tiles, dev_begin = ex.d_btiles.cpu().numpy(), list(ex.buf_tile_begin)
        ex.register_buffers(in_addr, out_addr, planned=True)
        assert dev_begin == list(ex.buf_tile_begin)
        assert np.array_equal(dev_tiles, ex.d_btiles.cpu().numpy())
        ex.register_buffers(in_addr, out_addr, planned=planned)
    for b in range(len(buckets)):
        ex.flush_buffers(b)
    torch.cuda.synchronize()
    # the oracle on the same offsets
    seen = [0] * len(numel)
    in_off, out_off, t_numel = [], [], []
    for bk in buckets:
        for (_, n, p, _) in bk.tasks:
            in_off.append([r * ld + poff[p] + seen[p] for r in range(W)])
            out_off.append([r * ld + poff[p] + seen[p] if hold[r, p] else -1 for r in range(W)])
            t_numel.append(n)
            seen[p] += n
    hin = np.ascontiguousarray(hx).ravel()
    hout = np.full(W * ld, U.SENTINEL16, np.uint16)
    oracle.flush_buffers(W, dtype, hin, np.array(in_off), hout, np.array(out_off), t_numel,
                         [0] * len(t_numel), [W], [1], pre)
    assert np.array_equal(U.to_host(y, dtype).ravel(), hout)
