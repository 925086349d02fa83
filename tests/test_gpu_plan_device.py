"""GPU: the device-side planners (dc_plan_flush_device,
dc_plan_flush_buffers_device, dc_plan_relayout_tiles_device).  Their records
against the tile records the header defines (the brute-force definitions of
the CPU tests) and against the host planners', bit for bit, with the flush
planner's root count; flushes from its plans against the oracle; the
full-size layouts' plans equal to the host's; a replayed graph of it; and
tables that break their contract keep every write inside the plan."""
import random

import numpy as np
import pytest

import oracle
from gradient_reduction_amd import dc, executor
from synth import workloads as wl
from tests import gpu_util as U
from tests import test_gpu_flush as F
from tests.test_abi import (_brute_plan, _brute_plan_buffers, _brute_relayout_tiles,
                            buffer_plan_cases, relayout_tile_cases)

pytestmark = pytest.mark.gpu

GUARD = 64   # records of sentinel past every plan


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dc.lib()
    yield
    torch.cuda.synchronize()


def _dev(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda() if a is not None else None


def _plan_on_device(W, dtype, col0, numel, t, owner, flat, psize, P, comms):
    """(records, root count) from dc_plan_flush_device, with a guard of
    sentinel records past the plan checked untouched."""
    import torch
    n = dc.dc_plan_flush_device(W, dtype, col0, numel, None, len(t), None, None, None, P, comms,
                                len(comms), None, 0)
    d_t = torch.from_numpy(t.view(np.uint8).copy()).cuda() if len(t) else None
    buf = torch.full(((n + GUARD) * 4,), -7, dtype=torch.int32, device="cuda")
    roots = torch.full((1,), -9, dtype=torch.int64, device="cuda")
    got_n = dc.dc_plan_flush_device(W, dtype, col0, numel, d_t, len(t), _dev(owner, torch),
                                    _dev(flat, torch), _dev(psize, torch), P, comms, len(comms), buf,
                                    n, roots)
    assert got_n == n
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    assert np.all(h[4 * n:] == -7), "a record past the plan was written"
    return h[:4 * n].view(dc.TILE_DTYPE).copy(), int(roots.cpu()[0])


def _definition_cases(seed):
    rng = random.Random(seed)
    ws = [wl.tiny_flush()]
    for k in range(6):
        W = rng.choice([1, 2, 3, 4, 8, 16, 64])
        dtype = rng.choice([wl.DT_BF16, wl.DT_F32])
        sizes = [rng.choice([0, 1, 7, 8, 9, 500, 1023, 1024, 1025, 4000, 9000, 70_000])
                 for _ in range(150)]
        ws.append(wl.custom_flush(f"d{seed}-{k}", W, dtype, sizes, group_begin=[0, 90, 150],
                                  group_comm=[0, 1 if W > 1 else 0],
                                  comms=[wl.Comm(W, 1), wl.Comm(1, W) if W > 1 else wl.Comm(1, 1)],
                                  capacity=rng.choice([3000, 20_000, 10 ** 6])))
    return rng, ws


@pytest.mark.parametrize("seed", [31, 32])
def test_device_plan_matches_definition_and_host(seed):
    """Every bucket of seeded workloads (W up to 64, both dtypes, empty and
    one-element tasks, a sub-communicator group), at the bucket's own start
    column and at a start inside a vector, in all three modes."""
    rng, ws = _definition_cases(seed)
    for w in ws:
        flat, ps, off, pids = oracle.partition_ids(w.numel, w.group_begin, w.group_parts())
        elig = oracle.group_eligible(w.W, [w.comms[c].size for c in w.group_comm],
                                     w.group_rank_to_global())
        owner, _ = oracle.owner_map(off, pids, w.group_begin, elig)
        owner = np.asarray(owner, np.int32)
        flat = np.asarray(flat, np.int64)
        psize = np.zeros(w.P, np.int64)
        for g in range(w.G):
            if elig[g]:
                psize[w.group_begin[g]:w.group_begin[g + 1]] = ps[g]
        comms = [(c.size, c.stride) for c in w.comms]
        U.say("device plan", w.name, f"W={w.W}", f"buckets={len(w.buckets)}")
        for bk in w.buckets[:12]:
            t = dc.tasks_array([(x.offset, x.numel, x.param, x.comm) for x in bk.tasks])
            for col0 in (bk.col, bk.col + rng.randint(1, 15)):
                for own, fl, pz in ((None, None, None), (owner, None, None), (None, flat, psize)):
                    got, roots = _plan_on_device(w.W, w.dtype, col0, bk.numel, t, own, fl, pz, w.P,
                                                 comms)
                    want = _brute_plan(w.W, w.dtype, col0, bk.numel, t, own, fl, pz)
                    assert np.array_equal(got, want), (w.name, col0, own is None, fl is None)
                    host, host_roots = dc.dc_plan_flush(w.W, w.dtype, col0, bk.numel, t, len(t), own,
                                                        fl, pz, w.P, comms, len(comms))
                    assert np.array_equal(got, host) and roots == host_roots


def test_device_plan_empty_bucket_and_no_tasks():
    """No tiles: the count is cleared and nothing else is written.  Tiles but
    no tasks (a table the host planner would reject): every record is
    (0, -1, -1, 0), no tile is whole."""
    import torch
    comms = [(8, 1)]
    roots = torch.full((1,), 5, dtype=torch.int64, device="cuda")
    buf = torch.full((GUARD * 4,), -7, dtype=torch.int32, device="cuda")
    assert dc.dc_plan_flush_device(8, wl.DT_BF16, 64, 0, None, 0, None, None, None, 1, comms, 1, buf,
                                   0, roots) == 0
    torch.cuda.synchronize()
    assert int(roots.cpu()[0]) == 0 and bool((buf == -7).all())
    got, r = _plan_on_device(8, wl.DT_F32, 3, 1000, dc.tasks_array([]), None, None, None, 1, comms)
    assert len(got) == 4 and r == 0
    assert np.all(got["first"] == 0) and np.all(got["last"] == -1) and np.all(got["flags"] == 0)


@pytest.mark.parametrize("w", F.small_flush_workloads(), ids=lambda w: w.name)
@pytest.mark.parametrize("mode", ["allreduce", "owner", "zero2"])
def test_flush_from_device_plans(w, mode):
    """The executor plans on the device and flushes with those plans: every
    output element against the oracle."""
    F.flush_case(w, mode == "owner", zero2=mode == "zero2", planned="device")


def _executor_plans(w, owner, zero2, on_device):
    ex = executor.from_workload(w, reduce_to_owner=owner, zero2=zero2)
    ex.build_owner_map()
    ex.plan(on_device=on_device)
    return ex.d_tiles.cpu().numpy(), list(ex.tile_begin), list(ex.root_tiles)


@pytest.mark.parametrize("name,mode", [("owner_flush_w8", "owner"), ("owner_flush_w8", "zero2"),
                                       ("owner_flush_w8", "allreduce"),
                                       ("owner_flush_w8_layered", "owner"),
                                       ("mixed_flush_w16", "owner"), ("mixed_flush_w16", "zero2")])
def test_full_size_device_plans_equal_host_plans(name, mode):
    """Every plan record and root count of the full-size layouts, planned on
    the device and on the host."""
    w = getattr(wl, name)()
    U.say("device vs host plans", w.name, mode)
    dev = _executor_plans(w, mode == "owner", mode == "zero2", True)
    host = _executor_plans(w, mode == "owner", mode == "zero2", False)
    assert dev[1] == host[1] and dev[2] == host[2]
    assert np.array_equal(dev[0], host[0])


def test_device_plan_graph_replays():
    """The planner recorded in a HIP graph (its root count is cleared by a
    kernel, not a memset): every replay, with eager fills between, writes the
    eager plan and count."""
    import torch
    w = wl.custom_flush("g-plan", 8, wl.DT_BF16, [7, 0, 3000, 65, 12000, 1, 9, 40000, 513] * 5,
                        capacity=10 ** 6)
    bk = w.buckets[0]
    t = dc.tasks_array([(x.offset, x.numel, x.param, x.comm) for x in bk.tasks])
    owner = np.array([(p * 5) % 8 if p % 4 else -1 for p in range(w.P)], np.int32)
    comms = [(8, 1)]
    want, want_roots = dc.dc_plan_flush(8, w.dtype, bk.col + 5, bk.numel, t, len(t), owner, None, None,
                                        w.P, comms, 1)
    n = len(want)
    d_t = torch.from_numpy(t.view(np.uint8).copy()).cuda()
    d_own = torch.from_numpy(owner).cuda()
    buf = torch.full((n * 4,), -7, dtype=torch.int32, device="cuda")
    roots = torch.full((1,), -9, dtype=torch.int64, device="cuda")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dc.dc_plan_flush_device(8, w.dtype, bk.col + 5, bk.numel, d_t, len(t), d_own, None, None, w.P,
                                comms, 1, buf, n, roots, torch.cuda.current_stream())
    for rep in range(4):
        buf.fill_(-7)
        roots.fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = buf.cpu().numpy().view(dc.TILE_DTYPE)
        assert np.array_equal(got, want), f"replay {rep}"
        assert int(roots.cpu()[0]) == want_roots, f"replay {rep}"


def test_device_plan_contract_breaking_tables_stay_in_range():
    """Task tables that break the contract (offsets out of order or negative,
    params and communicators outside their tables, negative sizes) give
    other records, but the planner writes exactly the plan's records, each
    with first in [0, n) and last in [-1, n), and reads the owner,
    flat-offset and size tables only inside [0, num_params)."""
    import torch
    rng = random.Random(91)
    comms = [(8, 1), (4, 1)]
    for k in range(12):
        n = rng.randint(1, 40)
        P = rng.randint(1, 10)
        t = dc.tasks_array([(rng.randint(-5000, 60_000), rng.randint(-100, 9000),
                             rng.randint(-5, P + 5), rng.randint(-3, 5)) for _ in range(n)])
        numel = rng.randint(1, 70_000)
        col0 = rng.randint(0, 5000)
        dtype = rng.choice([wl.DT_BF16, wl.DT_F32])
        owner = np.array([rng.randint(-3, 12) for _ in range(P)], np.int32)
        flat = np.array([rng.randint(-10 ** 6, 10 ** 6) for _ in range(P)], np.int64)
        psize = np.array([rng.choice([0, -4, 1, 1000, 10 ** 5]) for _ in range(P)], np.int64)
        U.say("contract-breaking table", k, n, P, numel, col0, dtype)
        for own, fl, pz in ((owner, None, None), (None, flat, psize)):
            got, roots = _plan_on_device(8, dtype, col0, numel, t, own, fl, pz, P, comms)
            assert np.all((got["first"] >= 0) & (got["first"] < n))
            assert np.all((got["last"] >= -1) & (got["last"] < n))
            assert np.all((got["root"] >= -1) & (got["root"] < 8))
            assert roots == int(np.sum((got["flags"] & 1).astype(bool) & (got["root"] >= 0)))


def _device_records(n, fill, call, width=4):
    """Run `call(buf)` on a device buffer of n records of `width` int32 each
    plus a guard; check the guard, return the n records' int32 words."""
    import torch
    buf = torch.full(((n + GUARD) * width,), fill, dtype=torch.int32, device="cuda")
    call(buf)
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    assert np.all(h[n * width:] == fill), "a record past the plan was written"
    return h[:n * width]


def _device_buffer_plan(W, dtype, numel, t, comms):
    import torch
    n = dc.dc_plan_flush_buffers_device(W, dtype, numel, None, len(t), comms, len(comms), None, 0)
    d_t = torch.from_numpy(t.view(np.uint8).copy()).cuda() if len(t) else None
    words = _device_records(n, -7, lambda buf: dc.dc_plan_flush_buffers_device(
        W, dtype, numel, d_t, len(t), comms, len(comms), buf, n))
    return words.view(dc.TILE_DTYPE).copy()


def _device_relayout_tiles(dtype, col, numel, pieces, out_numel):
    import torch
    n = dc.dc_plan_relayout_tiles_device(dtype, col, numel, None, len(pieces), out_numel, None, 0)
    d_p = torch.from_numpy(pieces.view(np.uint8).copy()).cuda() if len(pieces) else None
    words = _device_records(n, -7, lambda buf: dc.dc_plan_relayout_tiles_device(
        dtype, col, numel, d_p, len(pieces), out_numel, buf, n), width=2)
    return words.view(np.int64).copy()


@pytest.mark.parametrize("seed", [12, 13])
def test_device_buffer_plan_matches_definition_and_host(seed):
    """Seeded buffer-coordinate task tables (gaps, empty tasks, offsets on
    and off slot boundaries, a sub-communicator)."""
    U.say("device fused plan", seed)
    for k, (W, dtype, numel, t, comms) in enumerate(buffer_plan_cases(seed)):
        got = _device_buffer_plan(W, dtype, numel, t, comms)
        assert np.array_equal(got, _brute_plan_buffers(dtype, numel, t)), k
        assert np.array_equal(got, dc.dc_plan_flush_buffers(W, dtype, numel, t, len(t), comms,
                                                             len(comms))), k


@pytest.mark.parametrize("name", ["owner_flush_w8", "mixed_flush_w16"])
def test_device_buffer_plans_of_full_size_layouts(name):
    """The fused flush's full-size layouts: each bucket's tasks re-laid at
    128-byte steps in buffer coordinates, as the executor registers them."""
    w = getattr(wl, name)()
    step = 128 // w.elem_bytes()
    comms = [(c.size, c.stride) for c in w.comms]
    U.say("device fused plans", w.name)
    for bk in w.buckets:
        rows, pos = [], 0
        for x in bk.tasks:
            rows.append((pos, x.numel, x.param, x.comm))
            pos = -(-(pos + x.numel) // step) * step
        t = dc.tasks_array(rows)
        numel = rows[-1][0] + rows[-1][1]
        got = _device_buffer_plan(w.W, w.dtype, numel, t, comms)
        assert np.array_equal(got, dc.dc_plan_flush_buffers(w.W, w.dtype, numel, t, len(t), comms,
                                                             len(comms)))


@pytest.mark.parametrize("seed", [12, 14])
def test_device_relayout_tiles_match_definition_and_host(seed):
    """The relayout planner's pieces of seeded workloads at several start
    residues, and random piece tables (unaligned sources, gaps, empty and
    overlapping pieces)."""
    U.say("device relayout plan", seed)
    whole = 0
    for dt, col, numel, pieces, out_numel in relayout_tile_cases(seed):
        got = _device_relayout_tiles(dt, col, numel, pieces, out_numel)
        assert np.array_equal(got, _brute_relayout_tiles(dt, col, numel, pieces, out_numel))
        assert np.array_equal(got, dc.dc_plan_relayout_tiles(dt, col, numel, pieces, len(pieces),
                                                             out_numel))
        whole += int(np.sum(got >= 0))
    assert whole > 100


def test_device_relayout_tiles_full_size():
    """Every bucket of the 402.8M-element W = 8 relayout (pieces from
    dc_plan_relayout over the eight equal partitions)."""
    w = wl.owner_flush_w8()
    flat, ps, _, _ = oracle.partition_ids(w.numel, w.group_begin, w.group_parts())
    psize = np.full(w.P, ps[0], np.int64)
    U.say("device relayout plans", w.name)
    for bk in w.buckets:
        t = dc.tasks_array([(x.offset, x.numel, x.param, x.comm) for x in bk.tasks])
        pieces, seg = dc.dc_plan_relayout(w.W, t, len(t), flat, psize, w.P)
        got = _device_relayout_tiles(w.dtype, bk.col, bk.numel, pieces, int(seg[-1]))
        want = dc.dc_plan_relayout_tiles(w.dtype, bk.col, bk.numel, pieces, len(pieces), int(seg[-1]))
        assert np.array_equal(got, want) and np.sum(got >= 0) > 0.99 * len(got)


def test_device_plan_variants_contract_breaking_tables_stay_in_range():
    """Task and piece tables that break their contracts (out of order,
    negative offsets, sizes and sources) give other records, but every
    record stays in its range and nothing past the plan is written: a fused
    record's task range inside the table, a relayout record inside the
    bucket's vectors or -1."""
    rng = random.Random(93)
    for k in range(12):
        n = rng.randint(1, 40)
        dtype = rng.choice([wl.DT_BF16, wl.DT_F32])
        E = 8 if dtype == wl.DT_BF16 else 4
        t = dc.tasks_array([(rng.randint(-5000, 60_000), rng.randint(-100, 9000), rng.randint(-5, 50),
                             rng.randint(-3, 5)) for _ in range(n)])
        numel = rng.randint(1, 70_000)
        U.say("contract-breaking fused/relayout tables", k, n, numel, dtype)
        got = _device_buffer_plan(8, dtype, numel, t, [(8, 1), (4, 1)])
        assert np.all((got["first"] >= 0) & (got["first"] < n))
        assert np.all((got["last"] >= -1) & (got["last"] < n))
        assert np.all(got["root"] == -1) and np.all((got["flags"] == 0) | (got["flags"] == 1))
        pieces = np.array([(rng.randint(-3000, numel), rng.randint(-2000, 40_000), rng.randint(-50, 8000), 0)
                           for _ in range(n)], dc.PIECE_DTYPE)
        col = rng.randint(0, 5000)
        out_numel = rng.randint(0, 50_000)
        rec = _device_relayout_tiles(dtype, col, numel, pieces, out_numel)
        lo, hi = -(-col // E), (col + numel) // E - 64
        assert np.all((rec == -1) | ((rec >= lo) & (rec <= hi)))


def test_device_planners_on_drawn_layouts():
    """The property tests' hypothesis-drawn layouts (tests/test_planner_properties.py),
    planned on the device: every record equal to the brute-force definition,
    and the flush planner's root count."""
    from hypothesis import given
    from tests.test_planner_properties import (SETTINGS, buffer_layouts, flush_layouts,
                                               relayout_layouts)

    @SETTINGS
    @given(flush_layouts())
    def flush(layout):
        W, dtype, col0, numel, tasks, owner, flat, psize, comms = layout
        got, roots = _plan_on_device(W, dtype, col0, numel, tasks, owner, flat, psize, len(tasks),
                                     comms)
        want = _brute_plan(W, dtype, col0, numel, tasks, owner, flat, psize)
        assert np.array_equal(got, want) and roots == int(np.sum(want["root"] >= 0))

    @SETTINGS
    @given(buffer_layouts())
    def buffers(layout):
        W, dtype, numel, tasks, comms = layout
        assert np.array_equal(_device_buffer_plan(W, dtype, numel, tasks, comms),
                              _brute_plan_buffers(dtype, numel, tasks))

    @SETTINGS
    @given(relayout_layouts())
    def relayout(layout):
        dtype, col, numel, pieces, out_numel = layout
        assert np.array_equal(_device_relayout_tiles(dtype, col, numel, pieces, out_numel),
                              _brute_relayout_tiles(dtype, col, numel, pieces, out_numel))

    U.say("device planners on drawn layouts")
    flush()
    buffers()
    relayout()
