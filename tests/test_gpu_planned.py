"""GPU parity of the planned bucket flush (dc_plan_flush + dc_flush_bucket_planned)
through the C ABI: against the oracle bit for bit on the small edge-case
workloads (owner map, AllReduce, ZeRO-2, in place), on seeded random buckets
with every start residue, and at full size, where the whole output of the
planned flush is also compared with the searched flush's."""
import random

import numpy as np
import pytest

import oracle
from gradient_reduction_amd import dc, executor
from synth import workloads as wl
from tests import gpu_util as U
from tests import test_gpu_flush as F

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dc.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("w", F.small_flush_workloads(), ids=lambda w: w.name)
@pytest.mark.parametrize("owner", [False, True], ids=["allreduce", "owner"])
def test_planned_flush_small(w, owner):
    F.flush_case(w, owner, planned=True)


@pytest.mark.parametrize("w", F.small_flush_workloads() + [wl.tiny_flush()], ids=lambda w: w.name)
def test_planned_flush_zero2_small(w):
    F.flush_case(w, False, zero2=True, planned=True)


@pytest.mark.parametrize("w", F.small_flush_workloads()[2::5], ids=lambda w: w.name)
@pytest.mark.parametrize("mode", ["owner", "zero2"])
def test_planned_flush_in_place(w, mode):
    F.flush_case(w, mode == "owner", in_place=True, probe=False, zero2=mode == "zero2", planned=True)


def test_planned_flush_empty_bucket():
    """An empty bucket has no tiles: NULL plan, zero tiles, nothing written."""
    import torch
    W, dtype, ld = 8, wl.DT_BF16, 256
    x = U.gen_slab(dtype, W, ld, ld, 3, 0, wl.sigma_scale(1e-2))
    y = U.empty_slab(dtype, W, ld)
    before = y.cpu()
    tiles, roots = dc.dc_plan_flush(W, dtype, 64, 0, dc.tasks_array([]), 0, None, None, None, 1,
                                    [(W, 1)], 1)
    assert len(tiles) == 0 and roots == 0
    dc.dc_flush_bucket_planned(W, dtype, x, ld, y, ld, 64, 0, None, 0, None, None, None, 1,
                               [(W, 1)], 1, 1, None, 0, 0)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), before)


@pytest.mark.parametrize("seed", range(16))
def test_planned_flush_random_abi_cases(seed):
    """Seeded random buckets straight through the ABI: random W (up to the
    ABI's 64, where the run-time-W kernel takes over), dtype, communicators,
    owners or ZeRO-2 partitions, pre-division, start column of any residue,
    task sizes from 0 to several tiles, in and out of place."""
    import torch
    rng = random.Random(2000 + seed)
    W = rng.choice([1, 2, 3, 4, 6, 8, 12, 16]) if seed < 12 else [24, 32, 48, 64][seed - 12]
    dtype = rng.choice([wl.DT_BF16, wl.DT_F32])
    divs = [c for c in range(1, W) if W % c == 0]
    comms = [(W, 1)]
    if divs and rng.random() < 0.7:
        c = rng.choice(divs)
        comms.append((c, rng.choice([1, W // c])))
    n_tasks = rng.randint(1, 40)
    sizes = [rng.choice([0, 1, 7, 8, 9, 1023, 1024, 1025, 2048, 3000, 9000, 20_000])
             for _ in range(n_tasks)]
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(int).tolist()
    bucket_numel = int(sum(sizes))
    P = n_tasks
    t_comm = [rng.randrange(len(comms)) for _ in range(n_tasks)]
    tasks = [(offs[k], sizes[k], k, t_comm[k]) for k in range(n_tasks)]
    zero2 = rng.random() < 0.4
    if zero2:
        # each param sits at a random place in a flat buffer of random partition size
        psize = np.array([rng.choice([0, 1, 64, 1000, 5000, 40_000]) for _ in range(P)], np.int64)
        flat = np.array([rng.randint(0, max(int(s) * W - n, 0)) if s else 0
                         for s, n in zip(psize, sizes)], np.int64)
        psize = np.where(flat + np.array(sizes) <= psize * W, psize, 0)
        owner = None
    else:
        owner = np.array([rng.choice([-1, rng.randrange(W)]) for _ in range(P)], np.int32)
        if rng.random() < 0.3:
            owner = None
        flat = psize = None
    col0 = rng.randint(0, 2100)
    pre = rng.randint(0, 1)
    in_place = rng.random() < 0.3
    ld = max(64, wl.round_up(col0 + bucket_numel + rng.randint(0, 100), 64))
    scale = wl.sigma_scale(1e-2)
    U.say("planned random flush", seed, W, dtype, comms, n_tasks, bucket_numel, col0, pre, in_place,
          "zero2" if zero2 else ("owner" if owner is not None else "allreduce"))
    t = dc.tasks_array(tasks)
    tiles, roots = dc.dc_plan_flush(W, dtype, col0, bucket_numel, t, len(t), owner, flat, psize, P,
                                    comms, len(comms))
    x = U.gen_slab(dtype, W, ld, ld, 500 + seed, 0, scale)
    y = x if in_place else U.empty_slab(dtype, W, ld)
    d_tasks = torch.from_numpy(t.view(np.uint8).copy()).cuda()
    d_tiles = torch.from_numpy(tiles.view(np.uint8).copy()).cuda() if len(tiles) else None
    d_owner = torch.from_numpy(owner).cuda() if owner is not None else None
    d_flat = torch.from_numpy(flat).cuda() if zero2 else None
    d_psize = torch.from_numpy(psize).cuda() if zero2 else None
    dc.dc_flush_bucket_planned(W, dtype, x, ld, y, ld, col0, bucket_numel, d_tasks, len(tasks), d_owner,
                               d_flat, d_psize, P, comms, len(comms), pre, d_tiles, len(tiles),
                               rng.choice([roots, 0, len(tiles)]))   # the launch shape only
    torch.cuda.synchronize()
    hin = U.host_slab(dtype, W, ld, ld, 500 + seed, 0, scale)
    if in_place:
        hout = hin
    else:
        hout = np.zeros_like(hin)
        U.bits(hout, dtype)[:] = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
    if zero2:
        oracle.flush_zero2(W, dtype, hin, hout, col0, offs, sizes, list(range(n_tasks)), t_comm, flat,
                           psize, [c for c, _ in comms], [s for _, s in comms], pre)
    else:
        oracle.flush(W, dtype, hin, hout, col0, offs, sizes, list(range(n_tasks)), t_comm, owner,
                     [c for c, _ in comms], [s for _, s in comms], pre)
    assert np.array_equal(U.bits(U.to_host(y, dtype), dtype), U.bits(hout, dtype))


def _planned_equals_searched(w, owner, zero2=False, in_place=False):
    """The whole output of the planned flush against the searched flush's,
    on the same input (every column, both on the GPU)."""
    import torch
    U.say("planned == searched", w.name, "zero2" if zero2 else ("owner" if owner else "allreduce"),
          "in-place" if in_place else "", f"W={w.W} cols={w.total}")
    ld = w.ld
    outs = []
    for planned in (False, True):
        x = U.gen_slab(w.dtype, w.W, ld, w.total, w.value_seed, 0, w.scale)
        y = x if in_place else U.empty_slab(w.dtype, w.W, ld)
        ex = executor.from_workload(w, reduce_to_owner=owner, zero2=zero2)
        ex.build_owner_map()
        if planned:
            ex.plan()
        for b in range(len(w.buckets)):
            ex.flush(b, x, ld, y, ld)
        torch.cuda.synchronize()
        outs.append(y)
        del x
    same = bool(torch.equal(outs[0], outs[1]))
    del outs
    torch.cuda.empty_cache()
    assert same


@pytest.mark.parametrize("mode", ["owner", "allreduce", "zero2"])
def test_planned_equals_searched_w8_402m(mode):
    _planned_equals_searched(wl.owner_flush_w8(), mode == "owner", zero2=mode == "zero2")


def test_planned_equals_searched_w8_402m_layered():
    _planned_equals_searched(wl.owner_flush_w8_layered(), True)


@pytest.mark.parametrize("mode", ["owner", "zero2"])
def test_planned_equals_searched_w16_mixed_in_place(mode):
    _planned_equals_searched(wl.mixed_flush_w16(), mode == "owner", zero2=mode == "zero2", in_place=True)


@pytest.mark.parametrize("mode", ["owner", "zero2"])
def test_planned_flush_w8_402m_full_size(mode):
    """Sampled columns of the full-size planned flush against the oracle."""
    F.full_size_flush(wl.owner_flush_w8(), mode == "owner", in_place=False, zero2=mode == "zero2",
                      planned=True)


def test_planned_flush_stale_plan_stays_in_slabs():
    """The plan is device data that the kernel reads without a host check: a
    plan of random records (task ranges, roots, flags and communicators out
    of range included) can give wrong sums, but every write stays in the
    columns of the bucket's tile grid and the input slab is left as it was.
    Buckets sit behind a guard of columns on both sides to show it."""
    import torch
    rng = random.Random(77)
    for w in F.small_flush_workloads()[::3] + [wl.tiny_flush()]:
        E = 8 if w.dtype == wl.DT_BF16 else 4
        G = 64 * E * 4
        ld = wl.round_up(w.total + 2 * G, 64 * E)
        x = U.gen_slab(w.dtype, w.W, ld, ld, w.value_seed, 0, w.scale)
        hx = U.bits(U.to_host(x, w.dtype), w.dtype).copy()
        y = U.empty_slab(w.dtype, w.W, ld)
        ex = executor.from_workload(w, reduce_to_owner=True)
        ex.build_owner_map()
        ex.fetch_metadata()
        span = np.zeros(ld, bool)
        U.say("stale plan", w.name)
        for b, bk in enumerate(w.buckets):
            t = ex.h_tasks[b]
            c0 = G + bk.col
            tiles, _ = dc.dc_plan_flush(w.W, w.dtype, c0, bk.numel, t, len(t), ex.h_owner, None, None,
                                        w.P, ex.comms, len(ex.comms))
            n = len(tiles)
            if n == 0:
                continue
            tiles["first"] = [rng.randint(-3, len(t) + 3) for _ in range(n)]
            tiles["last"] = [rng.randint(-3, len(t) + 3) for _ in range(n)]
            tiles["root"] = [rng.randint(-3, w.W + 3) for _ in range(n)]
            tiles["flags"] = [rng.randint(0, 1) | (rng.randint(0, len(ex.comms) + 2) << 8)
                              for _ in range(n)]
            d_tiles = torch.from_numpy(tiles.view(np.uint8).copy()).cuda()
            dc.dc_flush_bucket_planned(w.W, w.dtype, x, ld, y, ld, c0, bk.numel, ex.task_table(b),
                                       len(t), ex.d_owner, None, None, w.P, ex.comms, len(ex.comms),
                                       w.pre_div, d_tiles, n, rng.randint(0, n))
            v0 = (c0 // E) // 64 * 64
            span[v0 * E:-(-(c0 + bk.numel) // E) * E] = True
        torch.cuda.synchronize()
        got = U.bits(U.to_host(y, w.dtype), w.dtype)
        sent = U.SENTINEL16 if w.dtype == wl.DT_BF16 else U.SENTINEL32
        assert np.all(got[:, ~span] == sent), f"{w.name}: a write left the buckets' tile grid"
        assert np.array_equal(U.bits(U.to_host(x, w.dtype), w.dtype), hx), f"{w.name}: input changed"


def test_flush_on_drawn_layouts():
    """The property tests' hypothesis-drawn bucket layouts
    (tests/test_planner_properties.py: W up to 64, sub-communicators, owners
    in and out of range, ZeRO-2 partitions, any start column) flushed on the
    GPU, searched and from a host plan, every element against the oracle
    (which takes the library's reading of owners outside [0, W))."""
    import torch
    from hypothesis import given, settings
    from tests.test_planner_properties import flush_layouts

    @settings(max_examples=100, deadline=None, derandomize=True)
    @given(flush_layouts())
    def run(layout):
        W, dtype, col0, numel, t, owner, flat, psize, comms = layout
        P = len(t)
        if flat is not None:
            # the ZeRO-2 contract: a param's flat range lies inside its W partitions
            psize = np.where(flat + t["numel"] <= psize * W, psize, 0).astype(np.int64)
        # the oracle takes the library's reading of owners outside [0, W): AllReduce
        own_fixed = None if owner is None else np.where((owner >= 0) & (owner < W), owner, -1)
        ld = max(64, wl.round_up(col0 + numel + 5, 64))
        scale = wl.sigma_scale(1e-2)
        x = U.gen_slab(dtype, W, ld, ld, 77, 0, scale)
        hin = U.host_slab(dtype, W, ld, ld, 77, 0, scale)
        hout = np.zeros_like(hin)
        U.bits(hout, dtype)[:] = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
        offs, sizes = t["offset"].tolist(), t["numel"].tolist()
        t_comm = t["comm"].tolist()
        csz, cst = [c for c, _ in comms], [s for _, s in comms]
        if flat is not None:
            oracle.flush_zero2(W, dtype, hin, hout, col0, offs, sizes, list(range(P)), t_comm, flat,
                               psize, csz, cst, 1)
        else:
            oracle.flush(W, dtype, hin, hout, col0, offs, sizes, list(range(P)), t_comm, own_fixed,
                         csz, cst, 1)
        d_tasks = torch.from_numpy(t.view(np.uint8).copy()).cuda()
        d_owner = torch.from_numpy(owner).cuda() if owner is not None else None
        d_flat = torch.from_numpy(flat).cuda() if flat is not None else None
        d_psize = torch.from_numpy(psize).cuda() if flat is not None else None
        tiles, roots = dc.dc_plan_flush(W, dtype, col0, numel, t, P, owner, flat, psize, P, comms,
                                        len(comms))
        d_tiles = torch.from_numpy(tiles.view(np.uint8).copy()).cuda() if len(tiles) else None
        for planned in (False, True):
            y = U.empty_slab(dtype, W, ld)
            if planned:
                dc.dc_flush_bucket_planned(W, dtype, x, ld, y, ld, col0, numel, d_tasks, P, d_owner,
                                           d_flat, d_psize, P, comms, len(comms), 1, d_tiles,
                                           len(tiles), roots)
            elif flat is not None:
                dc.dc_flush_bucket_zero2(W, dtype, x, ld, y, ld, col0, numel, d_tasks, P, d_flat,
                                         d_psize, P, comms, len(comms), 1)
            else:
                dc.dc_flush_bucket(W, dtype, x, ld, y, ld, col0, numel, d_tasks, P, d_owner, P,
                                   comms, len(comms), 1)
            torch.cuda.synchronize()
            assert np.array_equal(U.bits(U.to_host(y, dtype), dtype), U.bits(hout, dtype)), planned

    U.say("flush on drawn layouts")
    run()
