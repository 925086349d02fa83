"""GPU parity: generator, bf16 rounding, partition lists / owner map and the
bucket flush, all through the C ABI, against the CPU oracle.

Bit-exact everywhere (integer metadata and fixed-order sums).
"""
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


def test_generator_device_matches_host():
    for dtype, n in ((wl.DT_BF16, 100_003), (wl.DT_F32, 77_777)):
        scale = wl.sigma_scale(1e-3)
        U.say("generator", dtype, n)
        d = U.to_host(U.gen_slab(dtype, 3, wl.round_up(n, 64), n, 9, 5, scale), dtype)
        h = U.host_slab(dtype, 3, wl.round_up(n, 64), n, 9, 5, scale)
        assert np.array_equal(U.bits(d, dtype), U.bits(h, dtype))
    # a column origin: position j of row r holds column col0 + j
    import torch
    for dtype in (wl.DT_BF16, wl.DT_F32):
        col0, n, ld = 123_457, 5_003, 5_056
        x = U.empty_slab(dtype, 2, ld)
        synth.fill_slab_device(dtype, 9, 7, wl.sigma_scale(1e-2), 2, ld, n, x.data_ptr(),
                               torch.cuda.current_stream().cuda_stream, col0=col0)
        got = U.bits(U.to_host(x, dtype), dtype)
        for r in range(2):
            want = synth.fill_row(dtype, 9, 7 + r, wl.sigma_scale(1e-2), col0, n)
            assert np.array_equal(got[r, :n], want.view(got.dtype)), (dtype, r)


def test_round_bf16_matches_oracle():
    import torch
    rng = np.random.default_rng(3)
    highs = np.arange(65536, dtype=np.uint64)
    lows = np.concatenate([[0, 1, 2, 0x7FFF, 0x8000, 0x8001, 0xFFFE, 0xFFFF],
                           rng.integers(0, 65536, 24)]).astype(np.uint64)
    u = ((highs[:, None] << 16) | lows[None, :]).ravel().astype(np.uint32)
    U.say("round_bf16", len(u))
    x = torch.from_numpy(u.view(np.int32).copy()).cuda()
    y = torch.empty(len(u), dtype=torch.int16, device="cuda")
    dc.dc_round_bf16(x, y, len(u))
    got = y.cpu().numpy().view(np.uint16)
    want = oracle.bf16_round(u.view(np.float32))
    bad = np.nonzero(got != want)[0]
    assert len(bad) == 0, f"{len(bad)} mismatches, e.g. {u[bad[:4]]}: {got[bad[:4]]} vs {want[bad[:4]]}"


def run_owner_map(w):
    import torch
    ex = executor.from_workload(w, reduce_to_owner=True)
    ex.build_owner_map()
    ex.fetch_metadata()
    torch.cuda.synchronize()
    return ex, torch.cuda.current_stream()


def owner_workloads():
    out = [wl.tiny_flush(), wl.owner_flush_w8(), wl.owner_flush_w8_layered(), wl.mixed_flush_w16()]
    rng = random.Random(5)
    for k in range(6):
        G = rng.randint(1, 4)
        numel, gb, gcomm = [], [0], []
        W = rng.choice([2, 4, 8, 16])
        comms = [wl.Comm(W, 1), wl.Comm(max(1, W // 2), 1), wl.Comm(max(1, W // 2), 2)]
        for g in range(G):
            numel += [rng.choice([0, 1, 3, 7, 64, 1000, 5000]) for _ in range(rng.randint(1, 3000))]
            gb.append(len(numel))
            gcomm.append(rng.choice([0, 0, 1, 2]))
        out.append(wl.custom_flush(f"rand{k}", W, wl.DT_BF16, numel, group_begin=gb,
                                   group_comm=gcomm, comms=comms, capacity=10 ** 9))
    # the limits: W = 64, 64 groups, 8 communicators (contiguous and strided)
    numel, gb, gcomm = [], [0], []
    comms64 = [wl.Comm(64, 1), wl.Comm(32, 1), wl.Comm(16, 4), wl.Comm(8, 8), wl.Comm(4, 1),
               wl.Comm(2, 32), wl.Comm(1, 1), wl.Comm(32, 2)]
    for g in range(64):
        numel += [rng.choice([0, 1, 5, 63, 64, 65, 700, 4099]) for _ in range(rng.randint(1, 40))]
        gb.append(len(numel))
        gcomm.append(rng.choice(range(8)) if g % 3 else 0)
    out.append(wl.custom_flush("W64-G64-C8", 64, wl.DT_BF16, numel, group_begin=gb,
                               group_comm=gcomm, comms=comms64, capacity=25_000, pre_div=1,
                               value_seed=64))
    # parameter sizes up to 2^40, group totals far past 2^32: 64-bit offsets,
    # partition sizes and partition indices (no slab is allocated)
    numel, gb = [], [0]
    for g in range(3):
        numel += [rng.choice([0, 1, 1 << 20, (1 << 40) - 1, 1 << 40, rng.randrange(1 << 40)])
                  for _ in range(rng.randint(50, 400))]
        gb.append(len(numel))
    out.append(wl.custom_flush("W8-sizes-to-2^40", 8, wl.DT_BF16, numel, group_begin=gb,
                               group_comm=[0, 1, 0], comms=[wl.Comm(8, 1), wl.Comm(4, 2)],
                               capacity=1 << 46))
    return out


@pytest.mark.parametrize("w", owner_workloads(), ids=lambda w: f"{w.name}-P{w.P}")
def test_partition_ids_and_owner_map(w):
    U.say("owner map", w.name, w.P)
    ex, _ = run_owner_map(w)
    flat, ps, off, pids, owner, counts = U.oracle_owner(w)
    assert np.array_equal(ex.d_flat[:w.P].cpu().numpy(), flat)
    assert np.array_equal(ex.d_part_size.cpu().numpy(), ps)
    assert np.array_equal(ex.h_pid_off, off)
    assert np.array_equal(ex.h_pids, pids)
    assert np.array_equal(ex.h_owner, owner)
    assert np.array_equal(ex.h_counts, counts)


def flush_case(w, reduce_to_owner, in_place=False, probe=True, zero2=False, planned=False):
    """Run every bucket of w on the GPU and on the oracle; compare all of the
    output slab bit for bit, and the probe records.  planned: the executor
    plans every bucket first (on the host, or with planned="device" on the
    device) and flushes with the plans."""
    import torch
    U.say("flush", w.name, "zero2" if zero2 else ("owner" if reduce_to_owner else "allreduce"),
          "in-place" if in_place else "", {False: "", True: "planned", "device": "planned on device"}[planned])
    scale = w.scale
    ld = w.ld
    x = U.gen_slab(w.dtype, w.W, ld, w.total, w.value_seed, 0, scale)
    y = x if in_place else U.empty_slab(w.dtype, w.W, ld)
    ex = executor.from_workload(w, reduce_to_owner=reduce_to_owner, zero2=zero2)
    ex.build_owner_map()
    if planned:
        ex.plan(on_device=planned == "device")
    for b in range(len(w.buckets)):
        ex.flush(b, x, ld, y, ld)
    torch.cuda.synchronize()
    got = U.to_host(y, w.dtype)
    hin = U.host_slab(w.dtype, w.W, ld, w.total, w.value_seed, 0, scale)
    hout = hin if in_place else np.zeros_like(hin)
    if not in_place:
        U.bits(hout, w.dtype)[:] = U.SENTINEL16 if w.dtype == wl.DT_BF16 else U.SENTINEL32
    _, _, off, pids, owner, _ = U.oracle_owner(w)
    if zero2:
        flat, psize = U.psize_per_param(w)
        assert np.array_equal(ex.h_psize, psize)
        for b in range(len(w.buckets)):
            U.oracle_flush_bucket_zero2(w, b, hin, hout, flat, psize)
        probe = False
    else:
        for b in range(len(w.buckets)):
            U.oracle_flush_bucket(w, b, hin, hout, owner if reduce_to_owner else None)
    gb, hb = U.bits(got, w.dtype), U.bits(hout, w.dtype)
    bad = np.argwhere(gb != hb)
    assert len(bad) == 0, (f"{len(bad)} mismatches; first (row, col): {bad[:5].tolist()} "
                           f"gpu {gb[tuple(bad[0])]:#x} oracle {hb[tuple(bad[0])]:#x}")
    if probe:
        ex.fetch_metadata()
        for b, bk in enumerate(w.buckets):
            pr = ex.probe(b)
            want = oracle.probe(w.W, [t.numel for t in bk.tasks], [t.param for t in bk.tasks],
                                [t.comm for t in bk.tasks], owner if reduce_to_owner else None,
                                off, pids, [c.size for c in w.comms], [c.stride for c in w.comms])
            assert (pr.tasks, pr.owner_tasks, pr.reduced_elems, pr.owner_elems) == (
                want["tasks"], want["owner_tasks"], want["reduced_elems"], want["owner_elems"])
            assert list(pr.written)[:w.W] == list(want["written"])
            assert list(pr.kept)[:w.W] == list(want["kept"])
            assert list(pr.discarded)[:w.W] == list(want["discarded"])


@pytest.mark.parametrize("owner", [False, True], ids=["allreduce", "owner"])
def test_flush_tiny_workload(owner):
    flush_case(wl.tiny_flush(), owner)


def small_flush_workloads():
    """Edge cases at sizes the oracle finishes in seconds: every W the fast
    kernels specialise and several they do not, both dtypes, pre-division on
    and off, sub-communicators with both strides, tiny and empty tasks (task
    edges inside 16-byte vectors), more tasks per tile than the LDS stage,
    more tasks than one search round, and a bucket that starts mid-vector."""
    rng = random.Random(17)
    out = []
    for W in (1, 2, 3, 4, 5, 7, 8, 16):
        for dtype in (wl.DT_BF16, wl.DT_F32):
            sizes = [rng.choice([0, 1, 2, 3, 5, 7, 9, 15, 16, 17, 100, 1000, 4096, 20_000])
                     for _ in range(60)]
            divs = [c for c in range(1, W + 1) if W % c == 0 and c < W]
            comms = [wl.Comm(W, 1)]
            gcomm = [0, 0]
            if divs:
                c = rng.choice(divs)
                comms.append(wl.Comm(c, 1))
                comms.append(wl.Comm(c, W // c))
                gcomm = [0, rng.choice([1, 2])]
            gb = [0, 40, 60]
            out.append(wl.custom_flush(f"W{W}-{wl.DTYPE_NAME[dtype]}", W, dtype, sizes,
                                       group_begin=gb, group_comm=gcomm, comms=comms,
                                       capacity=30_000, pre_div=(W + dtype) % 2,
                                       value_seed=W * 10 + dtype))
    # many tiny tasks: > 256 tasks in one tile, and > 256 tasks in the table
    tiny = [rng.randint(0, 5) for _ in range(70_000)]
    out.append(wl.custom_flush("W8-bf16-70k-tiny", 8, wl.DT_BF16, tiny, capacity=10 ** 9,
                               pre_div=1, value_seed=91))
    out.append(wl.custom_flush("W16-f32-5k-tiny", 16, wl.DT_F32, tiny[:5000],
                               capacity=10 ** 9, pre_div=0, value_seed=92))
    # the limits: W = 64 (the ABI's maximum) with all 8 communicators, both dtypes
    comms64 = [wl.Comm(64, 1), wl.Comm(32, 1), wl.Comm(16, 4), wl.Comm(8, 8), wl.Comm(4, 1),
               wl.Comm(2, 32), wl.Comm(1, 1), wl.Comm(32, 2)]
    for dtype in (wl.DT_BF16, wl.DT_F32):
        sizes = [rng.choice([0, 1, 7, 9, 64, 333, 2000, 9000]) for _ in range(40)]
        out.append(wl.custom_flush(f"W64-C8-{wl.DTYPE_NAME[dtype]}", 64, dtype, sizes,
                                   group_begin=[0, 10, 20, 30, 40], group_comm=[0, 1, 3, 5],
                                   comms=comms64, capacity=25_000, pre_div=1 - dtype,
                                   value_seed=640 + dtype))
    return out


@pytest.mark.parametrize("w", small_flush_workloads(), ids=lambda w: w.name)
@pytest.mark.parametrize("owner", [False, True], ids=["allreduce", "owner"])
def test_flush_small(w, owner):
    flush_case(w, owner)


@pytest.mark.parametrize("w", small_flush_workloads()[::5], ids=lambda w: w.name)
def test_flush_in_place(w):
    flush_case(w, True, in_place=True, probe=False)


@pytest.mark.parametrize("w", small_flush_workloads() + [wl.tiny_flush()], ids=lambda w: w.name)
def test_flush_zero2_small(w):
    """ZeRO-2 owner path: every element of a data-parallel task goes to the
    rank of its partition, bit-exact against the oracle."""
    flush_case(w, False, zero2=True)


@pytest.mark.parametrize("w", small_flush_workloads()[1::6], ids=lambda w: w.name)
def test_flush_zero2_in_place(w):
    flush_case(w, False, in_place=True, probe=False, zero2=True)


def test_flush_unaligned_bucket_start():
    """A bucket whose first column is not on a 16-byte vector: columns before
    it stay untouched."""
    import torch
    W, dtype = 8, wl.DT_BF16
    sizes = [5, 3000, 1, 2, 999]
    w = wl.custom_flush("unaligned", W, dtype, sizes, capacity=10 ** 9, pre_div=1)
    col0 = 3
    ld = wl.round_up(col0 + w.total, 64)
    scale = w.scale
    x = U.gen_slab(dtype, W, ld, ld, w.value_seed, 0, scale)
    y = U.empty_slab(dtype, W, ld)
    bk = w.buckets[0]
    tasks = dc.tasks_array([(t.offset, t.numel, t.param, t.comm) for t in bk.tasks])
    d_tasks = torch.from_numpy(tasks.view(np.uint8).copy()).cuda()
    _, _, off, pids, owner, _ = U.oracle_owner(w)
    d_owner = torch.from_numpy(owner).cuda()
    dc.dc_flush_bucket(W, dtype, x, ld, y, ld, col0, bk.numel, d_tasks, len(tasks), d_owner,
                       w.P, [(W, 1)], 1, 1)
    torch.cuda.synchronize()
    hin = U.host_slab(dtype, W, ld, ld, w.value_seed, 0, scale)
    hout = np.full_like(hin, U.SENTINEL16)
    oracle.flush(W, dtype, hin, hout, col0, [t.offset for t in bk.tasks], [t.numel for t in bk.tasks],
                 [t.param for t in bk.tasks], [t.comm for t in bk.tasks], owner, [W], [1], 1)
    assert np.array_equal(U.to_host(y, dtype), hout)


def test_flush_empty_bucket_and_no_tasks():
    import torch
    W, dtype, ld = 4, wl.DT_F32, 64
    x = U.gen_slab(dtype, W, ld, ld, 1, 0, wl.sigma_scale(1e-3))
    y = U.empty_slab(dtype, W, ld)
    d_tasks = torch.zeros(32, dtype=torch.uint8, device="cuda")
    dc.dc_flush_bucket(W, dtype, x, ld, y, ld, 8, 0, d_tasks, 0, None, 0, [(W, 1)], 1, 0)
    dc.dc_flush_bucket(W, dtype, x, ld, y, ld, 8, 16, d_tasks, 0, None, 0, [(W, 1)], 1, 0)
    torch.cuda.synchronize()
    assert np.all(U.to_host(y, dtype).view(np.uint32) == U.SENTINEL32)


def _nan_mask(b, dtype):
    if dtype == wl.DT_BF16:
        return ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    return ((b & 0x7F800000) == 0x7F800000) & ((b & 0x7FFFFF) != 0)


def test_flush_nonfinite_and_subnormal_inputs():
    """NaN, infinities, subnormals and signed zeros.  A NaN result must be a
    NaN on both sides (its sign and payload are not part of the result: x86
    and gfx950 pick different default NaNs); every other element is
    bit-exact."""
    import torch
    rng = random.Random(8)
    for W, dtype, pre in ((4, wl.DT_BF16, 1), (8, wl.DT_BF16, 0), (3, wl.DT_BF16, 1),
                          (4, wl.DT_F32, 1), (5, wl.DT_F32, 1)):
        n = 4000
        ld = wl.round_up(n, 64)
        if dtype == wl.DT_BF16:
            pool = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F80, 0xFF80, 0x7FC0,
                    0x7F7F, 0xFF7F, 0x3F80, 0x4B80, 0xCB80]
            h = np.array([[rng.choice(pool) if rng.random() < 0.5 else rng.getrandbits(16)
                           for _ in range(ld)] for _ in range(W)], np.uint16)
            d = torch.from_numpy(h.view(np.int16).copy()).cuda()
        else:
            pool = [0, 0x80000000, 1, 0x80000001, 0x007FFFFF, 0x00800000, 0x7F800000, 0xFF800000,
                    0x7FC00000, 0x7F7FFFFF, 0x3F800000]
            h = np.array([[rng.choice(pool) if rng.random() < 0.5 else rng.getrandbits(32)
                           for _ in range(ld)] for _ in range(W)], np.uint32)
            d = torch.from_numpy(h.view(np.int32).copy()).cuda()
            h = h.view(np.float32)
        sizes = [1, 2, 3, 1000, 5, 2989]
        w = wl.custom_flush("nonfinite", W, dtype, sizes, capacity=10 ** 9, pre_div=pre)
        bk = w.buckets[0]
        tasks = dc.tasks_array([(t.offset, t.numel, t.param, t.comm) for t in bk.tasks])
        d_tasks = torch.from_numpy(tasks.view(np.uint8).copy()).cuda()
        y = U.empty_slab(dtype, W, ld)
        dc.dc_flush_bucket(W, dtype, d, ld, y, ld, 0, bk.numel, d_tasks, len(tasks), None, w.P,
                           [(W, 1)], 1, pre)
        torch.cuda.synchronize()
        hout = np.zeros_like(h)
        U.bits(hout, dtype)[:] = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
        oracle.flush(W, dtype, h, hout, 0, [t.offset for t in bk.tasks], [t.numel for t in bk.tasks],
                     [t.param for t in bk.tasks], [t.comm for t in bk.tasks], None, [W], [1], pre)
        got = U.bits(U.to_host(y, dtype), dtype)
        want = U.bits(hout, dtype)
        gn, wn = _nan_mask(got, dtype), _nan_mask(want, dtype)
        assert np.array_equal(gn, wn), (W, dtype, pre, "NaN positions differ")
        bad = np.argwhere((got != want) & ~wn)
        assert len(bad) == 0, (W, dtype, pre, bad[:4].tolist(), got[tuple(bad[0])], want[tuple(bad[0])])


def full_size_flush(w, reduce_to_owner, in_place, zero2=False, planned=False):
    import torch
    U.say("full-size flush", w.name, "zero2" if zero2 else ("owner" if reduce_to_owner else "allreduce"),
          f"W={w.W} cols={w.total} buckets={len(w.buckets)}", "planned" if planned else "")
    ld = w.ld
    x = U.gen_slab(w.dtype, w.W, ld, w.total, w.value_seed, 0, w.scale)
    y = x if in_place else U.empty_slab(w.dtype, w.W, ld)
    ex = executor.from_workload(w, reduce_to_owner=reduce_to_owner, zero2=zero2)
    ex.build_owner_map()
    if planned:
        ex.plan()
    for b in range(len(w.buckets)):
        ex.flush(b, x, ld, y, ld)
    torch.cuda.synchronize()
    cols = U.sample_columns(w)
    if zero2:
        # add the columns on both sides of every partition boundary
        _, psize = U.psize_per_param(w)
        flat, _ = U.psize_per_param(w)
        extra = []
        for bk in w.buckets:
            for t in bk.tasks:
                S = int(psize[t.param])
                if S <= 0 or t.numel == 0:
                    continue
                a = int(flat[t.param])
                q = a // S + 1
                while q * S < a + t.numel:
                    e = q * S - a
                    extra += [bk.col + t.offset + e - 1, bk.col + t.offset + e]
                    q += 1
        cols = np.unique(np.concatenate([cols, np.array(extra, np.int64)]))
    U.say("  sampled columns", len(cols))
    got = y[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    got = got.view(np.uint16) if w.dtype == wl.DT_BF16 else got.view(np.uint32)
    _, _, _, _, owner, _ = U.oracle_owner(w)
    want = U.oracle_sampled_flush(w, cols, owner if reduce_to_owner else None, zero2=zero2)
    if in_place:
        # rows the flush does not write keep the input
        inp = np.stack([synth.gather(w.dtype, w.value_seed, r, w.scale, cols) for r in range(w.W)])
        wb = U.bits(want, w.dtype)
        sent = U.SENTINEL16 if w.dtype == wl.DT_BF16 else U.SENTINEL32
        wb = np.where(wb == sent, inp.view(wb.dtype), wb)
        want = wb
    want = U.bits(want, w.dtype)
    bad = np.argwhere(got != want)
    del x, y
    torch.cuda.empty_cache()
    assert len(bad) == 0, f"{len(bad)} mismatches; first {bad[:5].tolist()} cols {cols[bad[:5, 1]]}"


@pytest.mark.parametrize("owner", [True, False], ids=["owner", "allreduce"])
def test_flush_w8_402m_full_size(owner):
    full_size_flush(wl.owner_flush_w8(), owner, in_place=False)


@pytest.mark.parametrize("owner", [True, False], ids=["owner", "allreduce"])
def test_flush_w8_402m_layered_full_size(owner):
    full_size_flush(wl.owner_flush_w8_layered(), owner, in_place=False)


def test_flush_w16_mixed_1_2b_full_size_in_place():
    full_size_flush(wl.mixed_flush_w16(), True, in_place=True)


def test_flush_zero2_w8_402m_full_size():
    full_size_flush(wl.owner_flush_w8(), False, in_place=False, zero2=True)


def test_flush_zero2_w16_mixed_1_2b_full_size_in_place():
    full_size_flush(wl.mixed_flush_w16(), False, in_place=True, zero2=True)


def test_flush_robust_to_bad_tables():
    """The documented contract for a task table that breaks the rules: an
    out-of-range param or owner entry means AllReduce, an out-of-range comm
    means comm 0, a task running past the bucket is cut at its end, and no
    column outside the bucket is written.  The oracle runs the same table
    with those readings applied by hand."""
    import torch
    W, dtype = 8, wl.DT_BF16
    P = 6
    owner = np.array([3, 9, -7, -1, 0, 7], np.int32)      # 9 and -7 are out of range
    col0, bucket_numel = 40, 5000
    tasks = [(0, 700, 0, 0), (700, 900, 1, 0), (1600, 333, 2, 0), (1933, 1000, P + 5, 0),
             (2933, 400, 4, 5), (3333, 2000, 5, 0)]             # param P+5, comm 5, past the end
    ld = wl.round_up(col0 + bucket_numel + 3000, 64)
    scale = wl.sigma_scale(1e-2)
    x = U.gen_slab(dtype, W, ld, ld, 123, 0, scale)
    y = U.empty_slab(dtype, W, ld)
    t = dc.tasks_array(tasks)
    d_tasks = torch.from_numpy(t.view(np.uint8).copy()).cuda()
    d_owner = torch.from_numpy(owner).cuda()
    dc.dc_flush_bucket(W, dtype, x, ld, y, ld, col0, bucket_numel, d_tasks, len(tasks), d_owner, P,
                       [(W, 1)], 1, 1)
    torch.cuda.synchronize()
    # the readings, applied by hand for the oracle
    own_fixed = np.where((owner >= 0) & (owner < W), owner, -1).astype(np.int32)
    own_fixed = np.concatenate([own_fixed, [-1]]).astype(np.int32)   # param P: the bad one
    fixed = []
    for off, n, p, c in tasks:
        p = p if 0 <= p < P else P
        c = c if c == 0 else 0
        n = min(n, bucket_numel - off)
        fixed.append((off, n, p, c))
    hin = U.host_slab(dtype, W, ld, ld, 123, 0, scale)
    hout = np.full_like(hin, U.SENTINEL16)
    oracle.flush(W, dtype, hin, hout, col0, [f[0] for f in fixed], [f[1] for f in fixed],
                 [f[2] for f in fixed], [f[3] for f in fixed], own_fixed, [W], [1], 1)
    assert np.array_equal(U.to_host(y, dtype), hout)


@pytest.mark.parametrize("seed", range(12))
def test_flush_random_abi_cases(seed):
    """Seeded random flushes straight through the ABI: random W, dtype,
    communicators, owners, pre-division, bucket start column (any residue),
    task sizes from 0 to several tiles, in and out of place."""
    import torch
    rng = random.Random(1000 + seed)
    W = rng.choice([1, 2, 3, 4, 6, 8, 12, 16])
    dtype = rng.choice([wl.DT_BF16, wl.DT_F32])
    divs = [c for c in range(1, W) if W % c == 0]
    comms = [(W, 1)]
    if divs and rng.random() < 0.7:
        c = rng.choice(divs)
        comms.append((c, rng.choice([1, W // c])))
    n_tasks = rng.randint(1, 40)
    sizes = [rng.choice([0, 1, 2, 7, 8, 9, 63, 64, 65, 511, 513, 1024, 3000, 9000]) for _ in range(n_tasks)]
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(int).tolist()
    bucket_numel = int(sum(sizes))
    P = n_tasks
    owner = np.array([rng.choice([-1, rng.randrange(W)]) for _ in range(P)], np.int32)
    t_comm = [rng.randrange(len(comms)) for _ in range(n_tasks)]
    tasks = [(offs[k], sizes[k], k, t_comm[k]) for k in range(n_tasks)]
    col0 = rng.randint(0, 17)
    pre = rng.randint(0, 1)
    in_place = rng.random() < 0.3
    ld = max(64, wl.round_up(col0 + bucket_numel + rng.randint(0, 100), 64))
    scale = wl.sigma_scale(1e-2)
    U.say("random flush", seed, W, dtype, comms, n_tasks, bucket_numel, col0, pre, in_place)
    x = U.gen_slab(dtype, W, ld, ld, 300 + seed, 0, scale)
    y = x if in_place else U.empty_slab(dtype, W, ld)
    t = dc.tasks_array(tasks)
    dc.dc_validate_tasks(W, t, len(t), bucket_numel, P, comms, len(comms))
    d_tasks = torch.from_numpy(t.view(np.uint8).copy()).cuda()
    use_owner = rng.random() < 0.7
    d_owner = torch.from_numpy(owner).cuda() if use_owner else None
    dc.dc_flush_bucket(W, dtype, x, ld, y, ld, col0, bucket_numel, d_tasks, len(tasks), d_owner, P,
                       comms, len(comms), pre)
    torch.cuda.synchronize()
    hin = U.host_slab(dtype, W, ld, ld, 300 + seed, 0, scale)
    if in_place:
        hout = hin
    else:
        hout = np.zeros_like(hin)
        U.bits(hout, dtype)[:] = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
    oracle.flush(W, dtype, hin, hout, col0, offs, sizes, list(range(n_tasks)), t_comm,
                 owner if use_owner else None, [c for c, _ in comms], [s for _, s in comms], pre)
    assert np.array_equal(U.bits(U.to_host(y, dtype), dtype), U.bits(hout, dtype))
