"""GPU parity of the bucket relayout and the variable-shard reduce-scatter
(the reduce-scatter alternative of the DeepSpeed issue), through the C ABI,
against the oracle: bit-exact."""
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


def run_bucket(w, b, x, ld, col_shift=0, planned=False, keep=None):
    """Relayout (searched, or from its tile plan) + reduce-scatter-v of
    bucket b on the GPU; returns host (relaid, shards, seg, pieces, flat,
    psize).  keep: a dict that receives the device relaid slab."""
    import torch
    bk = w.buckets[b]
    flat, psize = U.psize_per_param(w)
    t = dc.tasks_array([(k.offset, k.numel, k.param, k.comm) for k in bk.tasks])
    pieces, seg = dc.dc_plan_relayout(w.W, t, len(t), flat, psize, w.P)
    n = int(seg[-1])
    ld_r = max(64, wl.round_up(n, 64))
    relaid = U.empty_slab(w.dtype, w.W, ld_r)
    d_pieces = torch.from_numpy(pieces.view(np.uint8).copy()).cuda() if len(pieces) else \
        torch.zeros(32, dtype=torch.uint8, device="cuda")
    if planned:
        tiles = dc.dc_plan_relayout_tiles(w.dtype, bk.col + col_shift, bk.numel, pieces, len(pieces), n)
        d_tiles = torch.from_numpy(tiles).cuda() if len(tiles) else None
        dc.dc_relayout_bucket_planned(w.W, w.dtype, x, ld, relaid, ld_r, bk.col + col_shift, bk.numel,
                                      d_pieces, len(pieces), n, d_tiles, len(tiles))
    else:
        dc.dc_relayout_bucket(w.W, w.dtype, x, ld, relaid, ld_r, bk.col + col_shift, bk.numel,
                              d_pieces, len(pieces), n)
    maxlen = int(max(seg[1:] - seg[:-1])) if w.W else 0
    ld_s = max(64, wl.round_up(maxlen, 64))
    shards = U.empty_slab(w.dtype, w.W, ld_s)
    dc.dc_reduce_scatter_v(w.W, w.dtype, relaid, ld_r, shards, ld_s, seg, w.pre_div)
    torch.cuda.synchronize()
    if keep is not None:
        keep["relaid"], keep["ld_r"] = relaid, ld_r
        return None, U.to_host(shards, w.dtype), seg, pieces, flat, psize
    return U.to_host(relaid, w.dtype), U.to_host(shards, w.dtype), seg, pieces, flat, psize


def small_workloads():
    rng = random.Random(23)
    out = []
    for W in (2, 3, 4, 8, 16):
        for dtype in (wl.DT_BF16, wl.DT_F32):
            sizes = [rng.choice([0, 1, 3, 7, 9, 64, 100, 1000, 5000]) for _ in range(50)]
            out.append(wl.custom_flush(f"W{W}-{wl.DTYPE_NAME[dtype]}", W, dtype, sizes,
                                       group_begin=[0, 30, 50], group_comm=[0, 0],
                                       comms=[wl.Comm(W, 1)], capacity=20_000,
                                       pre_div=(W + dtype) % 2, value_seed=40 + W))
    return out


@pytest.mark.parametrize("planned", [False, True], ids=["searched", "planned"])
@pytest.mark.parametrize("w", small_workloads(), ids=lambda w: w.name)
def test_relayout_reduce_scatter_small(w, planned):
    U.say("relayout", w.name, "planned" if planned else "searched")
    ld = w.ld
    x = U.gen_slab(w.dtype, w.W, ld, w.total, w.value_seed, 0, w.scale)
    hx = U.host_slab(w.dtype, w.W, ld, w.total, w.value_seed, 0, w.scale)
    for b, bk in enumerate(w.buckets):
        relaid, shards, seg, pieces, flat, psize = run_bucket(w, b, x, ld, planned=planned)
        t_off = [k.offset for k in bk.tasks]
        t_numel = [k.numel for k in bk.tasks]
        t_param = [k.param for k in bk.tasks]
        t_comm = [k.comm for k in bk.tasks]
        dest, oseg = oracle.relayout_map(w.W, t_off, t_numel, t_param, t_comm, flat, psize, bk.numel)
        assert np.array_equal(seg, oseg)
        hr = np.zeros_like(relaid)
        U.bits(hr, w.dtype)[:] = U.SENTINEL16 if w.dtype == wl.DT_BF16 else U.SENTINEL32
        # the oracle relayout reads the bucket in place in the full slab
        oracle.relayout_apply(w.W, w.dtype, hx, hr, bk.col, bk.numel, dest)
        assert np.array_equal(U.bits(relaid, w.dtype), U.bits(hr, w.dtype)), (w.name, b)
        hs = np.zeros_like(shards)
        U.bits(hs, w.dtype)[:] = U.SENTINEL16 if w.dtype == wl.DT_BF16 else U.SENTINEL32
        oracle.reduce_scatter_v(w.W, w.dtype, hr, hs, oseg, w.pre_div)
        assert np.array_equal(U.bits(shards, w.dtype), U.bits(hs, w.dtype)), (w.name, b)


@pytest.mark.parametrize("planned", [False, True], ids=["searched", "planned"])
def test_relayout_unaligned_bucket_start(planned):
    """A bucket whose first column is not vector aligned: every source vector
    is misaligned, so the element path moves everything (the tile plan
    records no straight copy)."""
    import torch
    w = wl.custom_flush("unaligned", 8, wl.DT_BF16, [100, 37, 2000, 5], capacity=10 ** 9, pre_div=1)
    shift = 3
    ld = wl.round_up(w.total + shift, 64)
    x = U.gen_slab(w.dtype, w.W, ld, ld, 5, 0, w.scale)
    hx = U.host_slab(w.dtype, w.W, ld, ld, 5, 0, w.scale)
    relaid, shards, seg, pieces, flat, psize = run_bucket(w, 0, x, ld, col_shift=shift, planned=planned)
    bk = w.buckets[0]
    dest, oseg = oracle.relayout_map(w.W, [k.offset for k in bk.tasks], [k.numel for k in bk.tasks],
                                     [k.param for k in bk.tasks], [k.comm for k in bk.tasks], flat,
                                     psize, bk.numel)
    hr = np.full_like(relaid, U.SENTINEL16)
    oracle.relayout_apply(w.W, w.dtype, hx, hr, shift, bk.numel, dest)
    assert np.array_equal(relaid, hr)


def test_relayout_reduce_scatter_w8_402m_full_size():
    """Every bucket of the 402.8M-element W=8 workload, relaid from its tile
    plan as the bench does: every relaid column of every row against the
    relayout's definition (out[r][dst + i] = in[r][bucket_col + src + i],
    gathered by torch), and sampled shard positions against the oracle's
    ZeRO-2 values of their source columns."""
    import torch
    w = wl.owner_flush_w8()
    U.say("relayout full size", w.total)
    x = U.gen_slab(w.dtype, w.W, w.ld, w.total, w.value_seed, 0, w.scale)
    rng = np.random.default_rng(2)
    for b, bk in enumerate(w.buckets):
        keep = {}
        _, shards, seg, pieces, flat, psize = run_bucket(w, b, x, w.ld, planned=True, keep=keep)
        n = int(seg[-1])
        src_of = np.full(n, -1, np.int64)
        for pc in pieces:
            src_of[pc["dst"]:pc["dst"] + pc["len"]] = bk.col + pc["src"] + np.arange(pc["len"])
        assert np.all(src_of >= 0), b
        idx = torch.from_numpy(src_of).cuda()
        want = torch.index_select(x, 1, idx)
        assert torch.equal(keep["relaid"][:, :n], want), b
        del keep, idx, want
        # sample destination positions: piece ends and random
        picks = set()
        for pc in pieces[rng.choice(len(pieces), size=min(40, len(pieces)), replace=False)]:
            picks.update([int(pc["dst"]), int(pc["dst"] + pc["len"] - 1)])
        picks.update(rng.integers(0, int(seg[-1]), 200).tolist())
        picks = np.array(sorted(picks), np.int64)
        order = np.argsort(pieces["dst"])
        dsts = pieces["dst"][order]
        idx = np.searchsorted(dsts, picks, side="right") - 1
        pc = pieces[order][idx]
        src_cols = bk.col + pc["src"] + (picks - pc["dst"])
        want = U.oracle_sampled_flush(w, src_cols, None, zero2=True)
        q = np.searchsorted(seg, picks, side="right") - 1
        got = shards[q, picks - seg[q]]
        wb = U.bits(want, w.dtype)
        assert np.array_equal(U.bits(got, w.dtype), wb[q, np.arange(len(picks))]), b
    del x
    torch.cuda.empty_cache()


RSV_CASES = [(W, dtype, pre) for W in (1, 2, 3, 4, 8, 16) for dtype in (wl.DT_BF16, wl.DT_F32)
             for pre in (0, 1) if (W + pre) % 2 == 0 or W in (8, 16)]


@pytest.mark.parametrize("W,dtype,pre", RSV_CASES, ids=lambda v: str(v))
def test_reduce_scatter_v_every_offset(W, dtype, pre):
    """Segments starting at every offset inside a 16-byte vector, with
    lengths below, at and above a vector and spanning several tiles: the
    shifted-vector path and the element tail, bit-exact."""
    import torch
    rng = random.Random(500 + W + 10 * dtype)
    E = 8 if dtype == wl.DT_BF16 else 4
    lens = []
    for q in range(W):
        k = q % 6
        lens.append([0, 1, E - 1, E, E + 3, 3000 + rng.randint(0, 2 * E)][k] if W <= 6 else
                    rng.choice([0, 1, E, 2 * E + 1, 777, 5000 + rng.randint(0, E)]))
    # shift every segment start so starts cover all residues mod E
    seg = [0]
    for q in range(W):
        seg.append(seg[-1] + lens[q])
    pad = rng.randint(0, E - 1)
    seg = [s + pad for s in seg]
    seg[0] = 0   # the first shard runs from 0: it absorbs the pad
    n = seg[-1]
    ld = max(64, wl.round_up(n, 64))
    scale = wl.sigma_scale(1e-2)
    x = U.gen_slab(dtype, W, ld, n, 61 + W, 0, scale)
    hx = U.host_slab(dtype, W, ld, n, 61 + W, 0, scale)
    maxlen = max(seg[q + 1] - seg[q] for q in range(W))
    ld_s = max(64, wl.round_up(maxlen, 64))
    sh = U.empty_slab(dtype, W, ld_s)
    U.say("rs-v offsets", W, dtype, pre, [s % E for s in seg[:-1]])
    dc.dc_reduce_scatter_v(W, dtype, x, ld, sh, ld_s, seg, pre)
    torch.cuda.synchronize()
    hs = np.zeros((W, ld_s), hx.dtype)
    U.bits(hs, dtype)[:] = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
    oracle.reduce_scatter_v(W, dtype, hx, hs, seg, pre)
    assert np.array_equal(U.bits(U.to_host(sh, dtype), dtype), U.bits(hs, dtype))


def test_reduce_scatter_v_all_residues():
    """W=8 bf16 with segment q starting at residue q mod 8, several tiles long."""
    import torch
    W, dtype, E = 8, wl.DT_BF16, 8
    seg = [0]
    for q in range(W):
        seg.append(seg[-1] + 4099 * 8 + 1)   # each start advances the residue by one
    n = seg[-1]
    assert sorted(s % E for s in seg[:-1]) == list(range(E))
    ld = wl.round_up(n, 64)
    scale = wl.sigma_scale(1e-2)
    x = U.gen_slab(dtype, W, ld, n, 77, 0, scale)
    hx = U.host_slab(dtype, W, ld, n, 77, 0, scale)
    ld_s = wl.round_up(4099 * 8 + 1, 64)
    for pre in (0, 1):
        sh = U.empty_slab(dtype, W, ld_s)
        dc.dc_reduce_scatter_v(W, dtype, x, ld, sh, ld_s, seg, pre)
        torch.cuda.synchronize()
        hs = np.zeros((W, ld_s), np.uint16)
        hs[:] = U.SENTINEL16
        oracle.reduce_scatter_v(W, dtype, hx, hs, seg, pre)
        assert np.array_equal(U.to_host(sh, dtype), hs), pre


def test_relayout_planned_equals_searched_random_pieces():
    """dc_relayout_bucket_planned against dc_relayout_bucket on random piece
    tables (gaps, empty pieces, unaligned sources, and pieces that start
    inside earlier ones, where a column belongs to the last piece starting at
    or before it): the same output, bit for bit, sentinel where no piece
    writes."""
    import torch
    rng = random.Random(31)
    whole = 0
    for case in range(36):
        W = [1, 3, 2, 4, 8, 16, 5, 32, 64][case % 9]
        dtype = rng.choice([wl.DT_BF16, wl.DT_F32])
        numel = rng.randint(1, 30_000)
        col = rng.choice([0, 8, 64, 3, 1024])
        overlap = case % 2 == 1
        dst, pcs = 0, []
        for _ in range(rng.randint(1, 14)):
            dst += rng.choice([0, 0, 1, 8, 300])
            ln = rng.choice([0, 5, 512, 1024, 3000, 7000])
            src = rng.choice([0, 8, 512, 1000, rng.randint(0, numel)])
            ln = max(0, min(ln, numel - src))
            pcs.append((src, dst, ln, 0))
            dst += rng.choice([0, 100, ln // 2]) if overlap else ln
        pieces = np.array(pcs, dc.PIECE_DTYPE)
        out_numel = dst + rng.choice([0, 7, 600])
        ld_in = wl.round_up(col + numel, 64)
        ld_out = max(64, wl.round_up(out_numel, 64))
        U.say("relayout planned vs searched", case, W, wl.DTYPE_NAME[dtype], numel, len(pcs), out_numel)
        x = U.gen_slab(dtype, W, ld_in, ld_in, 50 + case, 0, wl.sigma_scale(0.01))
        d_pieces = torch.from_numpy(pieces.view(np.uint8).copy()).cuda()
        tiles = dc.dc_plan_relayout_tiles(dtype, col, numel, pieces, len(pieces), out_numel)
        d_tiles = torch.from_numpy(tiles).cuda() if len(tiles) else None
        outs = []
        for planned in (False, True):
            y = U.empty_slab(dtype, W, ld_out)
            if planned:
                dc.dc_relayout_bucket_planned(W, dtype, x, ld_in, y, ld_out, col, numel, d_pieces,
                                              len(pieces), out_numel, d_tiles, len(tiles))
            else:
                dc.dc_relayout_bucket(W, dtype, x, ld_in, y, ld_out, col, numel, d_pieces, len(pieces),
                                      out_numel)
            outs.append(y)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), case
        whole += int((tiles >= 0).sum())
    assert whole > 20          # the straight copy ran, not only the search


def test_relayout_stale_plan_stays_in_bounds():
    """A tile plan of random records (negative, huge, near the bucket's ends,
    other tiles' sources): the planned relayout may misplace data inside
    [0, out_numel) but writes nothing past it and leaves the input alone."""
    import torch
    rng = random.Random(5)
    for case in range(12):
        W = [1, 2, 4, 8, 16, 3][case % 6]
        dtype = rng.choice([wl.DT_BF16, wl.DT_F32])
        E = 8 if dtype == wl.DT_BF16 else 4
        numel = rng.randint(2000, 30_000)
        col = rng.choice([0, 8, 64, 3])
        dst, pcs = 0, []
        for _ in range(rng.randint(1, 10)):
            ln = rng.choice([512, 1024, 3000, 7000])
            src = rng.choice([0, 8, 512, rng.randint(0, numel)])
            ln = max(0, min(ln, numel - src))
            pcs.append((src, dst, ln, 0))
            dst += ln
        pieces = np.array(pcs, dc.PIECE_DTYPE)
        out_numel = dst
        tiles = dc.dc_plan_relayout_tiles(dtype, col, numel, pieces, len(pieces), out_numel)
        if len(tiles) == 0:
            continue
        hi = (col + numel) // E
        pool = [-1, -(2 ** 62), 2 ** 62, 2 ** 61 + 3, hi, hi - 64, hi - 63, col // E, 0]
        tiles = np.array([rng.choice(pool + [int(v) for v in tiles] + [rng.randint(0, hi + 100)])
                          for _ in range(len(tiles))], np.int64)
        ld_in = wl.round_up(col + numel, 64)
        ld_out = wl.round_up(out_numel + 1024, 64)
        U.say("relayout stale plan", case, W, wl.DTYPE_NAME[dtype], numel, out_numel)
        x = U.gen_slab(dtype, W, ld_in, ld_in, 70 + case, 0, wl.sigma_scale(0.01))
        hx = U.bits(U.to_host(x, dtype), dtype).copy()
        y = U.empty_slab(dtype, W, ld_out)
        d_pieces = torch.from_numpy(pieces.view(np.uint8).copy()).cuda()
        dc.dc_relayout_bucket_planned(W, dtype, x, ld_in, y, ld_out, col, numel, d_pieces, len(pieces),
                                      out_numel, torch.from_numpy(tiles).cuda(), len(tiles))
        torch.cuda.synchronize()
        got = U.bits(U.to_host(y, dtype), dtype)
        sent = U.SENTINEL16 if dtype == wl.DT_BF16 else U.SENTINEL32
        assert np.all(got[:, out_numel:] == sent), case
        assert np.array_equal(U.bits(U.to_host(x, dtype), dtype), hx), case


@pytest.mark.parametrize("planned", [False, True, "device"],
                         ids=["searched", "host-planned", "device-planned"])
@pytest.mark.parametrize("w", small_workloads()[::3], ids=lambda w: w.name)
def test_relayout_reduce_scatter_via_executor(w, planned):
    """The executor's relayout path (plan_relayout, relayout_reduce_scatter),
    searched or from tile plans built on the host or on the device: every
    bucket's relaid slab and shards against the oracle."""
    import torch
    U.say("executor relayout", w.name, planned)
    ld = w.ld
    x = U.gen_slab(w.dtype, w.W, ld, w.total, w.value_seed, 0, w.scale)
    hx = U.host_slab(w.dtype, w.W, ld, w.total, w.value_seed, 0, w.scale)
    ex = executor.from_workload(w, reduce_to_owner=False, zero2=True)
    ex.build_owner_map()
    ex.plan_relayout(planned=planned)
    flat, psize = U.psize_per_param(w)
    sent = U.SENTINEL16 if w.dtype == wl.DT_BF16 else U.SENTINEL32
    for b, bk in enumerate(w.buckets):
        n, longest = ex.relayout_sizes(b)
        ld_r, ld_s = max(64, wl.round_up(n, 64)), max(64, wl.round_up(longest, 64))
        relaid = U.empty_slab(w.dtype, w.W, ld_r)
        shards = U.empty_slab(w.dtype, w.W, ld_s)
        ex.relayout_reduce_scatter(b, x, ld, relaid, ld_r, shards, ld_s)
        torch.cuda.synchronize()
        dest, oseg = oracle.relayout_map(w.W, [k.offset for k in bk.tasks], [k.numel for k in bk.tasks],
                                         [k.param for k in bk.tasks], [k.comm for k in bk.tasks], flat,
                                         psize, bk.numel)
        hr = np.zeros((w.W, ld_r), hx.dtype)
        U.bits(hr, w.dtype)[:] = sent
        oracle.relayout_apply(w.W, w.dtype, hx, hr, bk.col, bk.numel, dest)
        assert np.array_equal(U.bits(U.to_host(relaid, w.dtype), w.dtype), U.bits(hr, w.dtype)), b
        hs = np.zeros((w.W, ld_s), hx.dtype)
        U.bits(hs, w.dtype)[:] = sent
        oracle.reduce_scatter_v(w.W, w.dtype, hr, hs, oseg, w.pre_div)
        assert np.array_equal(U.bits(U.to_host(shards, w.dtype), w.dtype), U.bits(hs, w.dtype)), b
