"""Pins that tie the CPU oracle to what the pages and the mathematics fix.

Each pin raises AssertionError when the oracle disagrees.  They are run
against the real oracle (tests/test_oracle_pins.py) and against builds of the
oracle with a planted mistake (tests/test_oracle_mutants.py), where at least
one pin must fail.

Nothing here computes an expected value with the oracle's own code path:
expected values come from printed tables (tests/golden), closed forms, exact
rational arithmetic (tests/ieee_exact.py), element-by-element brute force,
or torch's CPU bfloat16 conversion.
"""
import itertools
import math
import os
import random
from fractions import Fraction

import numpy as np

import oracle
from tests import ieee_exact as X

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

BF16, F32 = oracle.BF16, oracle.F32


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def one_task_flush(W, dtype, rows, pre_div, comm=(None, None), owner=None):
    """Flush one task covering every column of `rows` ([W, n] bits or floats)."""
    rows = np.ascontiguousarray(rows)
    n = rows.shape[1]
    out = np.zeros_like(rows)
    if comm[0] is None:
        cs, cst, tc = [W], [1], 0
    else:
        cs, cst, tc = [W, comm[0]], [1, comm[1]], 1
    ow = None if owner is None else np.array([owner], np.int32)
    oracle.flush(W, dtype, rows, out, 0, [0], [n], [0], [tc], ow, cs, cst, pre_div)
    return out


def random_bits(rng, dtype, shape, wide=True):
    """Random finite patterns over a range of exponents, including zeros of
    both signs and subnormals (bf16 exponent field 0), far from overflow."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint32)
    for k in range(n):
        sign = rng.getrandbits(1)
        pick = rng.random()
        if pick < 0.05:
            e = 0
            man = 0
        elif pick < 0.2 and wide:
            e = 0
            man = rng.getrandbits(7 if dtype == BF16 else 23) or 1
        elif pick < 0.3 and wide:
            e = rng.randint(1, 4)
            man = rng.getrandbits(7 if dtype == BF16 else 23)
        else:
            e = rng.randint(110, 135)
            man = rng.getrandbits(7 if dtype == BF16 else 23)
        if dtype == BF16:
            out[k] = (sign << 15) | (e << 7) | man
        else:
            out[k] = (sign << 31) | (e << 23) | man
    if dtype == BF16:
        return out.astype(np.uint16).reshape(shape)
    return out.view(np.float32).reshape(shape)


def to_floats(dtype, arr):
    if dtype == BF16:
        return [X.bf16_bits_to_float(int(b)) for b in np.asarray(arr).ravel()]
    return [float(v) for v in np.asarray(arr, np.float32).ravel()]


def bits_of(dtype, v):
    return X.float_to_bf16_bits(v) if dtype == BF16 else X.float_to_f32_bits(v)


def out_bits(dtype, arr):
    a = np.asarray(arr)
    return a.astype(np.uint32) if dtype == BF16 else a.view(np.uint32)


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

def _definitional_bf16(u):
    """Nearest bf16 neighbour by exact distance (double arithmetic holds every
    difference exactly), ties to the even pattern; unbounded exponent for the
    upper neighbour so the overflow threshold falls at max + half an ulp."""
    u = u.astype(np.uint64)
    sign = (u >> 31) & 1
    mag = u & 0x7FFFFFFF
    e32 = (mag >> 23).astype(np.int64)
    m32 = (mag & 0x7FFFFF).astype(np.float64)
    f = np.where(e32 == 0, np.ldexp(m32, -149), np.ldexp(m32 + 2.0 ** 23, (e32 - 150).astype(np.int32)))

    def val16(p):
        e = (p >> 7).astype(np.int64)
        m = (p & 0x7F).astype(np.float64)
        return np.where(e == 0, np.ldexp(m, -133), np.ldexp(m + 128.0, (e - 134).astype(np.int32)))

    lo = (mag >> 16)
    hi = lo + 1
    dlo = f - val16(lo)
    dhi = val16(hi) - f
    pick = np.where((dhi < dlo) | ((dhi == dlo) & ((lo & 1) == 1)), hi, lo)
    return ((sign << 15) | pick).astype(np.uint16)


def pin_bf16_rounding():
    rng = np.random.default_rng(11)
    highs = np.arange(65536, dtype=np.uint64)
    highs = highs[((highs >> 7) & 0xFF) != 0xFF]          # finite only
    lows = np.array([0, 1, 2, 0x7FFF, 0x8000, 0x8001, 0xFFFE, 0xFFFF], np.uint64)
    lows = np.concatenate([lows, rng.integers(0, 65536, 24).astype(np.uint64)])
    u = ((highs[:, None] << 16) | lows[None, :]).ravel().astype(np.uint32)
    got = oracle.bf16_round(u.view(np.float32))
    want = _definitional_bf16(u)
    bad = np.nonzero(got != want)[0]
    assert len(bad) == 0, f"bf16 rounding differs at {u[bad[:5]]}: {got[bad[:5]]} vs {want[bad[:5]]}"
    # specials: infinities stay, every NaN becomes the quiet NaN with its sign
    sp = np.array([0x7F800000, 0xFF800000, 0x7F800001, 0xFFC00000, 0x7FFFFFFF, 0x7FBF0000],
                  np.uint32)
    got = oracle.bf16_round(sp.view(np.float32))
    assert list(got) == [0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7FC0, 0x7FC0], [hex(g) for g in got]


def pin_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(12)
    u = rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    u = u[((u >> 23) & 0xFF) != 0xFF]
    got = oracle.bf16_round(u.view(np.float32))
    want = torch.from_numpy(u.view(np.float32).copy()).to(torch.bfloat16).view(torch.int16)
    want = want.numpy().view(np.uint16)
    assert np.array_equal(got, want), "bf16 rounding differs from torch's CPU conversion"


# ---------------------------------------------------------------------------
# the fold (flush, reduce-scatter, deferred reduce)
# ---------------------------------------------------------------------------

def pin_fold_rank_order():
    """Hand-derived: rows (2^24, 1, -2^24, 1) summed in rank order give
    2^24 + 1 -> 2^24 (a tie, to even), then 0, then 1.  Any other order of
    the first two additions gives a different answer (reversed: 2)."""
    for dtype in (F32, BF16):
        if dtype == F32:
            col = np.array([[2.0 ** 24], [1.0], [-(2.0 ** 24)], [1.0]], np.float32)
        else:
            col = np.array([[0x4B80], [0x3F80], [0xCB80], [0x3F80]], np.uint16)
        out = one_task_flush(4, dtype, col, pre_div=0)
        want = 0x3F800000 if dtype == F32 else 0x3F80
        got = out_bits(dtype, out)
        assert np.all(got[:, 0] == want), f"rank-order fold gave {got[:, 0]} (dtype {dtype})"


def pin_fold_exact_sums():
    """Values k * 2^-20 with |k| < 256: every partial sum is exact in fp32, so
    the result is the exact rational sum for any W (pre-division by a power of
    two is exact too)."""
    rng = random.Random(21)
    for dtype in (BF16, F32):
        for W in (1, 2, 3, 4, 5, 8, 16):
            n = 17
            ks = [[rng.randint(-255, 255) for _ in range(n)] for _ in range(W)]
            vals = np.array(ks, np.float64) * 2.0 ** -20
            rows = vals.astype(np.float32)
            if dtype == BF16:
                rows = (rows.view(np.uint32) >> 16).astype(np.uint16)
            for pre in ((0, 1) if (W & (W - 1)) == 0 else (0,)):
                out = one_task_flush(W, dtype, rows, pre_div=pre)
                got = np.array(to_floats(dtype, out[0]))
                exact = [Fraction(sum(ks[r][j] for r in range(W)), 2 ** 20) / (W if pre else 1)
                         for j in range(n)]
                want = [X.round_to(q, X.BFLOAT16 if dtype == BF16 else X.BINARY32) for q in exact]
                assert np.array_equal(got, np.array(want)), f"exact sums wrong, W={W} dtype={dtype}"


def pin_fold_identical_rows():
    """DeepSpeed issue, Numerics: identical input on every rank reproduces
    exactly.  With pre-division by W = 2^k each bf16 contribution is x/W and the
    k-fold sum is exactly x; without it the sum is exactly W*x."""
    rng = random.Random(22)
    for W in (2, 4, 8, 16):
        row = np.array([(rng.getrandbits(1) << 15) | (rng.randint(100, 140) << 7) |
                        rng.getrandbits(7) for _ in range(40)], np.uint16)
        rows = np.tile(row, (W, 1))
        out = one_task_flush(W, BF16, rows, pre_div=1)
        assert np.array_equal(out, rows), f"identical rows with pre-division not reproduced, W={W}"
        out = one_task_flush(W, BF16, rows, pre_div=0)
        want = np.array([X.float_to_bf16_bits(W * X.bf16_bits_to_float(int(b))) for b in row],
                        np.uint16)
        assert np.all(out == want[None, :]), f"identical rows without pre-division, W={W}"


def pin_fold_brute_force():
    """Random tiny slabs (subnormals and signed zeros included, W up to 16,
    sub-communicators, pre-division on and off) against the exact-rational
    model of the rank-order fp32 fold."""
    rng = random.Random(23)
    for trial in range(90):
        dtype = (BF16, F32)[trial % 2]
        W = (1, 2, 3, 4, 5, 6, 7, 8, 16)[trial % 9]
        pre = (trial // 9) % 2
        divs = [c for c in range(1, W + 1) if W % c == 0 and c < W]
        comm = (None, None)
        if divs and trial % 3 == 2:
            c = rng.choice(divs)
            comm = (c, rng.choice([1, W // c]) if c > 1 else 1)
        n = rng.randint(1, 12)
        rows = random_bits(rng, dtype, (W, n))
        out = one_task_flush(W, dtype, rows, pre_div=pre, comm=comm)
        vals = [to_floats(dtype, rows[r]) for r in range(W)]
        c, s = (W, 1) if comm[0] is None else comm
        for b in range(W // c):
            base = b * c if s == 1 else b
            members = [base + i * s for i in range(c)]
            for j in range(n):
                y = X.fold([vals[m][j] for m in members], dtype == BF16, bool(pre), c)
                for m in members:
                    got = int(out_bits(dtype, out)[m, j])
                    want = bits_of(dtype, y)
                    assert got == want, (f"fold differs: trial {trial} W={W} c={c} s={s} "
                                         f"pre={pre} col {j} row {m}: {got:#x} vs {want:#x}")


def pin_fold_error_bound():
    """|fold - exact| <= gamma_{W-1} * sum|x| (Higham, Accuracy and Stability of
    Numerical Algorithms, ch. 4, recursive summation), fp32, no pre-division."""
    rng = np.random.default_rng(24)
    for W in (2, 3, 8, 16, 64):
        rows = (rng.standard_normal((W, 500)) * 10.0 ** rng.integers(-3, 3, (W, 500))).astype(np.float32)
        out = one_task_flush(W, F32, rows, pre_div=0)
        exact = rows.astype(np.float64).sum(axis=0)          # exact enough: 64 fp32 terms in fp64
        u = 2.0 ** -24
        gamma = (W - 1) * u / (1 - (W - 1) * u)
        bound = gamma * np.abs(rows.astype(np.float64)).sum(axis=0)
        err = np.abs(out[0].astype(np.float64) - exact)
        assert np.all(err <= bound * 1.0000001 + 1e-45), f"error bound violated at W={W}"


def pin_prediv_non_power_of_two():
    """W in {3, 5, 7}: each contribution is x/W correctly rounded to fp32 and
    then to bf16; checked against the exact model, which decides the reading
    column by column."""
    rng = random.Random(25)
    for W in (3, 5, 7):
        rows = random_bits(rng, BF16, (W, 64))
        out = one_task_flush(W, BF16, rows, pre_div=1)
        vals = [to_floats(BF16, rows[r]) for r in range(W)]
        for j in range(64):
            y = X.fold([vals[r][j] for r in range(W)], True, True, W)
            assert int(out[0, j]) == X.float_to_bf16_bits(y), f"pre-division W={W} col {j}"


def pin_reduce_scatter_all_gather():
    """AllGather page: AllReduce = ReduceScatter + AllGather, bit for bit; the
    reduce-scatter shard sizes follow the duality table (M in, M/N out)."""
    rng = random.Random(26)
    for dtype, W, L, pre in ((BF16, 4, 9, 1), (F32, 8, 5, 0), (BF16, 3, 7, 1), (F32, 1, 4, 0)):
        M = W * L
        rows = random_bits(rng, dtype, (W, M), wide=False)
        ar = one_task_flush(W, dtype, rows, pre_div=pre)
        shards = np.zeros((W, L), rows.dtype)
        oracle.reduce_scatter(W, dtype, rows, shards, M, pre)
        assert shards.shape == (W, M // W)
        full = np.zeros((W, M), rows.dtype)
        oracle.all_gather(W, dtype, shards, full, L, 0)
        assert np.array_equal(out_bits(dtype, full), out_bits(dtype, ar)), \
            f"AllReduce != ReduceScatter + AllGather (W={W})"
        vals = [to_floats(dtype, rows[r]) for r in range(W)]
        for s in range(W):
            for k in range(L):
                y = X.fold([vals[r][s * L + k] for r in range(W)], dtype == BF16, bool(pre), W)
                assert int(out_bits(dtype, shards)[s, k]) == bits_of(dtype, y)


def pin_ring_reduce_scatter():
    """Ring reduce-scatter: chunk c's sum is folded in rank order c, c+1, ...
    (mod W).  Hand-derived: W=4, chunk 1 column (1, 2^24, 1, -2^24) gives 0 in
    rank order (2^24+1 rounds to 2^24) but 1 in ring order 1,2,3,0; exact-sum
    inputs give the exact sum; W <= 2 equals rank order; tiny inputs match
    the exact-rational model of the rotated fold."""
    for dtype in (F32, BF16):
        W, L = 4, 1
        if dtype == F32:
            col0 = [2.0 ** 24, 1.0, -(2.0 ** 24), 1.0]
            col1 = [1.0, 2.0 ** 24, 1.0, -(2.0 ** 24)]
            rows = np.array([[a, b, 0, 0] for a, b in zip(col0, col1)], np.float32)
        else:
            enc = {1.0: 0x3F80, 2.0 ** 24: 0x4B80, -(2.0 ** 24): 0xCB80}
            rows = np.array([[enc[a], enc[b], 0, 0] for a, b in zip(
                [2.0 ** 24, 1.0, -(2.0 ** 24), 1.0], [1.0, 2.0 ** 24, 1.0, -(2.0 ** 24)])], np.uint16)
        ring = np.zeros((W, 8), rows.dtype)
        oracle.reduce_scatter_ring(W, dtype, rows, ring, W * L, 0)
        rank = np.zeros((W, 8), rows.dtype)
        oracle.reduce_scatter(W, dtype, rows, rank, W * L, 0)
        one = 0x3F800000 if dtype == F32 else 0x3F80
        assert out_bits(dtype, ring)[0, 0] == one and out_bits(dtype, rank)[0, 0] == one
        assert out_bits(dtype, ring)[1, 0] == one and out_bits(dtype, rank)[1, 0] == 0
    rng = random.Random(101)
    for trial in range(40):
        dtype = (BF16, F32)[trial % 2]
        W = (1, 2, 3, 4, 5, 8)[trial % 6]
        L = rng.randint(1, 5)
        pre = trial % 3 == 0
        rows = random_bits(rng, dtype, (W, W * L + 3))
        ring = np.zeros((W, max(8, L)), rows.dtype)
        oracle.reduce_scatter_ring(W, dtype, rows, ring, W * L, int(pre))
        vals = [to_floats(dtype, rows[r]) for r in range(W)]
        for c in range(W):
            for k in range(L):
                order = [(c + j) % W for j in range(W)]
                y = X.fold([vals[r][c * L + k] for r in order], dtype == BF16, pre, W)
                assert int(out_bits(dtype, ring)[c, k]) == bits_of(dtype, y), (trial, W, c, k)
        if W <= 2:
            rank = np.zeros_like(ring)
            oracle.reduce_scatter(W, dtype, rows, rank, W * L, int(pre))
            assert np.array_equal(out_bits(dtype, ring), out_bits(dtype, rank))
    for W in (3, 8):
        ks = [[rng.randint(-255, 255) for _ in range(W * 3)] for _ in range(W)]
        rows = (np.array(ks, np.float64) * 2.0 ** -20).astype(np.float32)
        ring = np.zeros((W, 8), np.float32)
        oracle.reduce_scatter_ring(W, F32, rows, ring, W * 3, 0)
        for c in range(W):
            for k in range(3):
                assert ring[c, k] == np.float32(sum(ks[r][c * 3 + k] for r in range(W)) * 2.0 ** -20)


# ---------------------------------------------------------------------------
# partitions and the owner map
# ---------------------------------------------------------------------------

def _brute_pids(sizes, p):
    T = sum(sizes)
    S = -(-T // p) if T else 0
    out, a = [], 0
    for n in sizes:
        out.append(sorted({e // S for e in range(a, a + n)}) if n else [])
        a += n
    return out


def pin_partition_brute_force():
    """Element-by-element: partition of element e is floor(e / S) with
    S = ceil(T / p); a parameter's partition list is the set over its
    elements.  All size lists of up to 5 params with sizes 0..4, p = 1..4."""
    for k in range(1, 6):
        for sizes in itertools.product(range(5), repeat=k):
            for p in range(1, 5):
                flat, ps, off, pids = oracle.partition_ids(sizes, [0, k], [p])
                want = _brute_pids(sizes, p)
                for i in range(k):
                    got = list(pids[off[i]:off[i + 1]])
                    assert got == want[i], f"sizes {sizes} p={p} param {i}: {got} vs {want[i]}"
                    assert flat[i] == sum(sizes[:i])


def pin_owner_rules():
    """DeepSpeed issue, Design points: a single-element partition list names
    the owner; straddlers (2+ entries) and empty params keep AllReduce (-1);
    at most p-1 straddlers per group; an excluded group has no owners."""
    rng = random.Random(31)
    for trial in range(300):
        G = rng.randint(1, 3)
        sizes, gb, parts, elig = [], [0], [], []
        for g in range(G):
            k = rng.randint(1, 8)
            sizes += [rng.choice([0, 1, 2, 3, 5, 8, 13, 40]) for _ in range(k)]
            gb.append(len(sizes))
            parts.append(rng.randint(1, 8))
            elig.append(rng.getrandbits(1))
        flat, ps, off, pids = oracle.partition_ids(sizes, gb, parts)
        owner, counts = oracle.owner_map(off, pids, gb, elig)
        for g in range(G):
            gs = sizes[gb[g]:gb[g + 1]]
            want = _brute_pids(gs, parts[g])
            n_own = n_str = 0
            T = sum(gs)
            S = -(-T // parts[g]) if T else 0
            inner = 0
            a = 0
            for i, n in enumerate(gs):
                ent = want[i]
                exp_owner = ent[0] if (elig[g] and len(ent) == 1) else -1
                assert owner[gb[g] + i] == exp_owner, (sizes, gb, parts, elig, g, i)
                n_own += exp_owner >= 0
                n_str += len(ent) >= 2
                if S and any(a < b * S < a + n for b in range(1, parts[g])):
                    inner += 1
                a += n
            assert counts[2 * g] == n_own and counts[2 * g + 1] == n_str
            assert n_str <= parts[g] - 1, "more than p-1 straddlers in a group"
            assert n_str == inner, "straddlers != params holding an interior partition boundary"


def pin_group_eligibility():
    """DeepSpeed issue, Design points: a group is excluded unless its world
    size matches and group rank i is global rank i."""
    W = 4
    cs = [4, 2, 4, 4, 2]
    r2g = [[0, 1, 2, 3], [0, 1, -1, -1], [0, 1, 3, 2], [1, 2, 3, 0], [0, 1, 2, 3]]
    assert list(oracle.group_eligible(W, cs, r2g)) == [1, 0, 0, 0, 0]


# ---------------------------------------------------------------------------
# the probe
# ---------------------------------------------------------------------------

def _golden_lines():
    with open(os.path.join(GOLDEN, "probe_lines.txt")) as f:
        return [ln.rstrip("\n") for ln in f if ln.strip() and not ln.startswith("#")]


def pin_probe_printed_example():
    """The printed probe report: 118 tasks, 52,428,800 elements, rank 0 keeps
    6,553,600, 87.5% discarded, owner path off.  Rebuilt from a bucket of 118
    whole params laid out so that each of the 8 partitions is 6,553,600
    elements of whole params (so every param has exactly one holder)."""
    W, part = 8, 6_553_600
    sizes = []
    for q in range(W):
        k = 15 if q < 6 else 14
        base = part // k
        sz = [base] * k
        sz[-1] += part - base * k
        sizes += sz
    assert len(sizes) == 118 and sum(sizes) == 52_428_800
    flat, ps, off, pids = oracle.partition_ids(sizes, [0, len(sizes)], [W])
    arrival = list(range(len(sizes) - 1, -1, -1))
    t_numel = [sizes[p] for p in arrival]
    pr = oracle.probe(W, t_numel, arrival, [0] * len(arrival), None, off, pids, [W], [1])
    line = oracle.probe_line(0, 3, BF16, pr, 1)
    assert line == _golden_lines()[0], line


def _group_with_cuts(n_params, n_cut, W=8, part=1000):
    """W partitions of `part` elements made of whole params, except that the
    first n_cut partition boundaries each fall inside one (merged) param."""
    total = n_params + n_cut
    counts = [total // W + (1 if q < total % W else 0) for q in range(W)]
    sizes = []
    for q in range(W):
        c = counts[q]
        sz = [part // c] * c
        sz[-1] += part - (part // c) * c
        if 0 < q <= n_cut:
            sizes[-1] += sz[0]
            sz = sz[1:]
        sizes += sz
    return sizes


def pin_ratio_printed_example():
    """The printed init report "291/302": two groups of 8 partitions whose
    boundaries cut 6 and 5 params leave 291 of 302 params with one owner."""
    W = 8
    g0, g1 = _group_with_cuts(151, 6), _group_with_cuts(151, 5)
    sizes, gb = g0 + g1, [0, len(g0), len(g0) + len(g1)]
    flat, ps, off, pids = oracle.partition_ids(sizes, gb, [W, W])
    owner, counts = oracle.owner_map(off, pids, gb, [1, 1])
    assert list(counts[1::2]) == [6, 5]
    line = oracle.ratio_line(int(counts[0::2].sum()), len(sizes))
    assert line == _golden_lines()[1], line


def pin_probe_closed_forms():
    """With the owner path off every rank is written the whole bucket, so
    sum_r discarded_r = (W-1)*reduced - sum_t (|holders_t| - 1) * n_t; with
    one holder per task that is exactly (W-1)/W of W*reduced (87.5% at W=8).
    With the owner path on, an owned task is written only to its owner, who
    keeps it, so it adds nothing to discarded; owner_tasks/elems are 0 when
    the map is empty."""
    rng = random.Random(41)
    for trial in range(60):
        W = rng.choice([2, 4, 8, 16])
        sizes = [rng.randint(0, 300) for _ in range(rng.randint(1, 40))]
        flat, ps, off, pids = oracle.partition_ids(sizes, [0, len(sizes)], [W])
        owner, counts = oracle.owner_map(off, pids, [0, len(sizes)], [1])
        arrival = list(range(len(sizes) - 1, -1, -1))
        t_numel = [sizes[p] for p in arrival]
        holders = [len(pids[off[p]:off[p + 1]]) for p in arrival]
        off_pr = oracle.probe(W, t_numel, arrival, [0] * len(arrival), None, off, pids, [W], [1])
        red = sum(t_numel)
        assert off_pr["reduced_elems"] == red and off_pr["owner_tasks"] == 0
        assert off_pr["owner_elems"] == 0
        extra = sum((h - 1) * n for h, n in zip(holders, t_numel) if h > 0)
        assert int(off_pr["discarded"].sum()) == (W - 1) * red - extra
        if all(h == 1 for h, n in zip(holders, t_numel) if n > 0):
            assert int(off_pr["discarded"].sum()) * W == (W - 1) * W * red
        on_pr = oracle.probe(W, t_numel, arrival, [0] * len(arrival), owner, off, pids, [W], [1])
        own_elems = sum(n for p, n in zip(arrival, t_numel) if owner[p] >= 0)
        assert on_pr["owner_elems"] == own_elems
        assert on_pr["owner_tasks"] == sum(1 for p in arrival if owner[p] >= 0)
        stra = sum((W - h) * n for p, h, n in zip(arrival, holders, t_numel) if owner[p] < 0)
        assert int(on_pr["discarded"].sum()) == stra


def pin_probe_sub_comm_holders():
    """DeepSpeed issue, problem statement (kept and discarded counts) and
    design points (MoE groups): a param of a group on a size-c
    sub-communicator is held, in every block, by the member whose in-block
    index is one of its partitions.  Brute force over the ranks: contiguous
    blocks put rank r at index r mod c, strided blocks (stride W/c) at
    index r div (W/c).  Such tasks are AllReduced, so every rank is written
    every element."""
    rng = random.Random(43)
    for W, c in ((4, 2), (8, 4), (8, 2), (16, 4), (6, 3)):
        for stride in (1, W // c):
            sizes = [rng.randint(0, 50) for _ in range(rng.randint(1, 12))]
            P = len(sizes)
            flat, ps, off, pids = oracle.partition_ids(sizes, [0, P], [c])
            arrival = list(range(P - 1, -1, -1))
            t_numel = [sizes[p] for p in arrival]
            pr = oracle.probe(W, t_numel, arrival, [1] * P, None, off, pids, [W, c], [1, stride])
            kept = [0] * W
            for p, n in zip(arrival, t_numel):
                parts = set(int(q) for q in pids[off[p]:off[p + 1]])
                for r in range(W):
                    idx = r % c if stride == 1 else r // stride
                    if idx in parts:
                        kept[r] += n
            tot = sum(t_numel)
            assert list(pr["kept"]) == kept, (W, c, stride)
            assert list(pr["written"]) == [tot] * W
            assert list(pr["discarded"]) == [tot - k for k in kept]


# ---------------------------------------------------------------------------
# the owner path and the AllReduce path
# ---------------------------------------------------------------------------

def pin_owner_path_equivalences():
    """DeepSpeed issue: the owner path is the same reduction in the same
    operand order, to one destination; with an empty map the flush is the
    AllReduce path bit for bit; rows the owner path does not write keep what
    they held; every holder of a param ends with the sum (copy-out)."""
    rng = random.Random(51)
    for trial in range(20):
        W = rng.choice([2, 4, 8])
        dtype = rng.choice([BF16, F32])
        sizes = [rng.randint(0, 30) for _ in range(rng.randint(2, 12))]
        P = len(sizes)
        flat, ps, off, pids = oracle.partition_ids(sizes, [0, P], [W])
        owner, counts = oracle.owner_map(off, pids, [0, P], [1])
        arrival = list(range(P - 1, -1, -1))
        t_numel = [sizes[p] for p in arrival]
        t_off = np.concatenate([[0], np.cumsum(t_numel)[:-1]]).astype(np.int64)
        T = sum(sizes)
        ld = max(8, T + 3)
        rows = random_bits(rng, dtype, (W, ld), wide=False)
        sentinel = np.full_like(rows, 0x7E7E if dtype == BF16 else 0)
        if dtype == F32:
            sentinel = np.full((W, ld), 1234.5, np.float32)
        ar = sentinel.copy()
        oracle.flush(W, dtype, rows, ar, 0, t_off, t_numel, arrival, [0] * P, None, [W], [1], 1)
        ow = sentinel.copy()
        oracle.flush(W, dtype, rows, ow, 0, t_off, t_numel, arrival, [0] * P, owner, [W], [1], 1)
        empty = sentinel.copy()
        oracle.flush(W, dtype, rows, empty, 0, t_off, t_numel, arrival, [0] * P,
                     np.full(P, -1, np.int32), [W], [1], 1)
        assert np.array_equal(out_bits(dtype, empty), out_bits(dtype, ar))
        for t, p in enumerate(arrival):
            cols = slice(t_off[t], t_off[t] + t_numel[t])
            for r in range(W):
                if owner[p] >= 0 and r != owner[p]:
                    assert np.array_equal(out_bits(dtype, ow[r, cols]), out_bits(dtype, sentinel[r, cols]))
                else:
                    assert np.array_equal(out_bits(dtype, ow[r, cols]), out_bits(dtype, ar[r, cols]))
            for q in pids[off[p]:off[p + 1]]:
                assert np.array_equal(out_bits(dtype, ow[q, cols]), out_bits(dtype, ar[q, cols]))
        # columns outside every task are untouched
        assert np.array_equal(out_bits(dtype, ar[:, T:]), out_bits(dtype, sentinel[:, T:]))


def pin_owner_only_on_dp_comm():
    """DeepSpeed issue, design points (MoE groups): reduce-to-owner applies
    to the data-parallel communicator only.  A task on a sub-communicator
    keeps AllReduce inside each of its blocks even when the owner array has
    an entry for its param, while a data-parallel task with the same entry
    writes that rank's row alone.  Integer-valued inputs keep every sum
    exact, so the expected rows are the brute-force block sums."""
    rng = random.Random(57)
    for W, c, stride in ((4, 2, 1), (4, 2, 2), (8, 4, 2), (8, 2, 1)):
        n = 5
        vals = [[rng.randint(-40, 40) for _ in range(2 * n)] for _ in range(W)]
        rows = np.array(vals, np.float32)
        sent = np.full((W, 2 * n), 999.0, np.float32)
        out = sent.copy()
        owner = np.array([1, 1], np.int32)            # both params name rank 1
        # task 0: param 0 on the data-parallel comm; task 1: param 1 on comm 1
        oracle.flush(W, F32, rows, out, 0, [0, n], [n, n], [0, 1], [0, 1], owner, [W, c],
                     [1, stride], 0)
        for r in range(W):
            want0 = [float(sum(vals[q][j] for q in range(W))) if r == 1 else 999.0
                     for j in range(n)]
            assert list(out[r, :n]) == want0, ("data-parallel task", W, r)
            blk = [r - (r % c) + i for i in range(c)] if stride == 1 else \
                  [r % stride + i * stride for i in range(c)]
            want1 = [float(sum(vals[q][j] for q in blk)) for j in range(n, 2 * n)]
            assert list(out[r, n:]) == want1, ("sub-communicator task", W, c, stride, r)


def pin_zero2_routing():
    """ZeRO-2 owner path ([DS] Follow-up): every element of a data-parallel
    task is written to exactly one row, the rank whose partition holds that
    element (brute force: cumulative sizes, partition = floor(position / S)),
    with the AllReduce value; a param inside one partition matches the ZeRO-1
    owner path; sub-communicator tasks match AllReduce."""
    rng = random.Random(81)
    for trial in range(30):
        W = rng.choice([2, 4, 8])
        dtype = rng.choice([BF16, F32])
        g0 = [rng.choice([0, 1, 3, 7, 20, 33, 64]) for _ in range(rng.randint(2, 14))]
        g1 = [rng.choice([0, 2, 5, 11]) for _ in range(rng.randint(0, 6))]
        sizes = g0 + g1
        P = len(sizes)
        gb = [0, len(g0), P]
        sub = W // 2
        comm_size, comm_stride = [W, sub], [1, 1]
        gcomm = [0, 1]
        parts = [W, sub]
        flat, ps, off, pids = oracle.partition_ids(sizes, gb, parts)
        elig = oracle.group_eligible(W, [W, sub], [list(range(W)), list(range(sub)) + [-1] * (W - sub)])
        owner, _ = oracle.owner_map(off, pids, gb, elig)
        part_size = np.array([ps[0] if p < len(g0) else 0 for p in range(P)], np.int64)
        arrival = list(range(P - 1, -1, -1))
        t_numel = [sizes[p] for p in arrival]
        t_off = np.concatenate([[0], np.cumsum(t_numel)[:-1]]).astype(np.int64) if P else []
        t_comm = [0 if p < len(g0) else 1 for p in arrival]
        T = sum(sizes)
        ld = max(8, -(-T // 8) * 8)
        rows = random_bits(rng, dtype, (W, ld), wide=False)
        sentinel = 0x7E7E if dtype == BF16 else 0x7E7E7E7E
        def blank():
            o = np.zeros_like(rows)
            out_bits(dtype, o)  # view check
            if dtype == BF16:
                o[:] = sentinel
            else:
                o.view(np.uint32)[:] = sentinel
            return o
        z2 = blank()
        oracle.flush_zero2(W, dtype, rows, z2, 0, t_off, t_numel, arrival, t_comm, flat, part_size,
                           comm_size, comm_stride, 1)
        ar = blank()
        oracle.flush(W, dtype, rows, ar, 0, t_off, t_numel, arrival, t_comm, None, comm_size,
                     comm_stride, 1)
        z1 = blank()
        oracle.flush(W, dtype, rows, z1, 0, t_off, t_numel, arrival, t_comm, owner, comm_size,
                     comm_stride, 1)
        zb, ab, ob = out_bits(dtype, z2), out_bits(dtype, ar), out_bits(dtype, z1)
        S = -(-sum(g0) // W) if sum(g0) else 0
        pos0 = np.concatenate([[0], np.cumsum(g0)]) if g0 else [0]
        for t, p in enumerate(arrival):
            cols = range(int(t_off[t]), int(t_off[t]) + sizes[p])
            if p < len(g0):
                for e, j in enumerate(cols):
                    q = (int(pos0[p]) + e) // S
                    written = [r for r in range(W) if zb[r, j] != sentinel]
                    assert written == [q], (trial, p, e, written, q)
                    assert zb[q, j] == ab[q, j]
                if len(pids[off[p]:off[p + 1]]) == 1:
                    assert np.array_equal(zb[:, list(cols)], ob[:, list(cols)])
            else:
                assert np.array_equal(zb[:, list(cols)], ab[:, list(cols)])


def pin_relayout_reduce_scatter():
    """Relayout for a reduce-scatter over the bucket ([DS] alternatives): a
    bijection from the data-parallel columns onto [0, n) whose segment q holds
    exactly the columns of partition q (brute force), in bucket order; the
    reduce-scatter of the relaid bucket gives each rank the ZeRO-2 flush's
    values for its partition, bit for bit."""
    rng = random.Random(91)
    for trial in range(30):
        W = rng.choice([2, 4, 8])
        dtype = rng.choice([BF16, F32])
        g0 = [rng.choice([0, 1, 3, 8, 21, 40, 64]) for _ in range(rng.randint(2, 14))]
        g1 = [rng.choice([0, 2, 5]) for _ in range(rng.randint(0, 4))]
        sizes = g0 + g1
        P = len(sizes)
        gb = [0, len(g0), P]
        sub = W // 2
        flat, ps, off, pids = oracle.partition_ids(sizes, gb, [W, sub])
        part_size = np.array([ps[0] if p < len(g0) else 0 for p in range(P)], np.int64)
        arrival = list(range(P - 1, -1, -1))
        rng.shuffle(arrival) if trial % 3 == 0 else None
        t_numel = [sizes[p] for p in arrival]
        t_off = np.concatenate([[0], np.cumsum(t_numel)[:-1]]).astype(np.int64)
        t_comm = [0 if p < len(g0) else 1 for p in arrival]
        n = sum(sizes)
        dest, seg = oracle.relayout_map(W, t_off, t_numel, arrival, t_comm, flat, part_size, n)
        # brute force: partition of every data-parallel column, stable by column
        S = -(-sum(g0) // W) if sum(g0) else 0
        pos0 = np.concatenate([[0], np.cumsum(g0)]).astype(int)
        part_of = {}
        for t, p in enumerate(arrival):
            if p < len(g0):
                for e in range(sizes[p]):
                    part_of[int(t_off[t]) + e] = (int(pos0[p]) + e) // S
        order = sorted(part_of, key=lambda c: (part_of[c], c))
        want = np.full(n, -1, np.int64)
        for k, c in enumerate(order):
            want[c] = k
        assert np.array_equal(dest, want), trial
        for q in range(W):
            assert seg[q + 1] - seg[q] == sum(1 for c in part_of if part_of[c] == q)
        # values, with the bucket starting at a column other than 0
        col0 = rng.randint(0, 9)
        ld = max(8, -(-(col0 + n) // 8) * 8)
        rows = random_bits(rng, dtype, (W, ld), wide=False)
        relaid = np.zeros_like(rows)
        oracle.relayout_apply(W, dtype, rows, relaid, col0, n, dest)
        shard_ld = max(8, -(-int(max(seg[1:] - seg[:-1], default=0)) // 8) * 8)
        shards = np.zeros((W, shard_ld), rows.dtype)
        oracle.reduce_scatter_v(W, dtype, relaid, shards, seg, 1)
        z2 = np.zeros_like(rows)
        oracle.flush_zero2(W, dtype, rows, z2, col0, t_off, t_numel, arrival, t_comm, flat,
                           part_size, [W, sub], [1, 1], 1)
        sb, zb = out_bits(dtype, shards), out_bits(dtype, z2)
        for c, q in part_of.items():
            assert sb[q, dest[c] - seg[q]] == zb[q, col0 + c], (trial, c, q)


def _scatter_layout(rng, sizes, gap=3):
    """Disjoint offsets for buffers of the given sizes, in shuffled order with
    random gaps; returns (offsets, arena size)."""
    order = list(range(len(sizes)))
    rng.shuffle(order)
    off = [0] * len(sizes)
    pos = rng.randint(0, gap)
    for k in order:
        off[k] = pos
        pos += sizes[k] + rng.randint(0, gap)
    return off, pos + 1


def pin_flush_buffers():
    """Flush straight from per-rank gradient buffers into per-rank grad
    buffers equals copy-in to a bucket, the bucket flush, then copy-out into
    the non-empty buffers ([DS] problem statement), bit for bit, with every
    other element untouched; with one holder per data-parallel task it also
    equals the reduce-to-owner flush followed by the same copy-out ([DS]:
    copy-out unchanged and still correct); in place, holders get the sum and
    every other buffer keeps its gradient."""
    rng = random.Random(83)
    cases = [(4, BF16, 1, [(4, 1), (2, 1), (2, 2)]), (4, F32, 0, [(4, 1), (2, 1), (2, 2)]),
             (8, BF16, 0, [(8, 1), (4, 1), (2, 4)]), (6, F32, 1, [(6, 1), (3, 1), (2, 3)])]
    for W, dtype, pre, comms in cases:
        cs, cst = [c for c, _ in comms], [s for _, s in comms]
        numel = [0, 1, 13, 8, 5, 9, 16, 3]
        n = len(numel)
        t_comm = [rng.randrange(len(comms)) for _ in range(n)]
        t_comm[2], t_comm[3] = 0, 0
        hold = [[rng.random() < 0.4 for _ in range(W)] for _ in range(n)]
        hold[2] = [r == 1 for r in range(W)]          # one owner
        hold[3] = [True] * W                          # every rank
        hold[4] = [False] * W                         # nobody keeps it
        in_off, in_size = _scatter_layout(rng, [numel[t] for t in range(n) for _ in range(W)])
        held = [(t, r) for t in range(n) for r in range(W) if hold[t][r]]
        o_off, out_size = _scatter_layout(rng, [numel[t] for t, _ in held])
        out_off = np.full((n, W), -1, np.int64)
        for (t, r), o in zip(held, o_off):
            out_off[t, r] = o
        in_off = np.array(in_off, np.int64).reshape(n, W)
        arena = random_bits(rng, dtype, (in_size,))
        sent = np.zeros(out_size, arena.dtype)
        if dtype == BF16:
            sent[:] = 0x7E7E
        else:
            sent.view(np.uint32)[:] = 0x7E7E7E7E
        got = oracle.flush_buffers(W, dtype, arena, in_off, sent.copy(), out_off, numel, t_comm, cs,
                                   cst, pre)
        # copy-in, bucket flush, copy-out
        t_off = np.concatenate([[0], np.cumsum(numel)[:-1]]).astype(np.int64)
        M = int(sum(numel))
        slab = np.zeros((W, M), arena.dtype)
        for t in range(n):
            for r in range(W):
                slab[r, t_off[t]:t_off[t] + numel[t]] = arena[in_off[t, r]:in_off[t, r] + numel[t]]
        for owner in (None, [1 if t == 2 else -1 for t in range(n)]):
            bo = np.zeros_like(slab)
            ow = None if owner is None else np.array(owner, np.int32)
            oracle.flush(W, dtype, slab, bo, 0, t_off, numel, list(range(n)), t_comm, ow, cs, cst, pre)
            want = sent.copy()
            for t, r in held:
                o = out_off[t, r]
                want[o:o + numel[t]] = bo[r, t_off[t]:t_off[t] + numel[t]]
            assert np.array_equal(out_bits(dtype, got), out_bits(dtype, want)), (W, dtype, owner)
        # in place: the output buffers are the holders' own gradient buffers
        inplace = arena.copy()
        ip_off = np.where(out_off >= 0, in_off, -1)
        oracle.flush_buffers(W, dtype, inplace, in_off, inplace, ip_off, numel, t_comm, cs, cst, pre)
        want = arena.copy()
        for t, r in held:
            o = in_off[t, r]
            want[o:o + numel[t]] = got[out_off[t, r]:out_off[t, r] + numel[t]]
        assert np.array_equal(out_bits(dtype, inplace), out_bits(dtype, want)), (W, dtype, "in place")


# ---------------------------------------------------------------------------
# ring and recursive-doubling all-gather
# ---------------------------------------------------------------------------

def _ring_table():
    rows = []
    with open(os.path.join(GOLDEN, "ring_allgather_n4.txt")) as f:
        for ln in f:
            if ln.strip() and not ln.startswith("#"):
                parts = ln.split()
                rows.append([[ord(ch) - ord("A") for ch in cell] for cell in parts[1:]])
    return rows


def pin_ring_table():
    """The printed N=4 ring table, cell by cell, from the simulated ring; the
    gathered RING layout; every node receives N-1 chunks of M/N."""
    table = _ring_table()
    order, sends = oracle.ring_ag_schedule(4)
    for step, row in enumerate(table):
        for i in range(4):
            assert list(order[i, :step + 1]) == row[i], (step, i, list(order[i]), row[i])
    recv = np.bincount(sends[:, 2], minlength=4)
    assert list(recv) == [3, 3, 3, 3]
    # the gathered layout follows the table's final row
    W, L = 4, 3
    shards = np.arange(W * L, dtype=np.float32).reshape(W, L)
    out = np.zeros((W, W * L), np.float32)
    oracle.all_gather(W, F32, shards, out, L, 1)
    for i in range(W):
        for p in range(W):
            assert np.array_equal(out[i, p * L:(p + 1) * L], shards[table[-1][i][p]])


def pin_ring_closed_form():
    """Position p of node i holds chunk (i - p) mod N, for N up to 64; per-node
    receive volume is (N-1) chunks, the bandwidth lower bound's (N-1)M/N."""
    for N in range(1, 65):
        order, sends = oracle.ring_ag_schedule(N)
        for i in range(N):
            assert list(order[i]) == [(i - p) % N for p in range(N)], N
        if N > 1:
            assert np.all(np.bincount(sends[:, 2], minlength=N) == N - 1)
            # each step forwards the chunk received in the previous step
            for rec in sends:
                step, src, dst, chunk = rec
                assert dst == (src + 1) % N and chunk == (src - (step - 1)) % N


def pin_rd_table():
    """The printed N=8 recursive-doubling table (pairs, per-step volume,
    holdings); for every N = 2^k the per-step volumes M*2^(j-1)/N sum to
    (N-1)M/N in log2 N steps (the latency lower bound)."""
    partner, recv, held = oracle.rd_ag_schedule(8)
    with open(os.path.join(GOLDEN, "rd_allgather_n8.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    frac = {"M/8": 1, "M/4": 2, "M/2": 4, "M": 8}
    assert len(rows) == len(partner) == 3
    for j, (step, pairs, exch, held_after) in enumerate(rows):
        want_pairs = [tuple(int(x) for x in pr.split(",")) for pr in pairs.strip("()").split(")(")]
        got_pairs = sorted({tuple(sorted((i, int(partner[j, i])))) for i in range(8)})
        assert got_pairs == sorted(want_pairs), (j, got_pairs, want_pairs)
        assert recv[j] == frac[exch] and held[j] == frac[held_after]
    for k in range(0, 7):
        N = 1 << k
        partner, recv, held = oracle.rd_ag_schedule(N)
        assert len(recv) == k == math.ceil(math.log2(N)) if N > 1 else len(recv) == 0
        assert int(recv.sum()) == N - 1
        assert list(recv) == [1 << j for j in range(k)]


def pin_ring_step_replay():
    """RING layout built one step at a time (step mode) equals the full
    gather, and after replaying steps 0..s node i holds the table's row s."""
    W, L = 4, 5
    rng = np.random.default_rng(61)
    shards = rng.standard_normal((W, L)).astype(np.float32)
    full = np.zeros((W, W * L), np.float32)
    oracle.all_gather(W, F32, shards, full, L, 1)
    part = np.full((W, W * L), np.nan, np.float32)
    table = _ring_table()
    for s in range(W):
        oracle.all_gather(W, F32, shards, part, L, 1, s)
        for i in range(W):
            for p in range(s + 1):
                assert np.array_equal(part[i, p * L:(p + 1) * L], shards[table[s][i][p]])
            assert np.all(np.isnan(part[i, (s + 1) * L:]))
    assert np.array_equal(part, full)


def _ag_steps(N, algo):
    """Step count of each schedule: eq:ring-ag (N-1), eq:ag-bidir-ring
    (ceil((N-1)/2)), eq:rd-ag (log2 N)."""
    if algo == oracle.AG_RING:
        return N - 1
    if algo == oracle.AG_BIDIR:
        return math.ceil((N - 1) / 2)
    return int(round(math.log2(N)))


def pin_ag_step_executors():
    """Replaying steps 0..last of every schedule, chunks at their own index,
    gives the rank-order gather on every node, for N up to 16 (recursive
    doubling at powers of two); the step counts are those of eq:ring-ag,
    eq:ag-bidir-ring and eq:rd-ag; every (node, chunk) arrives exactly once
    (the (N-1)M/N receive volume of the bandwidth lower bound); a step reads
    only chunks held before it and never one it writes; ring and bidirectional
    transfers come from a neighbour only; per-step volumes are one chunk
    (ring), at most one per direction (bidirectional) and 2^(j-1) chunks
    (recursive doubling, the printed N = 8 table); ring step s delivers
    position s of the printed N = 4 table; the bidirectional ring's step s is
    that ring rule run in both directions (chunk (i-s) mod N from the left,
    (i+s) mod N from the right, once when the two coincide)."""
    ring4 = _ring_table()
    rd8 = {1: 1, 2: 2, 3: 4}
    rng = np.random.default_rng(67)
    for N in range(1, 17):
        algos = [oracle.AG_RING, oracle.AG_BIDIR]
        if N & (N - 1) == 0:
            algos.append(oracle.AG_RD)
        L = 3
        shards = rng.standard_normal((N, L)).astype(np.float32)
        want = np.zeros((N, N * L), np.float32)
        oracle.all_gather(N, F32, shards, want, L, 0)
        for algo in algos:
            S = _ag_steps(N, algo)
            assert oracle.ag_step_transfers(N, algo, S + 1) is None, (N, algo)
            assert oracle.ag_step_transfers(N, algo, 0) is None, (N, algo)
            held = {(i, i) for i in range(N)}
            got = np.full((N, N * L), np.nan, np.float32)
            oracle.all_gather_step(N, F32, shards, got, L, algo, 0)
            for s in range(1, S + 1):
                tr = oracle.ag_step_transfers(N, algo, s)
                assert tr is not None and len(tr) > 0, (N, algo, s)
                writes = {(d, c) for d, _, c in tr}
                assert len(writes) == len(tr), (N, algo, s, "chunk delivered twice")
                for d, src, c in tr:
                    assert (src, c) in held and (d, c) not in held, (N, algo, s, d, src, c)
                    assert (src, c) not in writes, (N, algo, s, "reads a chunk written in the step")
                    if algo != oracle.AG_RD:
                        assert (d - src) % N in (1, N - 1), (N, algo, s)
                per_node = np.bincount([d for d, _, _ in tr], minlength=N)
                if algo == oracle.AG_RING:
                    assert np.all(per_node == 1), (N, s)
                    for d, src, c in tr:
                        assert src == (d - 1) % N
                        if N == 4:
                            assert c == ring4[s][d][s], (s, d, c)
                elif algo == oracle.AG_BIDIR:
                    assert np.all((per_node >= 1) & (per_node <= 2)), (N, s)
                    for d in range(N):
                        srcs = [src for dd, src, _ in tr if dd == d]
                        assert len(set(srcs)) == len(srcs), (N, s, d)
                    # each direction is the printed ring rule: at step s node d
                    # takes chunk (d - s) mod N from its left neighbour and
                    # (d + s) mod N from its right one; the two coincide only
                    # at the last step of an even N, where the chunk comes once
                    want_tr = {(d, (d - 1) % N, (d - s) % N) for d in range(N)}
                    want_tr |= {(d, (d + 1) % N, (d + s) % N) for d in range(N)
                                if (d + s) % N != (d - s) % N}
                    assert {tuple(x) for x in tr} == want_tr, (N, s)
                else:
                    assert np.all(per_node == 1 << (s - 1)), (N, s)
                    if N == 8:
                        assert per_node[0] == rd8[s]
                held |= writes
                n = oracle.all_gather_step(N, F32, shards, got, L, algo, s)
                assert n == len(tr)
            assert held == {(i, c) for i in range(N) for c in range(N)}, (N, algo)
            assert np.array_equal(got, want), (N, algo)


# ---------------------------------------------------------------------------
# deferred reduction under gradient accumulation
# ---------------------------------------------------------------------------

def _per_microbatch(W, xs, M):
    """Status quo: reduce each micro-batch across replicas, accumulate the
    reduced gradients from a zero start."""
    A = np.zeros((1, M), np.float32)
    for k, x in enumerate(xs):
        g = np.zeros((1, M), np.float32)
        oracle.deferred_reduce(W, x, g, M, 1)
        oracle.accumulate(1, g, A, M, 1 if k == 0 else 0)
    return A


def _deferred(W, xs, M, out_rows=1):
    acc = np.zeros((W, M), np.float32)
    for k, x in enumerate(xs):
        oracle.accumulate(W, x, acc, M, 1 if k == 0 else 0)
    D = np.zeros((out_rows, M), np.float32)
    oracle.deferred_reduce(W, acc, D, M, out_rows)
    return D, acc


def pin_deferred_ga1_identity():
    """GA = 1: deferring changes nothing, bit for bit (signed zeros included,
    since both accumulators start from +0); every output row gets the sum."""
    rng = random.Random(71)
    for W in (1, 2, 4, 5):
        x = random_bits(rng, F32, (W, 40))
        D, _ = _deferred(W, [x], 40, out_rows=W)
        A = _per_microbatch(W, [x], 40)
        for i in range(W):
            assert np.array_equal(D[i].view(np.uint32), A[0].view(np.uint32)), (W, i)


def pin_accumulate_zero_start():
    """The accumulator starts from a zero tree: +0 + x, so a -0 gradient
    starts the accumulator at +0 (IEEE: +0 + -0 = +0 under round to
    nearest); later micro-batches add in fp32."""
    x = np.array([[-0.0, 1.5, -2.0, 3e-45]], np.float32)
    acc = np.full((1, 4), 7.0, np.float32)
    oracle.accumulate(1, x, acc, 4, 1)
    assert list(acc[0].view(np.uint32)) == [0, 0x3FC00000, 0xC0000000, 0x2]
    y = np.array([[-0.0, 2.0 ** -24, 2.0, -3e-45]], np.float32)
    oracle.accumulate(1, y, acc, 4, 0)
    assert list(acc[0].view(np.uint32)) == [0, 0x3FC00000, 0, 0]


def pin_deferred_rank_order():
    """MaxText PR, What: the deferred reduce is one cross-replica sum, read
    here as a fold in replica order 0..W-1 in fp32 that starts from replica
    0's value.  Hand-derived, as for the flush: replicas (2^24, 1, -2^24, 1)
    give 2^24 + 1 -> 2^24 (a tie, to even), then 0, then 1; the reverse
    order gives 2.  Replicas that are all -0 sum to -0 (a start from +0 would
    give +0).  Every output row holds the same sum."""
    acc = np.array([[2.0 ** 24, 3.0, -0.0], [1.0, 5.0, -0.0], [-(2.0 ** 24), -8.0, -0.0],
                    [1.0, 0.5, -0.0]], np.float32)
    for out_rows in (1, 4):
        out = np.full((out_rows, 3), 7.0, np.float32)
        oracle.deferred_reduce(4, acc, out, 3, out_rows)
        # the fold starts from replica 0's value, so replicas all -0 sum to -0
        want = np.tile(np.array([1.0, 0.5, -0.0], np.float32), (out_rows, 1))
        assert np.array_equal(out.view(np.uint32), want.view(np.uint32)), out


def pin_deferred_exact_reassociation():
    """MaxText PR, Results: where the reassociation is exact the two orders
    agree bit for bit.  Values k*2^-20 (|k| < 2^10) keep every partial sum
    exact, so both equal the exact rational total for any K."""
    rng = random.Random(72)
    for W, K in ((4, 1), (4, 4), (4, 8), (3, 5)):
        ks = [[[rng.randint(-1023, 1023) for _ in range(30)] for _ in range(W)] for _ in range(K)]
        xs = [(np.array(k, np.float64) * 2.0 ** -20).astype(np.float32) for k in ks]
        D, _ = _deferred(W, xs, 30)
        A = _per_microbatch(W, xs, 30)
        exact = [float(Fraction(sum(ks[k][r][j] for k in range(K) for r in range(W)), 2 ** 20))
                 for j in range(30)]
        assert np.array_equal(D[0], np.array(exact, np.float32))
        assert np.array_equal(A[0], np.array(exact, np.float32))


def pin_deferred_tolerance():
    """|D - A| <= 5e-5 * sum|x| elementwise, and within the exact bound
    2 * gamma_{WK} * sum|x| (Higham ch. 4)."""
    rng = np.random.default_rng(73)
    for W, K in ((4, 1), (4, 4), (4, 8)):
        xs = [(rng.standard_normal((W, 2000)) * 1e-3).astype(np.float32) for _ in range(K)]
        D, _ = _deferred(W, xs, 2000)
        A = _per_microbatch(W, xs, 2000)
        S = sum(np.abs(x.astype(np.float64)).sum(axis=0) for x in xs)
        err = np.abs(D[0].astype(np.float64) - A[0].astype(np.float64))
        u = 2.0 ** -24
        n = W * K
        assert np.all(err <= 5e-5 * S)
        assert np.all(err <= 2 * (n * u / (1 - n * u)) * S + 1e-45)


def pin_deferred_restore():
    """MaxText PR, Accumulator lifetime: placing a reduced total T onto the
    unreduced accumulator leaves T on one replica and zeros elsewhere, and the
    deferred reduce reproduces T exactly (-0 comes back as +0)."""
    rng = random.Random(74)
    W = 4
    T = random_bits(rng, F32, (1, 50))
    acc = np.zeros((W, 50), np.float32)
    acc[0] = T[0]
    D = np.zeros((1, 50), np.float32)
    oracle.deferred_reduce(W, acc, D, 50, 1)
    want = np.where(T[0] == 0, np.float32(0.0), T[0])
    assert np.array_equal(D[0].view(np.uint32), want.view(np.uint32))


def pin_deferred_round_trip():
    """Mid-step checkpoint: accumulate k1 micro-batches, reduce (save),
    restore onto replica 0, accumulate the rest, reduce: within the
    tolerance of the uninterrupted step."""
    rng = np.random.default_rng(75)
    W, K, M = 4, 8, 500
    xs = [(rng.standard_normal((W, M)) * 1e-3).astype(np.float32) for _ in range(K)]
    D, _ = _deferred(W, xs, M)
    Dsave, acc = _deferred(W, xs[:3], M)
    acc = np.zeros((W, M), np.float32)
    acc[0] = Dsave[0]
    for x in xs[3:]:
        oracle.accumulate(W, x, acc, M, 0)
    D2 = np.zeros((1, M), np.float32)
    oracle.deferred_reduce(W, acc, D2, M, 1)
    S = sum(np.abs(x.astype(np.float64)).sum(axis=0) for x in xs)
    assert np.all(np.abs(D2[0].astype(np.float64) - D[0]) <= 5e-5 * S)


ALL_PINS = [
    pin_bf16_rounding, pin_bf16_rounding_matches_torch, pin_fold_rank_order, pin_fold_exact_sums,
    pin_fold_identical_rows, pin_fold_brute_force, pin_fold_error_bound,
    pin_prediv_non_power_of_two, pin_reduce_scatter_all_gather, pin_ring_reduce_scatter, pin_partition_brute_force,
    pin_owner_rules, pin_group_eligibility, pin_probe_printed_example, pin_ratio_printed_example,
    pin_probe_closed_forms, pin_probe_sub_comm_holders, pin_owner_path_equivalences,
    pin_owner_only_on_dp_comm,
    pin_zero2_routing,
    pin_relayout_reduce_scatter, pin_flush_buffers, pin_ring_table, pin_ring_closed_form,
    pin_rd_table, pin_ring_step_replay, pin_ag_step_executors, pin_deferred_ga1_identity,
    pin_accumulate_zero_start, pin_deferred_rank_order, pin_deferred_exact_reassociation, pin_deferred_tolerance, pin_deferred_restore,
    pin_deferred_round_trip,
]
