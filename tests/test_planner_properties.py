"""Property tests of the three host planners (CPU, no GPU): hypothesis draws
bucket layouts -- sizes from empty to several tiles, any start column, owners
in and out of range, ZeRO-2 partitions, sub-communicator tasks, gaps and
overlapping relayout pieces -- and each planner's records must equal the
brute-force definition of its tile record (the header's definitions, built
from per-column indices in tests/test_abi.py)."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from gradient_reduction_amd import dc
from synth import workloads as wl
from tests.test_abi import _brute_plan, _brute_plan_buffers, _brute_relayout_tiles

SETTINGS = settings(max_examples=400, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
DTYPES = st.sampled_from([wl.DT_BF16, wl.DT_F32])
SIZES = st.one_of(st.integers(0, 20), st.integers(0, 3000), st.sampled_from([512, 1024, 2048, 4096, 9000]))


@st.composite
def flush_layouts(draw):
    W = draw(st.sampled_from([1, 2, 3, 4, 8, 16, 64]))
    dtype = draw(DTYPES)
    sizes = draw(st.lists(SIZES, min_size=1, max_size=30))
    P = len(sizes)
    comms = [(W, 1)]
    divs = [c for c in range(1, W) if W % c == 0]
    if divs and draw(st.booleans()):
        c = draw(st.sampled_from(divs))
        comms.append((c, draw(st.sampled_from([1, W // c]))))
    t_comm = draw(st.lists(st.integers(0, len(comms) - 1), min_size=P, max_size=P))
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)
    tasks = dc.tasks_array([(int(offs[k]), sizes[k], k, t_comm[k]) for k in range(P)])
    mode = draw(st.sampled_from(["allreduce", "owner", "zero2"]))
    owner = flat = psize = None
    if mode == "owner":
        owner = np.array(draw(st.lists(st.integers(-2, W + 1), min_size=P, max_size=P)), np.int32)
    elif mode == "zero2":
        flat = np.array(draw(st.lists(st.integers(0, 40_000), min_size=P, max_size=P)), np.int64)
        psize = np.array(draw(st.lists(st.sampled_from([0, 1, 63, 1000, 4096, 30_000]), min_size=P,
                                       max_size=P)), np.int64)
    col0 = draw(st.integers(0, 5000))
    return W, dtype, col0, int(sum(sizes)), tasks, owner, flat, psize, comms


@SETTINGS
@given(flush_layouts())
def test_plan_flush_equals_definition(layout):
    W, dtype, col0, numel, tasks, owner, flat, psize, comms = layout
    got, roots = dc.dc_plan_flush(W, dtype, col0, numel, tasks, len(tasks), owner, flat, psize,
                                  len(tasks), comms, len(comms))
    want = _brute_plan(W, dtype, col0, numel, tasks, owner, flat, psize)
    assert np.array_equal(got, want)
    assert roots == int(np.sum(want["root"] >= 0))


@st.composite
def buffer_layouts(draw):
    W = draw(st.sampled_from([2, 4, 8, 16]))
    dtype = draw(DTYPES)
    E = 8 if dtype == wl.DT_BF16 else 4
    rows, pos = [], draw(st.integers(0, 40))
    for i in range(draw(st.integers(1, 30))):
        n = draw(SIZES)
        rows.append((pos, n, i, draw(st.sampled_from([0, 0, 1]))))
        pos += n + draw(st.sampled_from([0, 1, 5, 64, 3000]))
        if draw(st.booleans()):
            pos = -(-pos // (4 * E)) * 4 * E
    numel = rows[-1][0] + rows[-1][1] + draw(st.sampled_from([0, 3, 100]))
    return W, dtype, numel, dc.tasks_array(rows), [(W, 1), (W // 2, 2)]


@SETTINGS
@given(buffer_layouts())
def test_plan_flush_buffers_equals_definition(layout):
    W, dtype, numel, tasks, comms = layout
    got = dc.dc_plan_flush_buffers(W, dtype, numel, tasks, len(tasks), comms, len(comms))
    assert np.array_equal(got, _brute_plan_buffers(dtype, numel, tasks))


@st.composite
def relayout_layouts(draw):
    dtype = draw(DTYPES)
    numel = draw(st.integers(0, 20_000))
    dst, pcs = 0, []
    overlap = draw(st.booleans())
    for _ in range(draw(st.integers(0, 12))):
        dst += draw(st.sampled_from([0, 0, 1, 8, 300]))
        ln = draw(st.sampled_from([0, 5, 512, 1024, 3000]))
        src = draw(st.one_of(st.integers(-4, max(numel, 0)), st.sampled_from([0, 8, 512, 1000])))
        pcs.append((src, dst, ln, 0))
        dst += draw(st.sampled_from([0, 100, ln // 2])) if overlap else ln
    pieces = np.array(pcs, dc.PIECE_DTYPE) if pcs else np.zeros(0, dc.PIECE_DTYPE)
    col = draw(st.sampled_from([0, 3, 8, 64, 4096, 4099]))
    return dtype, col, numel, pieces, dst + draw(st.sampled_from([0, 7, 600]))


@SETTINGS
@given(relayout_layouts())
def test_plan_relayout_tiles_equals_definition(layout):
    dtype, col, numel, pieces, out_numel = layout
    got = dc.dc_plan_relayout_tiles(dtype, col, numel, pieces, len(pieces), out_numel)
    assert np.array_equal(got, _brute_relayout_tiles(dtype, col, numel, pieces, out_numel))
