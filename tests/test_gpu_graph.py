"""A flush step recorded as a HIP graph: every replay, with eager work and
synchronizations between replays, matches the eager step bit for bit."""
import numpy as np
import pytest

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


def _workloads():
    rng_sizes = [7, 0, 3000, 65, 12000, 1, 9, 40000, 513, 2048]
    return [
        (wl.tiny_flush(), True, False),
        (wl.custom_flush("g-w8-f32", 8, wl.DT_F32, rng_sizes * 4, capacity=30_000, pre_div=1,
                         value_seed=5), False, False),
        (wl.custom_flush("g-w16-bf16-sub", 16, wl.DT_BF16, rng_sizes * 3, group_begin=[0, 15, 30],
                         group_comm=[0, 1], comms=[wl.Comm(16, 1), wl.Comm(4, 4)], capacity=25_000,
                         pre_div=1, value_seed=6), True, False),
        (wl.tiny_flush(), False, True),
    ]


@pytest.mark.parametrize("planned", [False, True], ids=["searched", "planned"])
@pytest.mark.parametrize("case", range(4))
def test_graph_replays_match_eager(case, planned):
    import torch
    w, owner, zero2 = _workloads()[case]
    U.say("graph", w.name, owner, zero2, "planned" if planned else "")
    ld = w.ld
    x = U.gen_slab(w.dtype, w.W, ld, w.total, w.value_seed, 0, w.scale)
    sent = U.SENTINEL16 if w.dtype == wl.DT_BF16 else U.SENTINEL32
    ex = executor.from_workload(w, reduce_to_owner=owner, zero2=zero2)
    # eager
    y_eager = U.empty_slab(w.dtype, w.W, ld)
    ex.build_owner_map()
    if planned:
        ex.plan()
    for b in range(len(w.buckets)):
        ex.flush(b, x, ld, y_eager, ld)
    torch.cuda.synchronize()
    want = y_eager.cpu()
    # graph on its own output slab
    y = U.empty_slab(w.dtype, w.W, ld)
    g = ex.capture_step(x, ld, y, ld)
    for rep in range(4):
        y.fill_(sent)                       # eager work between replays
        torch.cuda.synchronize()
        assert bool((y == sent).all())
        g.replay()
        if rep % 2:
            torch.cuda.synchronize()
        got = y.cpu()
        assert torch.equal(got, want), f"replay {rep}"
    # the eager path still works after capture
    y2 = U.empty_slab(w.dtype, w.W, ld)
    ex.build_owner_map()
    for b in range(len(w.buckets)):
        ex.flush(b, x, ld, y2, ld)
    torch.cuda.synchronize()
    assert torch.equal(y2.cpu(), want)


@pytest.mark.parametrize("planned", [False, True], ids=["searched", "planned"])
def test_graph_replays_fused_flush(planned):
    """The fused copy-in/copy-out flush recorded as a graph (capture_step with
    fused=True): every replay, with eager fills between, matches the eager
    flush bit for bit."""
    import torch
    W, dtype, pre = 4, wl.DT_BF16, 1
    numel = [100, 5000, 37, 777, 4096, 20_000]
    buckets = [executor.BucketSpec(0, 3100, [(0, 100, 0, 0), (100, 3000, 1, 0)]),
               executor.BucketSpec(3100, 2814, [(0, 2000, 1, 0), (2000, 37, 2, 0), (2037, 777, 3, 0)]),
               executor.BucketSpec(5914, 4096, [(0, 4096, 4, 0)]),
               executor.BucketSpec(10010, 20_000, [(0, 20_000, 5, 0)])]
    ex = executor.Zero1FlushExecutor(W, dtype, numel, [0, 6], [W], [W], [list(range(W))], [(W, 1)],
                                     buckets, pre, reduce_to_owner=True)
    ex.build_owner_map()
    ex.fetch_metadata()
    poff, pos = [], 0
    for n in numel:
        poff.append(pos)
        pos = wl.round_up(pos + n, 64)
    ld = wl.round_up(pos, 64)
    U.say("graph fused", "planned" if planned else "searched", "ld", ld)
    x = U.gen_slab(dtype, W, ld, ld, 81, 0, wl.sigma_scale(1e-2))
    y = U.empty_slab(dtype, W, ld)
    hold = np.zeros((W, len(numel)), bool)
    for b, bk in enumerate(buckets):
        h = ex.holders(b)
        for k, t in enumerate(bk.tasks):
            hold[:, t[2]] |= h[k]
    rows = np.arange(W, dtype=np.int64)[:, None] * ld
    po = np.array(poff, np.int64)[None, :]
    in_addr = (x.data_ptr() + (rows + po) * 2).astype(np.uint64)
    out_addr = np.where(hold, y.data_ptr() + (rows + po) * 2, 0).astype(np.uint64)
    ex.register_buffers(in_addr, out_addr, planned=planned)
    for b in range(len(buckets)):
        ex.flush_buffers(b)
    torch.cuda.synchronize()
    want = y.cpu()
    assert not bool((want == U.SENTINEL16).all())
    g = ex.capture_step(fused=True)
    for rep in range(4):
        y.fill_(U.SENTINEL16)
        torch.cuda.synchronize()
        g.replay()
        if rep % 2:
            torch.cuda.synchronize()
        assert torch.equal(y.cpu(), want), f"replay {rep}"
