"""The synthetic workloads have the shapes their docstrings state (CPU only).

The flush workloads stand in for the DeepSpeed issue's 8-rank, 402.8M-
parameter bf16 microbenchmark ("Additional context": buckets of 52,428,800
elements, about 118 tasks per bucket) and the mixed-stress flush; the flat
trees for qwen3-0.6b (MaxText PR, Results) and one 7B-class layer (AllGather
page, ZeRO Stage 3).  Partition lists and owners come from the oracle.
"""
import oracle
from synth import workloads as wl


def _owners(w):
    flat, ps, off, pids = oracle.partition_ids(w.numel, w.group_begin, w.group_parts())
    comm_sizes = [w.comms[c].size for c in w.group_comm]
    elig = oracle.group_eligible(w.W, comm_sizes, w.group_rank_to_global())
    owner, counts = oracle.owner_map(off, pids, w.group_begin, elig)
    return off, pids, owner, counts


def _buckets_cover_every_param_once(w):
    seen = sorted(t.param for b in w.buckets for t in b.tasks)
    assert seen == list(range(w.P))
    col = 0
    for b in w.buckets:
        assert b.col == col
        assert b.numel == sum(t.numel for t in b.tasks)
        assert b.numel <= w.capacity or len(b.tasks) == 1
        col += b.numel
    assert col == w.total


def test_headline_shuffled_mix():
    w = wl.owner_flush_w8()
    assert (w.W, w.dtype, w.pre_div, w.capacity) == (8, wl.DT_BF16, 1, 52_428_800)
    assert w.P == 554 and w.total == 403_487_744
    assert w.numel[0] == 151936 * 1024
    assert [len(b.tasks) for b in w.buckets] == [92, 117, 112, 102, 130, 1]
    _buckets_cover_every_param_once(w)
    off, pids, owner, counts = _owners(w)
    assert int((owner >= 0).sum()) == 549
    assert list(pids[off[0]:off[1]]) == [0, 1, 2, 3]       # the embedding straddles 4 partitions


def test_layered_variant():
    """19 decoder layers and a 20th cut after its up projection, the
    embedding first and a final norm last: 161 params, 403,088,384 elements,
    buckets of 33/32/32/32/31 tasks plus the embedding alone, and exactly 5
    straddlers -- the embedding over partitions 0..3 and four 1024x4096
    matrices, each over two neighbouring partitions."""
    w = wl.owner_flush_w8_layered()
    assert (w.W, w.dtype, w.pre_div, w.capacity) == (8, wl.DT_BF16, 1, 52_428_800)
    assert w.P == 161 and w.total == 403_088_384
    assert w.total >= 402_800_000 > w.total - w.numel[-2] - w.numel[-1]
    assert w.numel.count(1024) == 41
    assert w.numel.count(1024 * 1024) == 80
    assert w.numel.count(4096 * 1024) == 39
    assert [len(b.tasks) for b in w.buckets] == [33, 32, 32, 32, 31, 1]
    _buckets_cover_every_param_once(w)
    off, pids, owner, counts = _owners(w)
    straddlers = [p for p in range(w.P) if off[p + 1] - off[p] > 1]
    assert len(straddlers) == 5 and straddlers[0] == 0
    assert list(pids[off[0]:off[1]]) == [0, 1, 2, 3]
    for p in straddlers[1:]:
        assert w.numel[p] == 4096 * 1024
        a, b = pids[off[p]:off[p + 1]]
        assert b == a + 1
    assert int((owner >= 0).sum()) == 156
    assert list(counts) == [156, 5]


def test_mixed_stress():
    w = wl.mixed_flush_w16()
    assert (w.W, w.dtype, w.pre_div) == (16, wl.DT_F32, 0)
    assert w.total == 1_200_000_000 and w.P == 2487
    assert len(w.buckets) == 25
    assert [c.size for c in w.comms] == [16, 4] and w.group_comm == [0, 0, 1]
    _buckets_cover_every_param_once(w)
    off, pids, owner, counts = _owners(w)
    g2 = range(w.group_begin[2], w.group_begin[3])
    assert all(owner[p] == -1 for p in g2)                  # the sub-communicator group


def test_flat_trees():
    q = wl.qwen3_0_6b_tree()
    assert len(q) == 310 and sum(q) == 596_049_920
    assert sum(wl.layer_7b_tree()) == 202_383_360


def test_committed_param_lists_match_their_recipe():
    """The committed size lists are what synth/param_lists/generate.py
    writes from their seeds (the workloads read the files, not the
    generator), and hold what the workloads above pin."""
    from synth.param_lists import generate
    assert generate.main(check=True)
    a = wl.param_list("owner_flush_w8_402.8M")
    b = wl.param_list("mixed_flush_w16_1.2B")
    assert (len(a), sum(a), a[0]) == (554, 403_487_744, 151936 * 1024)
    assert set(a[1:]) == {1024, 1024 * 1024, 4 * 1024 * 1024}
    assert (len(b), sum(b)) == (2487, 1_200_000_000)
    assert 1 <= min(b) and max(b) <= 1 << 25
