"""Synthetic workloads: parameter lists, param groups, communicators and buckets.

Input construction only.  Nothing here reduces, rounds or sums gradient values;
it describes the *shape* of the gradients (which parameters exist, how large
they are, which group and communicator they belong to, and how a ZeRO-1 bucket
is assembled from them).  Both the CPU oracle and the GPU path read these
descriptions.

Sources for the shapes:
  * DeepSpeed issue "DeepCompile ZeRO-1: reduce-to-owner instead of AllReduce",
    problem statement and "Additional context": an 8-rank bf16 flush of a
    402.8M-parameter gradient in buckets of 52,428,800 elements, about 118
    tasks per bucket; one full-parameter task per bucket entry, assembled in
    gradient-arrival order (alternatives section).
  * MaxText PR "Defer the data-parallel gradient all-reduce to update() under
    gradient accumulation", Results: qwen3-0.6b on 4 data replicas.
  * AllGather page, ZeRO Stage 3: reduce-scatter of one layer's gradients and
    all-gather of its weights.

Arrival order is read as the reverse of declaration order (backward produces
gradients last layer first); a parameter larger than the bucket capacity is
flushed alone as a one-task bucket.
"""
from __future__ import annotations

import math
import random
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

DT_BF16 = 0
DT_F32 = 1
DTYPE_NAME = {DT_BF16: "bf16", DT_F32: "f32"}
DTYPE_BYTES = {DT_BF16: 2, DT_F32: 4}


def sigma_scale(sigma: float) -> Tuple[int, int]:
    """(C, E) with C in [2^15, 2^16) so that 37837.23 * C * 2^-E ~= sigma.

    37837.23 is the standard deviation of the generator's Irwin-Hall(4)
    integer (four 16-bit uniforms: sqrt(4 * (65536^2 - 1) / 12)).
    """
    ih_std = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)
    target = sigma / ih_std
    E = math.ceil(math.log2(32768.0 / target))
    C = int(round(target * 2.0 ** E))
    if C >= 65536:
        E -= 1
        C = int(round(target * 2.0 ** E))
    assert 32768 <= C < 65536 and 0 <= E <= 100
    return C, E


@dataclass
class Comm:
    """A communicator over the W simulated ranks.

    size c divides W; block b has members {base_b + i*stride : i < c} with
    base_b = b*c when stride == 1 (contiguous blocks) and base_b = b when
    stride == W/c (strided blocks).  Comm 0 is always the data-parallel comm
    {W, 1}.
    """
    size: int
    stride: int

    def blocks(self, W: int) -> List[List[int]]:
        nb = W // self.size
        out = []
        for b in range(nb):
            base = b * self.size if self.stride == 1 else b
            out.append([base + i * self.stride for i in range(self.size)])
        return out


@dataclass
class Task:
    param: int
    offset: int      # column offset relative to the bucket start
    numel: int
    comm: int


@dataclass
class Bucket:
    col: int         # first slab column of the bucket
    numel: int
    tasks: List[Task]


@dataclass
class FlushWorkload:
    name: str
    W: int
    dtype: int
    sigma: float
    value_seed: int
    numel: List[int]                 # declaration order, group by group
    group_begin: List[int]           # G+1 entries
    group_comm: List[int]            # comm id per group
    comms: List[Comm]
    capacity: int
    pre_div: int
    arrival: List[int] = field(default_factory=list)
    buckets: List[Bucket] = field(default_factory=list)

    @property
    def P(self) -> int:
        return len(self.numel)

    @property
    def G(self) -> int:
        return len(self.group_begin) - 1

    @property
    def total(self) -> int:
        return sum(self.numel)

    @property
    def ld(self) -> int:
        return max(64, round_up(self.total, 64))

    @property
    def scale(self) -> Tuple[int, int]:
        return sigma_scale(self.sigma)

    def group_of(self, p: int) -> int:
        for g in range(self.G):
            if self.group_begin[g] <= p < self.group_begin[g + 1]:
                return g
        raise IndexError(p)

    def group_parts(self) -> List[int]:
        """Partitions per group: W for the DP comm, the comm size otherwise."""
        return [self.comms[c].size for c in self.group_comm]

    def group_rank_to_global(self) -> List[List[int]]:
        """group rank -> global rank, as seen from rank 0's block (padded -1)."""
        out = []
        for c in self.group_comm:
            blk = self.comms[c].blocks(self.W)[0]
            out.append(blk + [-1] * (self.W - len(blk)))
        return out

    def task_comm(self, p: int) -> int:
        return self.group_comm[self.group_of(p)]

    def elem_bytes(self) -> int:
        return DTYPE_BYTES[self.dtype]


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def bucketize(numel: Sequence[int], arrival: Sequence[int], capacity: int,
              comm_of: Sequence[int]) -> List[Bucket]:
    """Greedy packing in arrival order.

    A task that would overflow the open bucket closes it first; a task larger
    than the capacity is flushed alone.  Tasks are packed contiguously inside a
    bucket and buckets follow each other on the slab's columns.
    """
    buckets: List[Bucket] = []
    cur: List[Task] = []
    used = 0
    col = 0

    def close():
        nonlocal cur, used, col
        if cur:
            buckets.append(Bucket(col=col, numel=used, tasks=cur))
            col += used
        cur, used = [], 0

    for p in arrival:
        n = int(numel[p])
        if n > capacity:
            close()
            cur = [Task(param=p, offset=0, numel=n, comm=comm_of[p])]
            used = n
            close()
            continue
        if used + n > capacity:
            close()
        cur.append(Task(param=p, offset=used, numel=n, comm=comm_of[p]))
        used += n
    close()
    return buckets


def finish(w: FlushWorkload, arrival: Optional[Sequence[int]] = None) -> FlushWorkload:
    w.arrival = list(arrival) if arrival is not None else list(range(w.P - 1, -1, -1))
    comm_of = [w.task_comm(p) for p in range(w.P)]
    w.buckets = bucketize(w.numel, w.arrival, w.capacity, comm_of)
    return w


# ---------------------------------------------------------------------------
# The five workloads.
# ---------------------------------------------------------------------------

def tiny_flush(seed_sizes: int = 101, value_seed: int = 1) -> FlushWorkload:
    """W=4 bf16, 16 params with sizes uniform in [1024, 65536], one group of 4
    equal partitions, one bucket holding every task, pre-division on."""
    rng = random.Random(seed_sizes)
    numel = [rng.randint(1024, 65536) for _ in range(16)]
    w = FlushWorkload(name="tiny_flush_w4_bf16", W=4, dtype=DT_BF16, sigma=1e-2,
                      value_seed=value_seed, numel=numel, group_begin=[0, 16],
                      group_comm=[0], comms=[Comm(4, 1)], capacity=sum(numel), pre_div=1)
    return finish(w)


HIDDEN = 1024
EMBED = 151936 * 1024


def param_list(name: str) -> List[int]:
    """A committed parameter-size list (synth/param_lists/<name>.json,
    written once by synth/param_lists/generate.py)."""
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "param_lists", name + ".json")
    with open(path) as f:
        rec = json.load(f)
    numel = [int(n) for n in rec["numel"]]
    assert len(numel) == rec["params"] and sum(numel) == rec["total"], path
    return numel


def owner_flush_w8(value_seed: int = 2, capacity: int = 52_428_800) -> FlushWorkload:
    """W=8 bf16 flush of a 402.8M-element transformer-shaped gradient.

    The committed list owner_flush_w8_402.8M (size seed 102): the embedding
    (151936 x 1024) declared first, then a seeded shuffle of a stratified mix
    of 1024-vectors (78.0%), 1024x1024 (15.2%) and 1024x4096 / 4096x1024
    (6.8%) matrices, the smallest such mix whose total reaches 402.8M.  The
    mix's mean size, 445,395, gives about 118 tasks per 52,428,800-element
    bucket.  One group, 8 equal partitions, pre-division on.
    """
    numel = param_list("owner_flush_w8_402.8M")
    w = FlushWorkload(name="owner_flush_w8_bf16_402.8M", W=8, dtype=DT_BF16, sigma=1e-3,
                      value_seed=value_seed, numel=numel, group_begin=[0, len(numel)],
                      group_comm=[0], comms=[Comm(8, 1)], capacity=capacity, pre_div=1)
    return finish(w)


def owner_flush_w8_layered(value_seed: int = 2, target: int = 402_800_000,
                           capacity: int = 52_428_800) -> FlushWorkload:
    """W=8 bf16 flush of the same 402.8M-element gradient laid out as layers.

    The embedding (151936 x 1024) is declared first, then decoder layers of
    hidden 1024 in declaration order -- input norm (1024), q, k, v, o
    (1024 x 1024 each), post norm (1024), up (1024 x 4096), down
    (4096 x 1024) -- stopping at the first parameter that brings the total to
    `target`, then a final norm (1024).  That is 19 whole layers and a 20th
    cut after its up projection: 161 params, 403,088,384 elements, buckets of
    33/32/32/32/31 tasks plus the embedding alone.  Only 5 params straddle a
    partition boundary (the embedding and four 1024 x 4096 matrices), so
    about 33 tasks per bucket instead of the ~118 of the shuffled mix.  Same
    group, partitions, values and pre-division as the shuffled mix.
    """
    layer = [HIDDEN, HIDDEN * HIDDEN, HIDDEN * HIDDEN, HIDDEN * HIDDEN, HIDDEN * HIDDEN, HIDDEN,
             HIDDEN * 4 * HIDDEN, 4 * HIDDEN * HIDDEN]
    numel = [EMBED]
    total = EMBED
    while total < target:
        for n in layer:
            numel.append(n)
            total += n
            if total >= target:
                break
    numel.append(HIDDEN)
    w = FlushWorkload(name="owner_flush_w8_bf16_402.8M_layered", W=8, dtype=DT_BF16, sigma=1e-3,
                      value_seed=value_seed, numel=numel, group_begin=[0, len(numel)],
                      group_comm=[0], comms=[Comm(8, 1)], capacity=capacity, pre_div=1)
    return finish(w)


def mixed_flush_w16(value_seed: int = 5, capacity: int = 52_428_800,
                    moe_stride: int = 1) -> FlushWorkload:
    """W=16 fp32, the committed list mixed_flush_w16_1.2B (size seed 105):
    lognormal sizes (median 64k, sigma_ln 2, clipped to [1, 2^25]), 2% tiny
    params (uniform 1..64), total exactly 1.2B.  Three groups (contiguous
    thirds by count); group 2 is an MoE expert group reduced over four 4-rank
    sub-communicators (contiguous blocks, or strided with moe_stride != 1)
    and so never gets an owner.  Pre-division off."""
    numel = param_list("mixed_flush_w16_1.2B")
    P = len(numel)
    gb = [0, P // 3, 2 * P // 3, P]
    sub = Comm(4, 1) if moe_stride == 1 else Comm(4, 16 // 4)
    w = FlushWorkload(name="mixed_flush_w16_f32_1.2B", W=16, dtype=DT_F32, sigma=1e-3,
                      value_seed=value_seed, numel=numel, group_begin=gb,
                      group_comm=[0, 0, 1], comms=[Comm(16, 1), sub], capacity=capacity,
                      pre_div=0)
    return finish(w)


def custom_flush(name: str, W: int, dtype: int, numel: Sequence[int], *,
                 group_begin: Optional[Sequence[int]] = None,
                 group_comm: Optional[Sequence[int]] = None,
                 comms: Optional[Sequence[Comm]] = None, capacity: Optional[int] = None,
                 pre_div: int = 1, sigma: float = 1e-2, value_seed: int = 7,
                 arrival: Optional[Sequence[int]] = None) -> FlushWorkload:
    numel = [int(n) for n in numel]
    w = FlushWorkload(name=name, W=W, dtype=dtype, sigma=sigma, value_seed=value_seed,
                      numel=numel,
                      group_begin=list(group_begin) if group_begin else [0, len(numel)],
                      group_comm=list(group_comm) if group_comm else [0],
                      comms=list(comms) if comms else [Comm(W, 1)],
                      capacity=capacity if capacity else max(1, sum(numel)), pre_div=pre_div)
    return finish(w, arrival)


# ---------------------------------------------------------------------------
# Flat trees for the reduce-scatter / all-gather and deferred-reduce workloads.
# ---------------------------------------------------------------------------

def qwen3_0_6b_tree() -> List[int]:
    """qwen3-0.6b parameter sizes in flattening order: per layer input norm,
    q (2048x1024), k, v (1024x1024), o (1024x2048), q/k norms (128), post
    norm, gate and up (3072x1024), down (1024x3072); 28 layers; then the tied
    151936x1024 embedding and the final norm.  596,049,920 elements."""
    layer = [1024, 2048 * 1024, 1024 * 1024, 1024 * 1024, 1024 * 2048, 128, 128, 1024,
             3072 * 1024, 3072 * 1024, 1024 * 3072]
    return layer * 28 + [EMBED, 1024]


def layer_7b_tree() -> List[int]:
    """One 7B-class decoder layer (hidden 4096, MLP 11008): input norm, q, k,
    v, o (4096^2), post norm, gate and up (11008x4096), down (4096x11008).
    202,383,360 elements."""
    h, f = 4096, 11008
    return [h, h * h, h * h, h * h, h * h, h, f * h, f * h, h * f]


@dataclass
class SlabWorkload:
    name: str
    W: int
    dtype: int
    sigma: float
    value_seed: int
    M: int
    K: int = 1          # micro-batches (deferred workload)

    @property
    def scale(self) -> Tuple[int, int]:
        return sigma_scale(self.sigma)

    @property
    def ld(self) -> int:
        return max(64, round_up(self.M, 64))


def deferred_ga_w4(K: int = 8) -> SlabWorkload:
    return SlabWorkload(name=f"deferred_ga_w4_f32_qwen3-0.6b_K{K}", W=4, dtype=DT_F32,
                        sigma=1e-3, value_seed=3, M=sum(qwen3_0_6b_tree()), K=K)


def rs_ag_w8() -> SlabWorkload:
    return SlabWorkload(name="rs_ag_w8_bf16_7b_layer", W=8, dtype=DT_BF16, sigma=1e-2,
                        value_seed=4, M=sum(layer_7b_tree()))


def microbatch_stream(mb: int, W: int, r: int) -> int:
    """Generator stream of rank r's gradient in micro-batch mb."""
    return mb * W + r
