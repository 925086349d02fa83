"""Benchmark of the data-parallel gradient-reduction hot path on one MI355X.

Default workload: the W=8 reduce-to-owner bucket flush of a 402.8M-element
bf16 gradient (DeepSpeed issue "DeepCompile ZeRO-1: reduce-to-owner instead
of AllReduce", "Additional context": 8 ranks, 402.8M parameters, buckets of
52,428,800 elements, about 118 tasks per bucket), held as a [8, M] slab in HBM.

One step = the owner map (partition lists + owner map kernels) and the flush
of every bucket, in arrival order.  Metric: algorithmic bytes read + written
per step / step time (GB/s), and the flush kernel against MI355X's 8 TB/s HBM
peak.  Algorithmic bytes of a task of n elements over W ranks, b bytes each:
W*n*b read + (owner ? 1 : W)*n*b written + its 32-byte task record.

Other workloads (--workload): allreduce_w8 and zero2_w8 (the same gradient
through the AllReduce and ZeRO-2 paths), layered_w8 and layered_allreduce_w8
(the same 402.8M gradient declared as whole layers: about 33 tasks per
bucket instead of 118, 5 straddlers), mixed and zero2_mixed (W=16 fp32
1.2B-element flush), deferred (qwen3-0.6b W=4 fp32 gradient accumulation),
rs_ag (7B layer reduce-scatter + all-gather), schedules_w8 (7B layer, ring-
order reduce-scatter and the ring / bidirectional-ring / recursive-doubling
all-gather step executors), relayout_rs_w8 (relayout by destination +
reduce-scatter-v), fused_w8 and fused_mixed (the flush with copy-in and
copy-out fused in, from per-rank gradient buffers into per-rank grad
buffers), tiny (W=4 flush).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flush_bytes(w, owner, psize=None, tiles=None):
    """Algorithmic bytes of every flush launch of workload w (ZeRO-2 when
    psize, the per-param partition size, is given): every row read, the rows
    written, 32 bytes per task record and, for a planned flush (tiles: the
    tile count of each bucket), 16 bytes per tile record."""
    b = w.elem_bytes()
    per = []
    for i, bk in enumerate(w.buckets):
        tot = 16 * int(tiles[i]) if tiles is not None else 0
        for t in bk.tasks:
            if psize is not None:
                one = t.comm == 0 and psize[t.param] > 0
            else:
                one = owner is not None and t.comm == 0 and owner[t.param] >= 0
            tot += w.W * t.numel * b + (1 if one else w.W) * t.numel * b + 32
        per.append(tot)
    return per


def owner_map_bytes(w):
    P, G = w.P, w.G
    pids = P + sum(p - 1 for p in w.group_parts())
    # numel read twice, offsets and CSR written, CSR read, owner and counts written
    return 16 * P + 8 * P + 8 * G + 4 * (P + 1) + 4 * pids + 4 * (P + 1) + 4 * pids + 4 * P + 8 * G


class Timer:
    """HIP events on the stream the kernels are launched on (torch's current
    stream: the library enqueues on the stream it is given)."""

    def __init__(self, torch, n):
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]
        # torch creates the HIP event at its first record(); do that now, not
        # inside the timed loop, where creating it can stall the host
        for a, b in self.ev:
            a.record()
            b.record()

    def ms(self):
        return [a.elapsed_time(b) for a, b in self.ev]


def run_timed(torch, args, step, n_events):
    """args.warmup untimed steps, then args.steps timed ones bracketed by a
    synchronize on both sides: the step time.  Then args.steps more with HIP
    events around every launch, for the per-launch kernel times (an event
    record is a packet of its own on the stream, so these steps run a little
    longer and are not the step time).  Python's garbage collector is off in
    both loops so a collection cannot stall the host mid-step.  Returns
    (ms per step, [steps, n_events] launch ms)."""
    import gc
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timers = [Timer(torch, n_events) for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    t1.record()
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    try:
        t0.record()
        for _ in range(args.steps):
            step()
        t1.record()
        torch.cuda.synchronize()
        for k in range(args.steps):
            step(timers[k])
        torch.cuda.synchronize()
    finally:
        gc.enable()
    return t0.elapsed_time(t1) / args.steps, np.array([tm.ms() for tm in timers])


def bench_flush(args, w, reduce_to_owner=True, zero2=False):
    import torch
    import synth
    from gradient_reduction_amd import executor

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    ld = w.ld
    dt = torch.int16 if w.dtype == 0 else torch.int32
    log(f"[bench] {w.name}: W={w.W} elements={w.total} buckets={len(w.buckets)} "
        f"tasks={[len(b.tasks) for b in w.buckets]} slab={w.W * ld * w.elem_bytes() / 1e9:.2f} GB")
    x = torch.empty((w.W, ld), dtype=dt, device=dev)
    synth.fill_slab_device(w.dtype, w.value_seed, 0, w.scale, w.W, ld, w.total, x.data_ptr(),
                           stream.cuda_stream)
    y = torch.zeros((w.W, ld), dtype=dt, device=dev)
    ex = executor.from_workload(w, reduce_to_owner=reduce_to_owner, log=log, zero2=zero2,
                                reduce_probe=args.probe)
    ex.build_owner_map()
    ex.fetch_metadata()
    log("[bench] " + ex.ratio_line())
    if not zero2:
        for b in range(min(len(w.buckets), 3)):
            log("[bench] " + ex.probe_line(b, b))
    owner = ex.h_owner if reduce_to_owner else None
    tiles = None
    if not args.searched:
        ex.plan()
        tiles = np.diff(ex.tile_begin)
        log(f"[bench] flush plans: {tiles.tolist()} tiles per bucket")
    per_launch = flush_bytes(w, owner, ex.h_psize if zero2 else None, tiles)
    step_bytes = sum(per_launch) + owner_map_bytes(w)
    nb = len(w.buckets)

    def step(timer=None):
        if timer is not None:
            timer.ev[nb][0].record()
        ex.build_owner_map()
        if timer is not None:
            timer.ev[nb][1].record()
        for b in range(nb):
            if timer is not None:
                timer.ev[b][0].record()
            ex.flush(b, x, ld, y, ld)
            if timer is not None:
                timer.ev[b][1].record()

    ms_step, kern_all = run_timed(torch, args, step, nb + 1)
    kern, owner_map_ms = kern_all[:, :nb], kern_all[:, nb]    # [steps, buckets], [steps]
    avg_launch_ms = float(kern.mean())
    flush_gbs = sum(per_launch) / (kern.sum(axis=1).mean() / 1e3) / 1e9
    flush_gbs_median = sum(per_launch) / (np.median(kern.sum(axis=1)) / 1e3) / 1e9
    value = step_bytes / (ms_step / 1e3) / 1e9
    log(f"[bench] step {ms_step:.3f} ms, {value:.1f} GB/s; flush kernels {kern.sum(axis=1).mean():.3f} ms "
        f"({flush_gbs:.1f} GB/s); per bucket ms {np.round(kern.mean(axis=0), 4).tolist()}")
    ceiling = access_mix_ceiling(w, owner, x, y, ld, ex.h_psize if zero2 else None)
    roofline = {"bound": "hbm", "achieved": round(flush_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(flush_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile(args.workload, w.name),
                "kernel": "k_flush", "launch_ms_avg": round(avg_launch_ms, 4),
                "bytes_per_launch_avg": int(np.mean(per_launch)),
                "bytes_per_launch": [int(b) for b in per_launch]}
    if ceiling is not None:
        roofline["access_mix_ceiling_gbs"] = round(ceiling, 1)
        roofline["frac_of_access_mix_ceiling"] = round(flush_gbs / ceiling, 4)
    extra = {"per_bucket_gbs": [round(b / (m / 1e3) / 1e9, 1) for b, m in zip(per_launch, kern.mean(axis=0))],
             "flush_gbs_median_step": round(flush_gbs_median, 1),
             "owner_map_us": round(float(owner_map_ms.mean()) * 1e3, 2),
             "graph_ms_per_step": round(graph_step_ms(torch, args, ex.capture_step(x, ld, y, ld)), 4)}
    log(f"[bench] the same step replayed as one HIP graph: {extra['graph_ms_per_step']:.4f} ms")
    del x, y
    torch.cuda.empty_cache()
    return ms_step, value, step_bytes, roofline, extra


def graph_step_ms(torch, args, g):
    """Average time of one replay of a captured step (same warm-up and step
    counts as the eager timing)."""
    for _ in range(max(args.warmup, 1)):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / args.steps


def stream_rows_gbs(src, src_ldv, rows_read, dst, dst_ldv, rows_written, nvec):
    """GB/s of dc_stream_rows (xor only) reading rows_read rows and writing
    rows_written rows of nvec 16-byte vectors: 3 untimed launches, then the
    average of 10."""
    import torch
    from gradient_reduction_amd import dc

    def run():
        dc.dc_stream_rows(src, src_ldv, rows_read, dst, dst_ldv, rows_written, nvec)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        run()
    e1.record()
    torch.cuda.synchronize()
    return nvec * 16 * (rows_read + rows_written) / (e0.elapsed_time(e1) / 10 / 1e3) / 1e9


def add_mix_ceiling(roofline, ceiling, what):
    roofline["access_mix_ceiling_gbs"] = round(ceiling, 1)
    roofline["frac_of_access_mix_ceiling"] = round(roofline["achieved"] / ceiling, 4)
    log(f"[bench] access-mix reference ({what}): {ceiling:.1f} GB/s; the kernel reaches "
        f"{roofline['frac_of_access_mix_ceiling']:.3f} of it")


def access_mix_ceiling(w, owner, x, y, ld, psize=None, split=None):
    """Bandwidth the memory system gives the flush's own access mix: W rows
    read and one row written (owned tasks) or W rows written (AllReduce
    tasks), measured with dc_stream_rows (xor only) at the bucket size and
    blended by the step's bytes (split = (one-row bytes, W-row bytes) when
    given).  None when W has no reference kernel."""
    import torch
    from gradient_reduction_amd import dc
    if w.W not in (4, 8, 16):
        return None
    E = 16 // w.elem_bytes()
    nvec = min(w.capacity, w.total) // E
    ldv = ld // E
    rates = {nw: stream_rows_gbs(x, ldv, w.W, y, ldv, nw, nvec) for nw in (1, w.W)}
    b = w.elem_bytes()
    own = ar = 0
    for bk in w.buckets:
        for t in bk.tasks:
            if split is not None:
                break
            if psize is not None:
                one = t.comm == 0 and psize[t.param] > 0
            else:
                one = owner is not None and t.comm == 0 and owner[t.param] >= 0
            if one:
                own += (w.W + 1) * t.numel * b
            else:
                ar += 2 * w.W * t.numel * b
    if split is not None:
        own, ar = split
    ceiling = (own + ar) / (own / rates[1] + ar / rates[w.W])
    log(f"[bench] access-mix reference: read {w.W} write 1 {rates[1]:.1f} GB/s, read {w.W} "
        f"write {w.W} {rates[w.W]:.1f} GB/s; blended for this step {ceiling:.1f} GB/s")
    return ceiling


def bench_flush_buffers(args, w):
    """The flush with copy-in and copy-out fused in: each rank's gradient of
    every param in a per-rank arena (params at 128-byte aligned positions, as
    separate allocations would be), grad buffers of the same layout for the
    ranks that keep one, one dc_flush_bucket_buffers launch per bucket."""
    import torch
    import synth
    from gradient_reduction_amd import executor
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    eb = w.elem_bytes()
    dt = torch.int16 if w.dtype == 0 else torch.int32
    ex = executor.from_workload(w, reduce_to_owner=True, log=log)
    ex.build_owner_map()
    ex.fetch_metadata()
    # every param is one task here, so its slab columns are contiguous
    pcol = np.full(w.P, -1, np.int64)
    for bk in w.buckets:
        for t in bk.tasks:
            assert pcol[t.param] < 0, "a param split over tasks"
            pcol[t.param] = bk.col + t.offset
    pad = 128 // eb
    poff = np.zeros(w.P, np.int64)
    pos = 0
    for p in range(w.P):
        poff[p] = pos
        pos = -(-(pos + w.numel[p]) // pad) * pad
    ld = -(-max(pos, 1) // 64) * 64
    log(f"[bench] {w.name}: fused copy-in/out flush, arenas [{w.W}, {ld}] "
        f"({2 * w.W * ld * eb / 1e9:.2f} GB in + out)")
    x = torch.empty((w.W, ld), dtype=dt, device=dev)
    for p in range(w.P):
        if w.numel[p]:
            synth.fill_slab_device(w.dtype, w.value_seed, 0, w.scale, w.W, ld, w.numel[p],
                                   x.data_ptr() + int(poff[p]) * eb, stream.cuda_stream,
                                   col0=int(pcol[p]))
    y = torch.zeros((w.W, ld), dtype=dt, device=dev)
    hold = np.zeros((w.W, w.P), bool)
    nb = len(w.buckets)
    per_launch, one_b, many_b, unfused = [], 0, 0, 0
    for b, bk in enumerate(w.buckets):
        h = ex.holders(b)
        tot = 0
        for k, t in enumerate(bk.tasks):
            hold[:, t.param] |= h[k]
            nh = int(h[k].sum())
            tot += w.W * t.numel * eb + nh * t.numel * eb + 32 + 16 * w.W
            if nh <= 1:
                one_b += (w.W + 1) * t.numel * eb
            else:
                many_b += (w.W + nh) * t.numel * eb
            rows = 1 if (t.comm == 0 and ex.h_owner[t.param] >= 0) else w.W
            # copy-in (read + write W rows), flush (read W, write `rows`), copy-out (holders)
            unfused += (2 * w.W + w.W + rows + 2 * nh) * t.numel * eb + 32
        per_launch.append(tot)
    rows_i = np.arange(w.W, dtype=np.int64)[:, None] * ld
    in_addr = (x.data_ptr() + (rows_i + poff[None, :]) * eb).astype(np.uint64)
    out_addr = np.where(hold, y.data_ptr() + (rows_i + poff[None, :]) * eb, 0).astype(np.uint64)
    ex.register_buffers(in_addr, out_addr, planned=not args.searched)
    if not args.searched:
        # 16 bytes per tile record read
        per_launch = [pl + 16 * int(ex.buf_tile_begin[i + 1] - ex.buf_tile_begin[i])
                      for i, pl in enumerate(per_launch)]
    step_bytes = sum(per_launch) + owner_map_bytes(w)

    def step(timer=None):
        if timer is not None:
            timer.ev[nb][0].record()
        ex.build_owner_map()
        if timer is not None:
            timer.ev[nb][1].record()
        for b in range(nb):
            if timer is not None:
                timer.ev[b][0].record()
            ex.flush_buffers(b)
            if timer is not None:
                timer.ev[b][1].record()

    ms_step, kern_all = run_timed(torch, args, step, nb + 1)
    kern, owner_map_ms = kern_all[:, :nb], kern_all[:, nb]
    gbs = sum(per_launch) / (kern.sum(axis=1).mean() / 1e3) / 1e9
    gbs_median = sum(per_launch) / (np.median(kern.sum(axis=1)) / 1e3) / 1e9
    value = step_bytes / (ms_step / 1e3) / 1e9
    log(f"[bench] step {ms_step:.3f} ms, {value:.1f} GB/s; fused flush kernels "
        f"{kern.sum(axis=1).mean():.3f} ms ({gbs:.1f} GB/s); per bucket ms "
        f"{np.round(kern.mean(axis=0), 4).tolist()}")
    ceiling = access_mix_ceiling(w, None, x, y, ld, split=(one_b, many_b))
    roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile(args.workload, w.name),
                "kernel": "k_flush_buffers", "launch_ms_avg": round(float(kern.mean()), 4),
                "bytes_per_launch_avg": int(np.mean(per_launch)),
                "bytes_per_launch": [int(b) for b in per_launch]}
    if ceiling is not None:
        roofline["access_mix_ceiling_gbs"] = round(ceiling, 1)
        roofline["frac_of_access_mix_ceiling"] = round(gbs / ceiling, 4)
    extra = {"per_bucket_gbs": [round(b / (m / 1e3) / 1e9, 1) for b, m in zip(per_launch, kern.mean(axis=0))],
             "flush_gbs_median_step": round(gbs_median, 1),
             "owner_map_us": round(float(owner_map_ms.mean()) * 1e3, 2),
             "fused_bytes_per_step": int(sum(per_launch)),
             "unfused_bytes_per_step": int(unfused),
             "bytes_saved_frac": round(1 - sum(per_launch) / unfused, 4)}
    del x, y
    torch.cuda.empty_cache()
    return ms_step, value, step_bytes, roofline, extra


# Counter summaries behind `traffic`: bench workload -> (profile stem, source
# file of its dominant kernel).  A summary counts only while the kernel's
# source and the shared device header still hash to what they were when the
# counters were taken.
TRAFFIC_PROFILES = {
    "owner_w8": ("flush_w8_402m", "flush.hip"),
    "allreduce_w8": ("flush_allreduce_w8_402m", "flush.hip"),
    "zero2_w8": ("flush_zero2_w8_402m", "flush.hip"),
    "layered_w8": ("flush_w8_402m_layered", "flush.hip"),
    "layered_allreduce_w8": ("flush_allreduce_w8_402m_layered", "flush.hip"),
    "mixed": ("flush_w16_1200m", "flush.hip"),
    "zero2_mixed": ("flush_zero2_w16_1200m", "flush.hip"),
    "fused_w8": ("flush_buffers_w8_402m", "flush_buffers.hip"),
    "fused_mixed": ("flush_buffers_w16_1200m", "flush_buffers.hip"),
    "relayout_rs_w8": ("relayout_rs_w8_402m", "slab_ops.hip"),
    "deferred": ("deferred_qwen3_k8", "slab_ops.hip"),
    "deferred_fused": ("deferred_qwen3_k8_fused", "slab_ops.hip"),
    "rs_ag": ("rs_ag_w8_202m", "slab_ops.hip"),
    "schedules_w8": ("schedules_w8_202m", "slab_ops.hip"),
}


def kernel_source_sha256(source):
    import hashlib
    h = hashlib.sha256()
    for name in (source, "device_common.h", "internal.h"):
        with open(os.path.join(ROOT, "gradient_reduction_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_profile(key, workload, config=None):
    """Measured HBM bytes per launch of the dominant kernel from the committed
    counter summary of bench workload `key`, if it was taken on the current
    kernel source, for the same workload (and config); else None."""
    if key not in TRAFFIC_PROFILES:
        return None
    stem, source = TRAFFIC_PROFILES[key]
    path = os.path.join(ROOT, "profiles", stem + "_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != kernel_source_sha256(source):
        return None
    if rec.get("workload") != workload or rec.get("config", {}) != (config or {}):
        return None
    return rec.get("hbm_bytes_per_launch_avg")


def host_threads():
    """Threads for the all-cores oracle run: the CPUs this process may run on,
    at most 16 (a one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def column_blocks(bk, nthreads, block=1 << 18):
    """Split a bucket's tasks into column blocks of the same param and comm,
    dealt to nthreads lists round-robin (a static schedule).  Every column of
    the oracle's flush is folded on its own, so the split changes no output."""
    lists = [([], [], [], []) for _ in range(nthreads)]
    k = 0
    for t in bk.tasks:
        for o in range(0, t.numel, block):
            dst = lists[k % nthreads]
            dst[0].append(t.offset + o)
            dst[1].append(min(block, t.numel - o))
            dst[2].append(t.param)
            dst[3].append(t.comm)
            k += 1
    return [x for x in lists if x[0]]


def cpu_baseline_flush(w, reduce_to_owner=True, max_buckets=2):
    """The oracle on the first buckets of the same workload (host inputs from
    the same generator; generation untimed), timed twice: on one thread (the
    reported baseline), and on all of the host's threads with each bucket's
    columns split into blocks (the oracle's C calls release the GIL).  The two
    outputs must be identical."""
    import concurrent.futures
    import oracle
    import synth
    flat, ps, off, pids = oracle.partition_ids(w.numel, w.group_begin, w.group_parts())
    comm_sizes = [w.comms[c].size for c in w.group_comm]
    elig = oracle.group_eligible(w.W, comm_sizes, w.group_rank_to_global())
    owner, _ = oracle.owner_map(off, pids, w.group_begin, elig)
    own = owner if reduce_to_owner else None
    per = flush_bytes(w, own)
    csize = [c.size for c in w.comms]
    cstride = [c.stride for c in w.comms]
    nthreads = host_threads()
    used = list(range(min(max_buckets, len(w.buckets))))
    nbytes = sum(per[b] for b in used)

    def run(rows, out, tasks):
        oracle.flush(w.W, w.dtype, rows, out, 0, tasks[0], tasks[1], tasks[2], tasks[3], own,
                     csize, cstride, w.pre_div)

    secs = psecs = 0.0
    same = True
    with concurrent.futures.ThreadPoolExecutor(nthreads) as pool:
        for b in used:
            bk = w.buckets[b]
            n = bk.numel
            ld = -(-n // 8) * 8
            rows = np.zeros((w.W, ld), synth.np_dtype(w.dtype))
            for r in range(w.W):
                rows[r, :n] = synth.fill_row(w.dtype, w.value_seed, r, w.scale, bk.col, n)
            if w.dtype == 1:
                rows = rows.view(np.float32)
            whole = ([t_.offset for t_ in bk.tasks], [t_.numel for t_ in bk.tasks],
                     [t_.param for t_ in bk.tasks], [t_.comm for t_ in bk.tasks])
            out1 = np.zeros_like(rows)
            t = time.perf_counter()
            run(rows, out1, whole)
            secs += time.perf_counter() - t
            outn = np.zeros_like(rows)
            parts = column_blocks(bk, nthreads)
            t = time.perf_counter()
            list(pool.map(lambda tl: run(rows, outn, tl), parts))
            psecs += time.perf_counter() - t
            same = same and np.array_equal(out1.view(np.uint8), outn.view(np.uint8))
            del rows, out1, outn
    log(f"[bench] cpu oracle: {nbytes / 1e9:.2f} GB in {secs:.2f} s on 1 thread, {psecs:.2f} s "
        f"on {nthreads} threads (outputs identical: {same})")
    sample = (f"buckets {used} of {len(w.buckets)} ({sum(w.buckets[b].numel for b in used)} columns, "
              f"{sum(len(w.buckets[b].tasks) for b in used)} tasks), oracle.c single thread, "
              f"{nbytes} algorithmic bytes, {secs:.2f} s")
    base = {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": sample}
    allc = {"value": round(nbytes / psecs / 1e9, 4), "unit": "GB/s", "threads": nthreads,
            "host_cpus": os.cpu_count(), "seconds": round(psecs, 3),
            "outputs_identical_to_one_thread": bool(same)}
    return base, allc


def bench_deferred(args):
    import torch
    import synth
    from gradient_reduction_amd import dc
    from synth import workloads as wl
    w = wl.deferred_ga_w4(args.ga)
    W, M, ld = w.W, w.M, w.ld
    dev = torch.device("cuda:0")
    xs = torch.empty((args.ga, W, ld), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    for k in range(args.ga):
        synth.fill_slab_device(1, w.value_seed, wl.microbatch_stream(k, W, 0), w.scale, W, ld, M,
                               xs[k].data_ptr(), s)
    acc = torch.empty((W, ld), dtype=torch.float32, device=dev)
    out = torch.empty((W, ld), dtype=torch.float32, device=dev)
    fused = args.fused
    n_acc = args.ga - 1 if fused else args.ga
    acc_b = [(2 if k else 1) * W * M * 4 + W * M * 4 for k in range(n_acc)]
    # fused last step: x (and acc unless K = 1) read, W result rows written
    red_b = ((W * M * 4 if args.ga > 1 else 0) + W * M * 4 + W * M * 4) if fused else W * M * 4 + W * M * 4
    step_bytes = sum(acc_b) + red_b
    n = n_acc + 1

    def step(tm=None):
        for k in range(n_acc):
            if tm: tm.ev[k][0].record()
            dc.dc_accumulate(W, xs[k], ld, acc, ld, M, 1 if k == 0 else 0)
            if tm: tm.ev[k][1].record()
        if tm: tm.ev[n_acc][0].record()
        if fused:
            dc.dc_accumulate_reduce(W, xs[args.ga - 1], ld, acc, ld, 1 if args.ga == 1 else 0, 0,
                                    out, ld, W, M)
        else:
            dc.dc_deferred_reduce(W, acc, ld, out, ld, M, W)
        if tm: tm.ev[n_acc][1].record()

    ms_step, kern_all = run_timed(torch, args, step, n)
    kern = kern_all.mean(axis=0)
    red_gbs = red_b / (kern[-1] / 1e3) / 1e9
    acc_gbs = sum(acc_b) / (kern[:-1].sum() / 1e3) / 1e9 if n_acc else 0.0
    log(f"[bench] deferred K={args.ga}: step {ms_step:.3f} ms; accumulate {acc_gbs:.1f} GB/s; "
        f"reduce {red_gbs:.1f} GB/s ({kern[-1]:.3f} ms)")
    roofline = {"bound": "hbm", "achieved": round(red_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(red_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile("deferred_fused" if fused else "deferred", w.name,
                                                {"ga": args.ga}),
                "kernel": "k_accum_reduce" if fused else "k_deferred",
                "launch_ms_avg": round(float(kern[-1]), 4),
                "bytes_per_launch_avg": red_b, "bytes_per_launch": [red_b]}
    if not fused and W in (4, 8, 16):
        add_mix_ceiling(roofline, stream_rows_gbs(acc, ld // 4, W, out, ld // 4, W, M // 4),
                        f"read {W} rows, write {W}")
    extra = {"accumulate_gbs": round(acc_gbs, 1)}

    # The pages' status quo beside it: every micro-batch reduced across the
    # replicas, the reduced gradients accumulated (one row).  Timed on its own.
    g = torch.empty((1, ld), dtype=torch.float32, device=dev)
    A = torch.empty((1, ld), dtype=torch.float32, device=dev)

    def quo():
        for k in range(args.ga):
            dc.dc_deferred_reduce(W, xs[k], ld, g, ld, M, 1)
            dc.dc_accumulate(1, g, ld, A, ld, M, 1 if k == 0 else 0)

    quo()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        quo()
    e1.record()
    torch.cuda.synchronize()
    extra["status_quo_ms_per_step"] = round(e0.elapsed_time(e1) / args.steps, 4)
    # numerics of the deferred sum D against the per-micro-batch sum A: the
    # 5e-5 * sum|x| gate, the normwise difference and the largest relative
    # difference where |A| > 1e-3 max|A|
    step()
    torch.cuda.synchronize()
    d, a = out[0, :M].double(), A[0, :M].double()
    diff = (d - a).abs()
    sabs = torch.zeros(M, dtype=torch.float64, device=dev)
    for k in range(args.ga):
        sabs += xs[k, :, :M].abs().sum(dim=0).double()
    big = a.abs() > 1e-3 * a.abs().max()
    extra["deferred_vs_per_microbatch"] = {
        "max_diff_over_gate": float((diff / (5e-5 * sabs).clamp_min(1e-300)).max()),
        "normwise": float(diff.norm() / a.norm()),
        "max_rel_where_abs_gt_1e-3_max": float((diff[big] / a.abs()[big]).max()),
        "bit_identical_frac": round(float((diff == 0).double().mean()), 6)}
    log(f"[bench] status quo (reduce every micro-batch, then accumulate): "
        f"{extra['status_quo_ms_per_step']:.3f} ms; D vs A: {extra['deferred_vs_per_microbatch']}")
    del d, a, diff, sabs, big
    return w.name, ms_step, step_bytes / (ms_step / 1e3) / 1e9, roofline, extra, "f32"


def bench_rs_ag(args):
    import torch
    import synth
    from gradient_reduction_amd import dc
    from synth import workloads as wl
    w = wl.rs_ag_w8()
    W, M, L = w.W, w.M, w.M // w.W
    dev = torch.device("cuda:0")
    x = torch.empty((W, w.ld), dtype=torch.int16, device=dev)
    synth.fill_slab_device(0, w.value_seed, 0, w.scale, W, w.ld, M, x.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    ld_sh = wl.round_up(L, 64)
    sh = torch.empty((W, ld_sh), dtype=torch.int16, device=dev)
    out = torch.empty((W, w.ld), dtype=torch.int16, device=dev)
    rs_b = W * M * 2 + M * 2
    ag_b = M * 2 + W * M * 2

    def step(tm=None):
        if tm: tm.ev[0][0].record()
        dc.dc_reduce_scatter(W, 0, x, w.ld, sh, ld_sh, M, 0)
        if tm: tm.ev[0][1].record(); tm.ev[1][0].record()
        dc.dc_all_gather(W, 0, sh, ld_sh, out, w.ld, L, dc.DC_ORDER_RANK, -1)
        if tm: tm.ev[1][1].record(); tm.ev[2][0].record()
        dc.dc_all_gather(W, 0, sh, ld_sh, out, w.ld, L, dc.DC_ORDER_RING, -1)
        if tm: tm.ev[2][1].record()

    ms_step, kern_all = run_timed(torch, args, step, 3)
    kern = kern_all.mean(axis=0)
    gbs = [rs_b / (kern[0] / 1e3) / 1e9, ag_b / (kern[1] / 1e3) / 1e9, ag_b / (kern[2] / 1e3) / 1e9]
    log(f"[bench] rs {gbs[0]:.1f} GB/s, ag rank {gbs[1]:.1f} GB/s, ag ring {gbs[2]:.1f} GB/s")
    roofline = {"bound": "hbm", "achieved": round(gbs[0], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs[0] / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile("rs_ag", w.name), "kernel": "k_rs_vec",
                "launch_ms_avg": round(float(kern[0]), 4), "bytes_per_launch_avg": rs_b,
                "bytes_per_launch": [rs_b]}
    add_mix_ceiling(roofline, stream_rows_gbs(x, w.ld // 8, W, out, w.ld // 8, 1, M // 8),
                    f"read {W} rows, write 1")
    extra = {"all_gather_rank_gbs": round(gbs[1], 1), "all_gather_ring_gbs": round(gbs[2], 1)}
    return w.name, ms_step, (rs_b + 2 * ag_b) / (ms_step / 1e3) / 1e9, roofline, extra, "bf16"


def bench_schedules(args):
    """The 7B-layer slab through the schedule-faithful collectives: reduce-
    scatter in rank order and in ring order, then all-gather by the ring,
    bidirectional-ring and recursive-doubling step executors (one launch per
    step, chunks at their own index)."""
    import torch
    import synth
    from gradient_reduction_amd import dc
    from synth import workloads as wl
    w = wl.rs_ag_w8()
    W, M, L = w.W, w.M, w.M // w.W
    dev = torch.device("cuda:0")
    x = torch.empty((W, w.ld), dtype=torch.int16, device=dev)
    synth.fill_slab_device(0, w.value_seed, 0, w.scale, W, w.ld, M, x.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    ld_sh = wl.round_up(L, 64)
    sh = torch.empty((W, ld_sh), dtype=torch.int16, device=dev)
    out = torch.empty((W, w.ld), dtype=torch.int16, device=dev)
    scheds = [("ring", dc.DC_SCHED_RING, W - 1), ("bidir", dc.DC_SCHED_BIDIR, W // 2),
              ("rd", dc.DC_SCHED_RD, W.bit_length() - 1)]
    rs_b = W * M * 2 + M * 2
    # step 0 reads the W shards and writes them in place; every later chunk
    # moved is read from one node's row and written to another's: W*(W-1)
    # chunks of L in all, whatever the schedule.
    ag_b = 2 * (M + (W - 1) * M) * 2
    names = ["rs_rank", "rs_ring"] + [f"ag_{n}" for n, _, _ in scheds]

    def step(tm=None):
        if tm: tm.ev[0][0].record()
        dc.dc_reduce_scatter(W, 0, x, w.ld, sh, ld_sh, M, 1)
        if tm: tm.ev[0][1].record(); tm.ev[1][0].record()
        dc.dc_reduce_scatter_ring(W, 0, x, w.ld, sh, ld_sh, M, 1)
        if tm: tm.ev[1][1].record()
        for k, (_, algo, S) in enumerate(scheds):
            if tm: tm.ev[2 + k][0].record()
            for s in range(S + 1):
                dc.dc_all_gather_step(W, 0, sh, ld_sh, out, w.ld, L, algo, s)
            if tm: tm.ev[2 + k][1].record()

    ms_step, kern_all = run_timed(torch, args, step, len(names))
    kern = kern_all.mean(axis=0)
    byts = [rs_b, rs_b] + [ag_b] * len(scheds)
    gbs = {n: b / (t / 1e3) / 1e9 for n, b, t in zip(names, byts, kern)}
    log("[bench] " + ", ".join(f"{n} {kern[i]:.3f} ms {gbs[n]:.1f} GB/s" for i, n in enumerate(names)))
    roofline = {"bound": "hbm", "achieved": round(gbs["rs_ring"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs["rs_ring"] / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile("schedules_w8", w.name),
                "kernel": "k_rs_ring", "launch_ms_avg": round(float(kern[1]), 4),
                "bytes_per_launch_avg": rs_b, "bytes_per_launch": [rs_b]}
    add_mix_ceiling(roofline, stream_rows_gbs(x, w.ld // 8, W, out, w.ld // 8, 1, M // 8),
                    f"read {W} rows, write 1")
    extra = {n: {"ms": round(float(kern[i]), 4), "gbs": round(gbs[n], 1)} for i, n in enumerate(names)}
    extra["ag_launches"] = {n: S + 1 for n, _, S in scheds}
    # rank-order against ring-order shards: both are correct sums, in
    # different orders; how far apart they land in bf16
    rk = torch.empty_like(sh)
    dc.dc_reduce_scatter(W, 0, x, w.ld, rk, ld_sh, M, 1)
    dc.dc_reduce_scatter_ring(W, 0, x, w.ld, sh, ld_sh, M, 1)
    a = rk[:, :L].view(torch.bfloat16).float()
    r = sh[:, :L].view(torch.bfloat16).float()
    diff = (a - r).abs()
    extra["ring_vs_rank"] = {
        "elements_differing": int((diff > 0).sum()),
        "elements": int(diff.numel()),
        "max_abs_diff_over_max_abs": float(diff.max() / a.abs().max()),
        "max_rel_diff_where_abs_ge_1pct_of_max": float(
            (diff / a.abs().clamp_min(1e-30))[a.abs() >= 0.01 * a.abs().max()].max())}
    log(f"[bench] ring vs rank order: {extra['ring_vs_rank']}")
    return w.name, ms_step, sum(byts) / (ms_step / 1e3) / 1e9, roofline, extra, "bf16"


def bench_relayout_rs(args):
    """Every bucket of the W=8 402.8M workload relaid by destination rank and
    reduce-scattered with variable shards (the issue's reduce-scatter
    alternative): one step = relayout + reduce-scatter-v of every bucket."""
    import torch
    import synth
    from gradient_reduction_amd import dc, executor
    from synth import workloads as wl
    w = wl.owner_flush_w8()
    W, ld, b = w.W, w.ld, w.elem_bytes()
    dev = torch.device("cuda:0")
    x = torch.empty((W, ld), dtype=torch.int16, device=dev)
    synth.fill_slab_device(0, w.value_seed, 0, w.scale, W, ld, w.total, x.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    ex = executor.from_workload(w, reduce_to_owner=False, log=log, zero2=True)
    ex.build_owner_map()
    flat = ex.d_flat[:w.P].cpu().numpy()
    plans = []
    for bk in w.buckets:
        t = dc.tasks_array([(k.offset, k.numel, k.param, k.comm) for k in bk.tasks])
        pieces, seg = dc.dc_plan_relayout(W, t, len(t), flat, ex.h_psize, w.P)
        plans.append((torch.from_numpy(pieces.view(np.uint8).copy()).to(dev), len(pieces), seg))
    maxn = max(int(p[2][-1]) for p in plans)
    maxseg = max(int(max(p[2][1:] - p[2][:-1])) for p in plans)
    ld_r, ld_s = wl.round_up(maxn, 64), wl.round_up(maxseg, 64)
    relaid = torch.empty((W, ld_r), dtype=torch.int16, device=dev)
    shards = torch.empty((W, ld_s), dtype=torch.int16, device=dev)
    nb = len(w.buckets)
    rl_b = [2 * W * int(p[2][-1]) * b + 32 * p[1] for p in plans]
    rs_b = [W * int(p[2][-1]) * b + int(p[2][-1]) * b for p in plans]

    def step(tm=None):
        for k, bk in enumerate(w.buckets):
            d_pieces, npc, seg = plans[k]
            if tm: tm.ev[2 * k][0].record()
            dc.dc_relayout_bucket(W, 0, x, ld, relaid, ld_r, bk.col, bk.numel, d_pieces, npc,
                                  int(seg[-1]))
            if tm: tm.ev[2 * k][1].record(); tm.ev[2 * k + 1][0].record()
            dc.dc_reduce_scatter_v(W, 0, relaid, ld_r, shards, ld_s, seg, w.pre_div)
            if tm: tm.ev[2 * k + 1][1].record()

    ms_step, kern_all = run_timed(torch, args, step, 2 * nb)
    kern = kern_all.mean(axis=0)
    rl_gbs = sum(rl_b) / (kern[0::2].sum() / 1e3) / 1e9
    rs_gbs = sum(rs_b) / (kern[1::2].sum() / 1e3) / 1e9
    log(f"[bench] relayout + reduce-scatter-v: step {ms_step:.3f} ms; relayout {rl_gbs:.1f} GB/s "
        f"({kern[0::2].sum():.3f} ms); reduce-scatter-v {rs_gbs:.1f} GB/s ({kern[1::2].sum():.3f} ms)")
    roofline = {"bound": "hbm", "achieved": round(rs_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(rs_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile("relayout_rs_w8", w.name), "kernel": "k_rs_v",
                "launch_ms_avg": round(float(kern[1::2].mean()), 4),
                "bytes_per_launch_avg": int(np.mean(rs_b)),
                "bytes_per_launch": [int(b) for b in rs_b]}
    extra = {"relayout_gbs": round(rl_gbs, 1), "relayout_ms": round(float(kern[0::2].sum()), 4),
             "reduce_scatter_v_ms": round(float(kern[1::2].sum()), 4)}
    # references at the largest relaid bucket: reduce-scatter-v reads W rows and
    # writes one row's worth; the relayout reads and writes all W rows (the
    # input slab is not used after the timed steps)
    nvec = maxn // 8
    add_mix_ceiling(roofline, stream_rows_gbs(relaid, ld_r // 8, W, x, ld // 8, 1, nvec),
                    f"read {W} rows, write 1")
    rl_ref = stream_rows_gbs(x, ld // 8, W, relaid, ld_r // 8, W, nvec)
    extra["relayout_access_mix_ceiling_gbs"] = round(rl_ref, 1)
    extra["relayout_frac_of_access_mix_ceiling"] = round(rl_gbs / rl_ref, 4)
    return w.name, ms_step, (sum(rl_b) + sum(rs_b)) / (ms_step / 1e3) / 1e9, roofline, extra, "bf16"


def copy_calibration():
    """Achievable bandwidth of a plain 16-byte streaming copy (1 GiB)."""
    import torch
    from gradient_reduction_amd import dc
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        dc.dc_stream_copy(a, b, n)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dc.dc_stream_copy(a, b, n)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    return round(2 * n / (ms / 1e3) / 1e9, 1)


def system_info():
    """Host and GPU state next to the figures: CPU model, cores, memory, and
    rocm-smi's clocks and power (when the tool answers)."""
    import subprocess
    info = {"cpu_threads": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            lines = f.read().splitlines()
        names = [ln.split(":", 1)[1].strip() for ln in lines if ln.startswith("model name")]
        phys = {ln.split(":", 1)[1].strip() for ln in lines if ln.startswith("physical id")}
        info["cpu_model"] = names[0] if names else None
        info["sockets"] = len(phys) or None
        with open("/proc/meminfo") as f:
            info["mem_total_gb"] = round(int(f.readline().split()[1]) / 2 ** 20, 1)
    except OSError:
        pass
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"],
                           capture_output=True, text=True, timeout=20)
        if r.returncode == 0 and r.stdout.strip().startswith("{"):
            card = next(iter(json.loads(r.stdout).values()))
            info["gpu"] = {k: v for k, v in card.items()
                           if any(t in k.lower() for t in ("sclk", "mclk", "fclk", "power"))}
    except (OSError, subprocess.SubprocessError, ValueError, StopIteration, AttributeError):
        pass
    return info


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="owner_w8",
                    choices=["owner_w8", "allreduce_w8", "zero2_w8", "layered_w8",
                             "layered_allreduce_w8", "mixed", "zero2_mixed",
                             "deferred", "rs_ag", "schedules_w8", "relayout_rs_w8", "fused_w8",
                             "fused_mixed", "tiny"])
    ap.add_argument("--ga", type=int, default=8)
    ap.add_argument("--fused", action="store_true",
                    help="deferred workload: fuse the last accumulate into the reduce")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--searched", action="store_true",
                    help="flush and fused workloads: flush without plans (each tile searches "
                         "the task table) instead of with the per-bucket tile plans")
    ap.add_argument("--probe", action="store_true",
                    help="flush workloads: print the probe line of each of the first 20 flushes "
                         "(the executor's reduce_probe), as they are issued")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path simulates W data-parallel ranks as rows "
              f"of one GPU's gradient slab, so --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from gradient_reduction_amd import dc
    dc.lib()
    from synth import workloads as wl

    calib = copy_calibration()
    log(f"[bench] streaming copy reference: {calib} GB/s")
    cpu = None
    flush_workloads = {"owner_w8": wl.owner_flush_w8, "allreduce_w8": wl.owner_flush_w8,
                       "zero2_w8": wl.owner_flush_w8, "layered_w8": wl.owner_flush_w8_layered,
                       "layered_allreduce_w8": wl.owner_flush_w8_layered,
                       "mixed": wl.mixed_flush_w16, "zero2_mixed": wl.mixed_flush_w16,
                       "tiny": wl.tiny_flush}
    if args.workload in flush_workloads:
        w = flush_workloads[args.workload]()
        zero2 = args.workload.startswith("zero2")
        owner_mode = "allreduce" not in args.workload and not zero2
        ms, value, step_bytes, roof, extra = bench_flush(args, w, owner_mode, zero2)
        name, dtype = w.name, wl.DTYPE_NAME[w.dtype]
        config = {"workload": name, "W": w.W, "elements": w.total, "buckets": len(w.buckets),
                  "tasks_per_bucket": [len(b.tasks) for b in w.buckets],
                  "bucket_capacity": w.capacity,
                  "mode": "zero2" if zero2 else ("reduce_to_owner" if owner_mode else "allreduce"),
                  "pre_div": w.pre_div, "step": "owner map + every bucket flush",
                  "flush": ("searched: each tile looks up its tasks" if args.searched else
                            "planned: per-bucket tile plans built once at init on the host"),
                  "step_bytes": step_bytes}
        if not args.no_cpu_baseline and not zero2:
            # the whole step when its slab fits a few GB of host memory (about 20 s
            # of single-threaded oracle work for the W=8 402.8M workload), else
            # the first two buckets
            whole = w.W * w.total * w.elem_bytes() < 8e9
            cpu, cpu_par = cpu_baseline_flush(w, owner_mode,
                                              max_buckets=len(w.buckets) if whole else 2)
            extra["cpu_oracle_all_threads"] = cpu_par
    elif args.workload in ("fused_w8", "fused_mixed"):
        w = wl.owner_flush_w8() if args.workload == "fused_w8" else wl.mixed_flush_w16()
        ms, value, step_bytes, roof, extra = bench_flush_buffers(args, w)
        name, dtype = w.name, wl.DTYPE_NAME[w.dtype]
        config = {"workload": name, "W": w.W, "elements": w.total, "buckets": len(w.buckets),
                  "mode": "copy-in/copy-out fused flush into per-rank grad buffers",
                  "flush": ("searched: each tile looks up its tasks" if args.searched else
                            "planned: per-bucket tile plans built once at registration"),
                  "pre_div": w.pre_div, "step": "owner map + every bucket flush",
                  "step_bytes": step_bytes}
    elif args.workload == "deferred":
        name, ms, value, roof, extra, dtype = bench_deferred(args)
        config = {"workload": name, "W": 4, "K": args.ga,
                  "step": ("K-1 accumulates + fused accumulate-reduce" if args.fused
                           else "K accumulates + deferred reduce")}
    elif args.workload == "relayout_rs_w8":
        name, ms, value, roof, extra, dtype = bench_relayout_rs(args)
        config = {"workload": name, "W": 8,
                  "step": "relayout by destination + reduce-scatter-v of every bucket"}
    elif args.workload == "schedules_w8":
        name, ms, value, roof, extra, dtype = bench_schedules(args)
        config = {"workload": name, "W": 8,
                  "step": "reduce-scatter rank + ring order, all-gather ring/bidir/rd step executors"}
    else:
        name, ms, value, roof, extra, dtype = bench_rs_ag(args)
        config = {"workload": name, "W": 8, "step": "reduce-scatter + all-gather rank + all-gather ring"}
    roof["copy_reference_gbs"] = calib
    line = {"metric": "bucket-flush GB/s (bytes read+written/time) and % of MI355X HBM peak, W=8",
            "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic (seeded SplitMix64 Irwin-Hall gradients, random-init shapes)",
            "config": config, "roofline": roof, "cpu_baseline": cpu, "detail": extra,
            "system": system_info()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
