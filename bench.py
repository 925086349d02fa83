"""Benchmark of the data-parallel gradient-reduction hot path on one MI355X.

Default workload: the W=8 reduce-to-owner bucket flush of a 402.8M-element
bf16 gradient (DeepSpeed issue "DeepCompile ZeRO-1: reduce-to-owner instead
of AllReduce", "Additional context": 8 ranks, 402.8M parameters, buckets of
52,428,800 elements, about 118 tasks per bucket), held as a [8, M] slab in HBM.

One step = the owner map (partition lists + owner map kernels) and the flush
of every bucket, in arrival order.  Metric: algorithmic bytes read + written
per step / step time (GB/s), and the flush kernel against MI355X's 8 TB/s HBM
peak.  Algorithmic bytes of a task of n elements over W ranks, b bytes each:
W*n*b read + (owner ? 1 : W)*n*b written + its 32-byte task record (+ 16
bytes per plan record a planned launch reads).

The default run also
  * compares every output element of the timed step with the oracle (the
    CPU oracle on the host's threads, inputs from the same seeded generator)
    and exits with status 3 on any mismatch;
  * times the oracle itself (one thread on a sample, all threads on the
    whole step, medians of 3) as the CPU baseline;
  * times the qwen3-0.6b W=4 fp32 gradient-accumulation step at K = 8, with
    the deferred reduce and with the last accumulate fused into it, checks
    its every output against the oracle, and reports both under
    detail.deferred (MaxText PR "Defer the data-parallel gradient
    all-reduce to update() under gradient accumulation", What and Results).

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
import statistics
import subprocess
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "bucket-flush GB/s (bytes read+written/time) and % of MI355X HBM peak, W={W}"
PARITY_EXIT = 3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Algorithmic bytes
# ---------------------------------------------------------------------------

def flush_bytes(w, owner, psize=None, tiles=None):
    """Algorithmic bytes of every flush launch of workload w (ZeRO-2 when
    psize, the per-param partition size, is given): every row read, the rows
    written, 32 bytes per task record and, for a planned flush (tiles: the
    plan record count of each bucket), 16 bytes per plan record."""
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


# ---------------------------------------------------------------------------
# Timing
# ---------------------------------------------------------------------------

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


def time_steps(torch, args, step):
    """ms per step of `step` alone (warm-up, then args.steps bracketed by
    events), for variants reported beside the main step."""
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        step()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / args.steps


def region_launch_ms(torch, args, launches, n):
    """Average duration of one launch of a kernel, timed as a region:
    `launches` issues n launches of it back to back with nothing else on the
    stream, and one HIP event pair brackets args.steps rounds of that (after
    warm-up).  The gaps between the launches count against the kernel.  The
    events run_timed records around every launch add a packet of their own to
    each launch, which the kernel trace does not see (about 2% on a
    quarter-millisecond launch), so roofline figures use this timing."""
    return time_steps(torch, args, launches) / n


REGION_TIMING = ("one HIP event pair around args.steps rounds of the kernel's launches issued back to "
                 "back on its stream, no other work between; launch_ms_avg = that time / launches")


def per_launch_events(gbs, ms):
    return {"gbs": round(gbs, 1), "launch_ms_avg": round(ms, 4),
            "what": "HIP events around every launch inside the step; each event adds its own packet"}


def graph_step_ms(torch, args, g):
    """Average time of one replay of a captured step (same warm-up and step
    counts as the eager timing)."""
    return time_steps(torch, args, g.replay)


def gpu_state_under_load(torch, step, seconds=1.5):
    """rocm-smi's clocks and power while `step` runs: the steps are enqueued
    (the host runs ahead of the GPU), the tool is sampled from a second
    thread while they execute, then the stream is drained."""
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t0, 1e-4)
    n = int(min(20000, max(50, seconds / one)))
    sample = {}

    def smi():
        sample.update(rocm_smi())
    th = threading.Thread(target=smi)
    for i in range(n):
        step()
        if i == min(n - 1, 20):
            th.start()
    th.join()
    torch.cuda.synchronize()
    return {"steps_enqueued": n, **sample}


def rocm_smi():
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"],
                           capture_output=True, text=True, timeout=20)
        if r.returncode == 0 and r.stdout.strip().startswith("{"):
            card = next(iter(json.loads(r.stdout).values()))
            return {k: v for k, v in card.items()
                    if any(t in k.lower() for t in ("sclk", "mclk", "fclk", "power"))}
    except (OSError, subprocess.SubprocessError, ValueError, StopIteration, AttributeError):
        pass
    return {}


# ---------------------------------------------------------------------------
# Access-mix reference
# ---------------------------------------------------------------------------

def stream_rows_gbs(src, src_ld_vec, rows_read, dst, dst_ld_vec, rows_written, nvec, shape=None):
    """GB/s of the access-mix reference (xor only) reading rows_read rows and
    writing rows_written rows of nvec 16-byte vectors: dc_stream_rows (one
    vector per thread, full occupancy) or, with shape = (group, cap),
    dc_stream_rows_shaped.  3 untimed launches, then the average of 10."""
    import torch
    from gradient_reduction_amd import dc

    def run():
        if shape is None:
            dc.dc_stream_rows(src, src_ld_vec, rows_read, dst, dst_ld_vec, rows_written, nvec)
        else:
            dc.dc_stream_rows_shaped(src, src_ld_vec, rows_read, dst, dst_ld_vec, rows_written,
                                     nvec, shape[0], shape[1])
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


# Launch shapes the access-mix reference is swept over: full occupancy with
# one vector per thread, and (runs of 64 vectors per workgroup, workgroups
# per compute unit) covering the shapes the library's streaming kernels
# launch with.  The reference for a mix is the best of them.
REFERENCE_SHAPES = [None, (1, 0), (1, 3), (1, 4), (1, 5), (1, 6), (1, 7), (1, 8), (1, 9), (1, 10),
                    (1, 12), (1, 14), (2, 6), (2, 8), (2, 10), (2, 12), (4, 5), (4, 6), (4, 7),
                    (4, 8)]


def shape_name(sh):
    return ("1 vector per thread, full occupancy" if sh is None else
            f"{64 * sh[0]} vectors per workgroup, " +
            (f"at most {sh[1]} per CU" if sh[1] else "full occupancy"))


def best_reference(src, src_ld_vec, rows_read, dst, dst_ld_vec, rows_written, nvec):
    """(best GB/s, its shape) of the access-mix reference over REFERENCE_SHAPES."""
    best, shape = 0.0, None
    for sh in REFERENCE_SHAPES:
        if sh is None and not (rows_read in (4, 8, 16) and rows_written in (1, rows_read)):
            continue          # other mixes: shaped launches only
        g = stream_rows_gbs(src, src_ld_vec, rows_read, dst, dst_ld_vec, rows_written, nvec, sh)
        if g > best:
            best, shape = g, sh
    return best, shape_name(shape)


def add_mix_reference(roofline, ref, what):
    gbs, shape = ref
    roofline["access_mix_reference_gbs"] = round(gbs, 1)
    roofline["frac_of_access_mix_reference"] = round(roofline["achieved"] / gbs, 4)
    roofline["access_mix_reference"] = (f"{what}, xor only: the best of {len(REFERENCE_SHAPES)} "
                                        f"launch shapes ({shape})")
    log(f"[bench] access-mix reference ({what}): {gbs:.1f} GB/s at {shape}; the kernel reaches "
        f"{roofline['frac_of_access_mix_reference']:.3f} of it")


def flush_mix_reference(w, owner, x, y, ld, psize=None, split=None):
    """The memory system's rate for the flush's own access mix: W rows read
    and one row written (owned tasks) or W rows written (AllReduce tasks),
    each the best over REFERENCE_SHAPES at the bucket size, blended by the
    step's bytes (split = (one-row bytes, W-row bytes) when given).  None
    when W has no reference kernel."""
    if w.W not in (4, 8, 16):
        return None
    E = 16 // w.elem_bytes()
    nvec = min(w.capacity, w.total) // E
    ldv = ld // E
    refs = {nw: best_reference(x, ldv, w.W, y, ldv, nw, nvec) for nw in (1, w.W)}
    b = w.elem_bytes()
    own = ar = 0
    if split is not None:
        own, ar = split
    else:
        for bk in w.buckets:
            for t in bk.tasks:
                if psize is not None:
                    one = t.comm == 0 and psize[t.param] > 0
                else:
                    one = owner is not None and t.comm == 0 and owner[t.param] >= 0
                if one:
                    own += (w.W + 1) * t.numel * b
                else:
                    ar += 2 * w.W * t.numel * b
    ref = (own + ar) / ((own / refs[1][0] if own else 0.0) + (ar / refs[w.W][0] if ar else 0.0))
    log(f"[bench] access-mix reference: read {w.W} write 1 {refs[1][0]:.1f} GB/s ({refs[1][1]}), "
        f"read {w.W} write {w.W} {refs[w.W][0]:.1f} GB/s ({refs[w.W][1]}); blended {ref:.1f} GB/s")
    return ref, f"read {w.W} write 1 at {refs[1][1]}; read {w.W} write {w.W} at {refs[w.W][1]}"


# ---------------------------------------------------------------------------
# Counter summaries behind `traffic`
# ---------------------------------------------------------------------------

# bench workload -> (profile stem, source file of its dominant kernel).  A
# summary counts only while the kernel's source and the shared device
# headers still hash to what they were when the counters were taken.
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
    "relayout_rs_relayout": ("relayout_w8_402m", "relayout.hip"),
    "deferred": ("deferred_qwen3_k8", "slab_ops.hip"),
    "deferred_fused": ("deferred_qwen3_k8_fused", "slab_ops.hip"),
    "deferred_accumulate": ("deferred_qwen3_k8_accumulate", "slab_ops.hip"),
    "rs_ag": ("rs_ag_w8_202m", "slab_ops.hip"),
    "rs_ag_allgather": ("allgather_w8_202m", "slab_ops.hip"),
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


# ---------------------------------------------------------------------------
# The oracle on the host: whole-output parity and the CPU baseline
# ---------------------------------------------------------------------------

def _median3(fn):
    """Median of three timed runs of fn() (seconds) and fn's last result."""
    ts, res = [], None
    for _ in range(3):
        t = time.perf_counter()
        res = fn()
        ts.append(time.perf_counter() - t)
    return statistics.median(ts), res


def _bits(a, dtype):
    return a.view(np.uint16) if dtype == 0 else a.view(np.uint32)


def _gpu_cols(y, c0, n, dtype):
    a = y[:, c0:c0 + n].contiguous().cpu().numpy()
    return _bits(a, dtype)


def flush_oracle(w, y, mode, init="zero", max_buckets=None, sample_buckets=2):
    """The oracle against the GPU's flush output y ([W, ld] device slab
    holding the step's result) on every column of every bucket (or the first
    max_buckets), and the CPU baseline:
      parity       {"columns_checked", "elements_checked", "mismatches"}
      all_threads  the oracle over the checked buckets on the host's threads,
                   median of 3 (inputs generated first, untimed)
      one_thread   the oracle on one thread over the first sample_buckets
                   buckets, median of 3 (the reported baseline)
    mode: "owner", "allreduce" or "zero2"; init: what y held before the step."""
    import concurrent.futures
    from oracle import columns as OC
    owner = OC.owner_of(w) if mode == "owner" else None
    zero2 = OC.zero2_tables(w) if mode == "zero2" else None
    psize = zero2[1] if zero2 is not None else None
    per = flush_bytes(w, owner, psize)
    nb = len(w.buckets) if max_buckets is None else min(max_buckets, len(w.buckets))
    sample_buckets = min(sample_buckets, nb)
    k = OC.nthreads()
    cols = elems = bad = 0
    first_bad = None
    par_s = one_s = 0.0

    def fresh(hin):
        if init == "input":
            return hin.copy()
        out = np.zeros_like(hin)
        if init != "zero":
            _bits(out, w.dtype)[:] = init
        return out

    with concurrent.futures.ThreadPoolExecutor(k) as pool:
        for b in range(nb):
            bk = w.buckets[b]
            hin = OC.host_rows(w.dtype, w.value_seed, 0, w.scale, w.W, bk.col, bk.numel)
            hin = np.ascontiguousarray(hin[:, :bk.numel])
            tasks = OC.bucket_tasks(bk)

            def par():
                out = fresh(hin)
                OC.flush_blocks(w, hin, out, tasks, owner=owner, zero2=zero2, pool=pool)
                return out
            t, want = _median3(par)
            par_s += t
            if b < sample_buckets:
                def one():
                    out = fresh(hin)
                    OC.flush_blocks(w, hin, out, tasks, owner=owner, zero2=zero2, threads=1,
                                    block=1 << 62)
                    return out
                t1, want1 = _median3(one)
                one_s += t1
                assert np.array_equal(_bits(want1, w.dtype), _bits(want, w.dtype)), \
                    "one-thread and all-thread oracle runs differ"
            got = _gpu_cols(y, bk.col, bk.numel, w.dtype)
            diff = got != _bits(want, w.dtype)
            nbad = int(np.count_nonzero(diff))
            if nbad and first_bad is None:
                r, c = np.argwhere(diff)[0]
                first_bad = {"bucket": b, "row": int(r), "column": int(bk.col + c)}
            bad += nbad
            cols += bk.numel
            elems += got.size
            log(f"[bench] oracle parity bucket {b}: {bk.numel} columns x {w.W} rows, {nbad} mismatches")
            del hin, want, got, diff
    checked = sum(per[:nb])
    sampled = sum(per[:sample_buckets])
    parity = {"columns_checked": int(cols), "elements_checked": int(elems), "mismatches": int(bad),
              "columns_total": int(w.total)}
    if first_bad:
        parity["first_mismatch"] = first_bad
    base = {"value": round(sampled / one_s / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": (f"buckets 0..{sample_buckets - 1} of {len(w.buckets)} "
                       f"({sum(w.buckets[i].numel for i in range(sample_buckets))} columns, "
                       f"{sampled} algorithmic bytes), oracle.c on one thread, median of 3 runs "
                       f"of {one_s / 1:.2f} s in all; inputs generated first, untimed")}
    allc = {"value": round(checked / par_s / 1e9, 4), "unit": "GB/s", "threads": k,
            "host_cpus": os.cpu_count(), "seconds_median": round(par_s, 3),
            "sample": f"{nb} of {len(w.buckets)} buckets, every column, median of 3"}
    log(f"[bench] cpu oracle: one thread {base['value']} GB/s, {k} threads {allc['value']} GB/s; "
        f"parity: {bad} mismatches over {elems} elements")
    return parity, base, allc


# ---------------------------------------------------------------------------
# Flush workloads
# ---------------------------------------------------------------------------

def device_plan_check(torch, args, ex, host_plan_s):
    """The step's plans built again on the device (dc_plan_flush_device, from
    the device task table and owner map), compared with the host planner's
    record for record, and the device planner's launches timed as one region
    per step.  The flushes keep the host's plans."""
    from gradient_reduction_amd import dc
    host_tiles, host_roots, host_begin = ex.d_tiles, list(ex.root_tiles), ex.tile_begin.copy()
    ex.plan(on_device=True)
    same = (np.array_equal(ex.tile_begin, host_begin) and ex.root_tiles == host_roots
            and bool(torch.equal(ex.d_tiles, host_tiles)))
    dev_tiles = ex.d_tiles
    nb = len(ex.buckets)
    counts = np.diff(host_begin)
    roots = torch.empty(max(nb, 1), dtype=torch.int64, device=dev_tiles.device)
    if ex.zero2:
        owner, flat, psize = None, ex.d_flat, ex.d_psize
    else:
        owner, flat, psize = (ex.d_owner if ex.reduce_to_owner else None), None, None

    def launches():
        for b, bk in enumerate(ex.buckets):
            dc.dc_plan_flush_device(ex.W, ex.dtype, bk.col, bk.numel, ex.task_table(b), len(bk.tasks),
                                    owner, flat, psize, ex.P, ex.comms, len(ex.comms),
                                    dev_tiles.data_ptr() + 16 * int(host_begin[b]), int(counts[b]),
                                    roots.data_ptr() + 8 * b)
    ms = region_launch_ms(torch, args, launches, 1)
    ex.d_tiles, ex.root_tiles = host_tiles, host_roots
    log(f"[bench] device-built plans {'equal' if same else 'DIFFER FROM'} the host's; device planner "
        f"{ms * 1e3:.1f} us per step, host planner {host_plan_s * 1e3:.1f} ms")
    return {"records_equal_host": same, "device_us_per_step": round(ms * 1e3, 2),
            "device_us_per_bucket": round(ms * 1e3 / max(nb, 1), 2),
            "host_ms_per_step": round(host_plan_s * 1e3, 2), "tiles": int(host_begin[-1]),
            "timing": ("one HIP event pair around args.steps rounds of the step's planner calls "
                       "(per bucket: the count-clearing kernel and k_plan_flush) issued back to back "
                       "on the stream after warm-up; device_us_per_step = that time / rounds"),
            "what": ("the step's flush plans built on the device (dc_plan_flush_device) against the "
                     "host planner's, record for record; the flushes use the host's")}


def bench_flush(args, w, mode):
    """The step (owner map + every bucket flush) of flush workload w in mode
    "owner", "allreduce" or "zero2"."""
    import torch
    import synth
    from gradient_reduction_amd import executor

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    ld = w.ld
    dt = torch.int16 if w.dtype == 0 else torch.int32
    zero2 = mode == "zero2"
    log(f"[bench] {w.name}: W={w.W} elements={w.total} buckets={len(w.buckets)} "
        f"tasks={[len(b.tasks) for b in w.buckets]} slab={w.W * ld * w.elem_bytes() / 1e9:.2f} GB")
    x = torch.empty((w.W, ld), dtype=dt, device=dev)
    synth.fill_slab_device(w.dtype, w.value_seed, 0, w.scale, w.W, ld, w.total, x.data_ptr(),
                           stream.cuda_stream)
    y = torch.zeros((w.W, ld), dtype=dt, device=dev)
    ex = executor.from_workload(w, reduce_to_owner=(mode == "owner"), log=log, zero2=zero2,
                                reduce_probe=args.probe)
    ex.build_owner_map()
    ex.fetch_metadata()
    log("[bench] " + ex.ratio_line())
    if not zero2:
        for b in range(min(len(w.buckets), 3)):
            log("[bench] " + ex.probe_line(b, b))
    owner = ex.h_owner if mode == "owner" else None
    tiles = None
    device_plans = None
    if not args.searched:
        t0 = time.perf_counter()
        ex.plan()
        host_plan_s = time.perf_counter() - t0
        tiles = np.diff(ex.tile_begin)
        log(f"[bench] flush plans: {tiles.tolist()} records per bucket")
        device_plans = device_plan_check(torch, args, ex, host_plan_s)
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

    def flushes_only():
        for b in range(nb):
            ex.flush(b, x, ld, y, ld)

    ms_step, kern_all = run_timed(torch, args, step, nb + 1)
    kern, owner_map_ms = kern_all[:, :nb], kern_all[:, nb]    # [steps, buckets], [steps]
    avg_launch_ms = float(kern.mean())
    flush_gbs = sum(per_launch) / (kern.sum(axis=1).mean() / 1e3) / 1e9
    flush_gbs_median = sum(per_launch) / (np.median(kern.sum(axis=1)) / 1e3) / 1e9
    value = step_bytes / (ms_step / 1e3) / 1e9
    log(f"[bench] step {ms_step:.3f} ms, {value:.1f} GB/s; flush kernels {kern.sum(axis=1).mean():.3f} ms "
        f"({flush_gbs:.1f} GB/s); per bucket ms {np.round(kern.mean(axis=0), 4).tolist()}")
    once_ms = region_launch_ms(torch, args, flushes_only, 1)
    region_gbs = sum(per_launch) / (once_ms / 1e3) / 1e9
    log(f"[bench] flushes back to back: {once_ms:.4f} ms per step, {region_gbs:.1f} GB/s")
    roofline = {"bound": "hbm", "achieved": round(region_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(region_gbs / HBM_PEAK_GBS, 4),
                "traffic": (None if args.searched or getattr(args, "bucket_numel", 0)
                            else traffic_from_profile(args.workload, w.name)),
                "kernel": "k_flush_planned" if not args.searched else "k_flush",
                "launch_ms_avg": round(once_ms / nb, 4), "timing": REGION_TIMING,
                "per_launch_events": per_launch_events(flush_gbs, avg_launch_ms),
                "bytes_per_launch_avg": int(np.mean(per_launch)),
                "bytes_per_launch": [int(b) for b in per_launch]}
    ref = flush_mix_reference(w, owner, x, y, ld, ex.h_psize if zero2 else None)
    if ref is not None:
        add_mix_reference(roofline, ref, "the flush's own mix, blended by the step's bytes")
    extra = {"per_bucket_gbs": [round(b / (m / 1e3) / 1e9, 1) for b, m in zip(per_launch, kern.mean(axis=0))],
             "flush_gbs_median_step": round(flush_gbs_median, 1),
             "owner_map_us": round(float(owner_map_ms.mean()) * 1e3, 2),
             "owner_map_once": {
                 "ms_per_step": round(once_ms, 4),
                 "value": round(sum(per_launch) / (once_ms / 1e3) / 1e9, 1),
                 "what": "the same step with the owner map built once at init (the issue's design "
                         "points build it at init and reuse it), flushes only"}}
    if device_plans is not None:
        extra["device_plans"] = device_plans
    extra["graph_ms_per_step"] = round(graph_step_ms(torch, args, ex.capture_step(x, ld, y, ld)), 4)
    log(f"[bench] owner map once: {once_ms:.4f} ms per step; the step replayed as one HIP graph: "
        f"{extra['graph_ms_per_step']:.4f} ms")
    if args.load_sample_s > 0:
        extra["gpu_during_steps"] = gpu_state_under_load(torch, step, args.load_sample_s)
    # the reference runs above wrote into y: clear it and run the step once
    # more, so y holds exactly one step's result over zeros
    y.zero_()
    step()
    torch.cuda.synchronize()
    del x
    return {"ms": ms_step, "value": value, "step_bytes": step_bytes, "roofline": roofline,
            "extra": extra, "y": y}


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

    def flushes_only():
        for b in range(nb):
            ex.flush_buffers(b)

    ms_step, kern_all = run_timed(torch, args, step, nb + 1)
    kern, owner_map_ms = kern_all[:, :nb], kern_all[:, nb]
    ev_gbs = sum(per_launch) / (kern.sum(axis=1).mean() / 1e3) / 1e9
    once_ms = region_launch_ms(torch, args, flushes_only, 1)
    gbs = sum(per_launch) / (once_ms / 1e3) / 1e9
    gbs_median = sum(per_launch) / (np.median(kern.sum(axis=1)) / 1e3) / 1e9
    value = step_bytes / (ms_step / 1e3) / 1e9
    log(f"[bench] step {ms_step:.3f} ms, {value:.1f} GB/s; fused flush kernels back to back "
        f"{once_ms:.3f} ms ({gbs:.1f} GB/s), with events {kern.sum(axis=1).mean():.3f} ms; per bucket ms "
        f"{np.round(kern.mean(axis=0), 4).tolist()}")
    roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4),
                "traffic": None if args.searched else traffic_from_profile(args.workload, w.name),
                "kernel": "k_flush_buffers", "launch_ms_avg": round(once_ms / nb, 4),
                "timing": REGION_TIMING, "per_launch_events": per_launch_events(ev_gbs, float(kern.mean())),
                "bytes_per_launch_avg": int(np.mean(per_launch)),
                "bytes_per_launch": [int(b) for b in per_launch]}
    ref = flush_mix_reference(w, None, x, y, ld, split=(one_b, many_b))
    if ref is not None:
        add_mix_reference(roofline, ref, "the flush's own mix, blended by the step's bytes")
    extra = {"per_bucket_gbs": [round(b / (m / 1e3) / 1e9, 1) for b, m in zip(per_launch, kern.mean(axis=0))],
             "flush_gbs_median_step": round(gbs_median, 1),
             "owner_map_us": round(float(owner_map_ms.mean()) * 1e3, 2),
             "fused_bytes_per_step": int(sum(per_launch)),
             "unfused_bytes_per_step": int(unfused),
             "bytes_saved_frac": round(1 - sum(per_launch) / unfused, 4)}
    del x, y
    torch.cuda.empty_cache()
    return {"ms": ms_step, "value": value, "step_bytes": step_bytes, "roofline": roofline,
            "extra": extra}


# ---------------------------------------------------------------------------
# Deferred reduce under gradient accumulation
# ---------------------------------------------------------------------------

def deferred_oracle(w, K, gpu, chunks=8):
    """The oracle against the deferred step's outputs on every column (in
    column chunks): the accumulators after K accumulates, the deferred
    reduce in every replica row, the fused path's reduce, and the status
    quo; and the oracle's own timing on a sample (one thread and all
    threads, medians of 3).  gpu: dict of device tensors acc, D, Df, A."""
    from oracle import columns as OC
    from synth import workloads as wl
    W, M = w.W, w.M

    def so(k, r):
        return wl.microbatch_stream(k, W, r)
    bad = 0
    elems = 0
    for c in range(chunks):
        c0, c1 = c * M // chunks, (c + 1) * M // chunks
        n = c1 - c0
        acc, D, A = OC.deferred_columns(W, w.value_seed, w.scale, K, so, c0, n)
        d = D.view(np.uint32)
        checks = [(gpu["acc"], acc.view(np.uint32)), (gpu["D"], np.broadcast_to(d, (W, n))),
                  (gpu["Df"], np.broadcast_to(d, (W, n))), (gpu["A"], A.view(np.uint32)[None, :])]
        for t, want in checks:
            got = _gpu_cols(t, c0, n, 1)
            bad += int(np.count_nonzero(got != want))
            elems += got.size
        log(f"[bench] deferred parity, columns [{c0}, {c1}): {bad} mismatches so far")
    parity = {"columns_checked": int(M), "elements_checked": int(elems), "mismatches": int(bad),
              "outputs": "accumulators (W rows), deferred reduce (W rows), fused reduce (W rows), "
                         "status quo (1 row)"}
    # CPU baseline: the deferred step (K accumulates, then the reduce) on a
    # sample of the columns, inputs generated first
    ns = 1 << 27
    xs = [OC.host_rows(1, w.value_seed, 0, w.scale, W, 0, ns, stream_of=lambda r, k=k: so(k, r))
          for k in range(K)]
    xs = [np.ascontiguousarray(x[:, :ns]) for x in xs]
    import oracle

    def one():
        a = np.zeros((W, ns), np.float32)
        for k, x in enumerate(xs):
            oracle.accumulate(W, x, a, ns, 1 if k == 0 else 0)
        d = np.zeros((W, ns), np.float32)
        oracle.deferred_reduce(W, a, d, ns, W)
        return d
    t1, _ = _median3(one)
    sbytes = K * 3 * W * ns * 4 - W * ns * 4 + 2 * W * ns * 4
    base = {"value": round(sbytes / t1 / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the K={K} deferred step (K accumulates + reduce to every replica) over the "
                      f"first {ns} of {M} columns, oracle.c on one thread, median of 3 runs of "
                      f"{t1:.2f} s; inputs generated first, untimed"}
    k_threads = OC.nthreads()
    import concurrent.futures
    blk = 1 << 18

    def par():
        a = np.zeros((W, ns), np.float32)
        d = np.zeros((W, ns), np.float32)

        def run(s):
            m = min(blk, ns - s)
            aa = np.zeros((W, m), np.float32)
            for k, x in enumerate(xs):
                oracle.accumulate(W, np.ascontiguousarray(x[:, s:s + m]), aa, m, 1 if k == 0 else 0)
            dd = np.zeros((W, m), np.float32)
            oracle.deferred_reduce(W, aa, dd, m, W)
            a[:, s:s + m] = aa
            d[:, s:s + m] = dd
        with concurrent.futures.ThreadPoolExecutor(k_threads) as p:
            list(p.map(run, range(0, ns, blk)))
        return d
    tp, dpar = _median3(par)
    allc = {"value": round(sbytes / tp / 1e9, 4), "unit": "GB/s", "threads": k_threads,
            "seconds_median": round(tp, 3), "sample": "the same columns, column blocks over threads"}
    log(f"[bench] deferred cpu oracle: one thread {base['value']} GB/s, {k_threads} threads "
        f"{allc['value']} GB/s; parity: {bad} mismatches over {elems} elements")
    return parity, base, allc


def bench_deferred(args, K, check=True):
    """qwen3-0.6b tree, W = 4 replicas, K micro-batches generated on the
    device (untimed).  Times the deferred step (K accumulates + the deferred
    reduce to every replica), the same with the last accumulate fused into
    the reduce, and the status quo (every micro-batch reduced, the reduced
    gradients accumulated); checks every output against the oracle."""
    import torch
    import synth
    from gradient_reduction_amd import dc
    from synth import workloads as wl
    w = wl.deferred_ga_w4(K)
    W, M, ld = w.W, w.M, w.ld
    dev = torch.device("cuda:0")
    xs = torch.empty((K, W, ld), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    for k in range(K):
        synth.fill_slab_device(1, w.value_seed, wl.microbatch_stream(k, W, 0), w.scale, W, ld, M,
                               xs[k].data_ptr(), s)
    acc = torch.empty((W, ld), dtype=torch.float32, device=dev)
    acc_f = torch.empty((W, ld), dtype=torch.float32, device=dev)
    out = torch.empty((W, ld), dtype=torch.float32, device=dev)
    out_f = torch.empty((W, ld), dtype=torch.float32, device=dev)
    res = {}
    for fused in (False, True):
        n_acc = K - 1 if fused else K
        a_t, o_t = (acc_f, out_f) if fused else (acc, out)
        acc_b = [(2 if k else 1) * W * M * 4 + W * M * 4 for k in range(n_acc)]
        # fused last step: x (and acc unless K = 1) read, W result rows written
        red_b = (((W * M * 4 if K > 1 else 0) + W * M * 4 + W * M * 4) if fused
                 else W * M * 4 + W * M * 4)
        step_bytes = sum(acc_b) + red_b

        def step(tm=None, fused=fused, n_acc=n_acc, a_t=a_t, o_t=o_t):
            for k in range(n_acc):
                if tm: tm.ev[k][0].record()
                dc.dc_accumulate(W, xs[k], ld, a_t, ld, M, 1 if k == 0 else 0)
                if tm: tm.ev[k][1].record()
            if tm: tm.ev[n_acc][0].record()
            if fused:
                dc.dc_accumulate_reduce(W, xs[K - 1], ld, a_t, ld, 1 if K == 1 else 0, 0, o_t, ld, W, M)
            else:
                dc.dc_deferred_reduce(W, a_t, ld, o_t, ld, M, W)
            if tm: tm.ev[n_acc][1].record()

        ms_step, kern_all = run_timed(torch, args, step, n_acc + 1)
        kern = kern_all.mean(axis=0)
        ev_gbs = red_b / (kern[-1] / 1e3) / 1e9
        if fused:
            # repeated, it keeps adding the last micro-batch to the
            # accumulators; the outputs are recomputed from scratch below
            red_ms = region_launch_ms(torch, args, lambda: dc.dc_accumulate_reduce(
                W, xs[K - 1], ld, a_t, ld, 1 if K == 1 else 0, 0, o_t, ld, W, M), 1)
        else:
            red_ms = region_launch_ms(torch, args, lambda: dc.dc_deferred_reduce(
                W, a_t, ld, o_t, ld, M, W), 1)
        red_gbs = red_b / (red_ms / 1e3) / 1e9
        acc_gbs = sum(acc_b) / (kern[:-1].sum() / 1e3) / 1e9 if n_acc else 0.0
        # the accumulates alone, back to back (each round starts from init,
        # so repeating them recomputes the same accumulators)
        acc_ms = region_launch_ms(torch, args, lambda: [
            dc.dc_accumulate(W, xs[k], ld, a_t, ld, M, 1 if k == 0 else 0) for k in range(n_acc)],
            n_acc) if n_acc else 0.0
        acc_region_gbs = sum(acc_b) / (acc_ms * n_acc / 1e3) / 1e9 if n_acc else 0.0
        name = "k_accum_reduce" if fused else "k_deferred"
        log(f"[bench] deferred K={K}{' fused' if fused else ''}: step {ms_step:.3f} ms; accumulate "
            f"{acc_region_gbs:.1f} GB/s back to back ({acc_gbs:.1f} with events); {name} {red_gbs:.1f} GB/s "
            f"({red_ms:.3f} ms back to back, "
            f"{kern[-1]:.3f} ms with events)")
        roofline = {"bound": "hbm", "achieved": round(red_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(red_gbs / HBM_PEAK_GBS, 4),
                    "traffic": traffic_from_profile("deferred_fused" if fused else "deferred",
                                                    w.name, {"ga": K}),
                    "kernel": name, "launch_ms_avg": round(red_ms, 4), "timing": REGION_TIMING,
                    "per_launch_events": per_launch_events(ev_gbs, float(kern[-1])),
                    "bytes_per_launch_avg": red_b, "bytes_per_launch": [red_b]}
        if not fused:
            add_mix_reference(roofline, best_reference(acc, ld // 4, W, out_f, ld // 4, W, M // 4),
                              f"read {W} rows, write {W}")
        elif W == 4:
            # accumulators and micro-batch read (2W rows: the first two
            # micro-batches' rows stand in), every replica row written
            add_mix_reference(roofline, best_reference(xs, ld // 4, 2 * W, out, ld // 4, W, M // 4),
                              f"read {2 * W} rows, write {W}")
        accumulate = {"kernel": "k_accumulate", "bound": "hbm", "achieved": round(acc_region_gbs, 1),
                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(acc_region_gbs / HBM_PEAK_GBS, 4),
                      "launch_ms_avg": round(acc_ms, 4), "timing": REGION_TIMING,
                      "per_launch_events": per_launch_events(acc_gbs, float(kern[:-1].mean()) if n_acc else 0.0),
                      "bytes_per_launch": [int(b) for b in acc_b],
                      "traffic": None if fused else traffic_from_profile("deferred_accumulate", w.name,
                                                                         {"ga": K}),
                      "what": "the step's accumulates (most of its time), timed back to back"}
        res["fused" if fused else "unfused"] = {
            "ms_per_step": round(ms_step, 4), "value": round(step_bytes / (ms_step / 1e3) / 1e9, 1),
            "step_bytes": int(step_bytes), "accumulate_gbs": round(acc_region_gbs, 1),
            "accumulate": accumulate, "roofline": roofline,
            "step": ("K-1 accumulates + fused accumulate-reduce" if fused
                     else "K accumulates + deferred reduce")}
    # both steps once more, so the outputs hold exactly one step's results
    for fused in (False, True):
        n_acc = K - 1 if fused else K
        a_t, o_t = (acc_f, out_f) if fused else (acc, out)
        for k in range(n_acc):
            dc.dc_accumulate(W, xs[k], ld, a_t, ld, M, 1 if k == 0 else 0)
        if fused:
            dc.dc_accumulate_reduce(W, xs[K - 1], ld, a_t, ld, 1 if K == 1 else 0, 0, o_t, ld, W, M)
        else:
            dc.dc_deferred_reduce(W, a_t, ld, o_t, ld, M, W)
    # The pages' status quo beside it: every micro-batch reduced across the
    # replicas, the reduced gradients accumulated (one row).  Timed on its own.
    g = torch.empty((1, ld), dtype=torch.float32, device=dev)
    A = torch.empty((1, ld), dtype=torch.float32, device=dev)

    def quo():
        for k in range(K):
            dc.dc_deferred_reduce(W, xs[k], ld, g, ld, M, 1)
            dc.dc_accumulate(1, g, ld, A, ld, M, 1 if k == 0 else 0)

    res["status_quo_ms_per_step"] = round(time_steps(torch, args, quo), 4)
    torch.cuda.synchronize()
    # numerics of the deferred sum D against the per-micro-batch sum A: the
    # 5e-5 * sum|x| gate, the normwise difference and the largest relative
    # difference where |A| > 1e-3 max|A|
    d, a = out[0, :M].double(), A[0, :M].double()
    diff = (d - a).abs()
    sabs = torch.zeros(M, dtype=torch.float64, device=dev)
    for k in range(K):
        sabs += xs[k, :, :M].abs().sum(dim=0).double()
    big = a.abs() > 1e-3 * a.abs().max()
    res["deferred_vs_per_microbatch"] = {
        "max_diff_over_gate": float((diff / (5e-5 * sabs).clamp_min(1e-300)).max()),
        "normwise": float(diff.norm() / a.norm()),
        "max_rel_where_abs_gt_1e-3_max": float((diff[big] / a.abs()[big]).max()),
        "bit_identical_frac": round(float((diff == 0).double().mean()), 6)}
    log(f"[bench] status quo (reduce every micro-batch, then accumulate): "
        f"{res['status_quo_ms_per_step']:.3f} ms; D vs A: {res['deferred_vs_per_microbatch']}")
    del d, a, diff, sabs, big, xs
    torch.cuda.empty_cache()
    if check:
        parity, base, allc = deferred_oracle(w, K, {"acc": acc, "D": out, "Df": out_f, "A": A})
        res["parity"] = parity
        res["cpu_baseline"] = base
        res["cpu_oracle_all_threads"] = allc
    res["workload"] = w.name
    del acc, acc_f, out, out_f, A, g
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# Reduce-scatter / all-gather and the schedules
# ---------------------------------------------------------------------------

def rs_ag_oracle(w, sh, rank, ring, ld_sh):
    """The oracle against the 7B-layer reduce-scatter shards and both
    all-gathers on every element, and the oracle's reduce-scatter timing
    (one thread on a quarter of the shard columns, all threads on all of
    them, medians of 3)."""
    from oracle import columns as OC
    from gradient_reduction_amd import dc
    W, M, dtype = w.W, w.M, w.dtype
    L = M // W
    hin = OC.host_rows(dtype, w.value_seed, 0, w.scale, W, 0, M)
    hin = np.ascontiguousarray(hin[:, :M])
    tp, want_sh = _median3(lambda: OC.reduce_scatter_columns(W, dtype, hin, M, 0))
    q = L // 4
    sub = np.ascontiguousarray(np.concatenate([hin[:, s * L:s * L + q] for s in range(W)], axis=1))
    t1, _ = _median3(lambda: OC.reduce_scatter_columns(W, dtype, sub, W * q, 0, threads=1,
                                                       block=1 << 62))
    del hin, sub
    bad = 0
    elems = 0
    got = _gpu_cols(sh, 0, L, dtype)
    bad += int(np.count_nonzero(got != want_sh))
    elems += got.size
    for order, y in ((dc.DC_ORDER_RANK, rank), (dc.DC_ORDER_RING, ring)):
        want = OC.all_gather_rows(W, dtype, want_sh, L, order)
        got = _gpu_cols(y, 0, M, dtype)
        bad += int(np.count_nonzero(got != want))
        elems += got.size
    parity = {"columns_checked": int(M), "elements_checked": int(elems), "mismatches": int(bad),
              "outputs": "reduce-scatter shards, all-gather in rank order, all-gather in ring order"}
    rs_b = W * M * 2 + M * 2
    base = {"value": round(rs_b / 4 / t1 / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the reduce-scatter over the first quarter of every shard ({W * q} columns), "
                      f"oracle.c on one thread, median of 3 runs of {t1:.2f} s"}
    allc = {"value": round(rs_b / tp / 1e9, 4), "unit": "GB/s", "threads": OC.nthreads(),
            "seconds_median": round(tp, 3), "sample": "the whole reduce-scatter, shard column blocks"}
    log(f"[bench] rs/ag parity: {bad} mismatches over {elems} elements; cpu oracle one thread "
        f"{base['value']} GB/s")
    return parity, base, allc


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
    out_ring = torch.empty((W, w.ld), dtype=torch.int16, device=dev)
    rs_b = W * M * 2 + M * 2
    ag_b = M * 2 + W * M * 2

    def step(tm=None):
        if tm: tm.ev[0][0].record()
        dc.dc_reduce_scatter(W, 0, x, w.ld, sh, ld_sh, M, 0)
        if tm: tm.ev[0][1].record(); tm.ev[1][0].record()
        dc.dc_all_gather(W, 0, sh, ld_sh, out, w.ld, L, dc.DC_ORDER_RANK, -1)
        if tm: tm.ev[1][1].record(); tm.ev[2][0].record()
        dc.dc_all_gather(W, 0, sh, ld_sh, out_ring, w.ld, L, dc.DC_ORDER_RING, -1)
        if tm: tm.ev[2][1].record()

    ms_step, kern_all = run_timed(torch, args, step, 3)
    kern = kern_all.mean(axis=0)
    ev = [rs_b / (kern[0] / 1e3) / 1e9, ag_b / (kern[1] / 1e3) / 1e9, ag_b / (kern[2] / 1e3) / 1e9]
    reg = [region_launch_ms(torch, args, lambda: dc.dc_reduce_scatter(W, 0, x, w.ld, sh, ld_sh, M, 0), 1),
           region_launch_ms(torch, args, lambda: dc.dc_all_gather(W, 0, sh, ld_sh, out, w.ld, L,
                                                                  dc.DC_ORDER_RANK, -1), 1),
           region_launch_ms(torch, args, lambda: dc.dc_all_gather(W, 0, sh, ld_sh, out_ring, w.ld, L,
                                                                  dc.DC_ORDER_RING, -1), 1)]
    gbs = [b / (t / 1e3) / 1e9 for b, t in zip((rs_b, ag_b, ag_b), reg)]
    log(f"[bench] back to back: rs {gbs[0]:.1f} GB/s, ag rank {gbs[1]:.1f} GB/s, ag ring {gbs[2]:.1f} GB/s; "
        f"with events: {ev[0]:.1f}, {ev[1]:.1f}, {ev[2]:.1f}")
    roofline = {"bound": "hbm", "achieved": round(gbs[0], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs[0] / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile("rs_ag", w.name), "kernel": "k_rs_vec",
                "launch_ms_avg": round(reg[0], 4), "timing": REGION_TIMING,
                "per_launch_events": per_launch_events(ev[0], float(kern[0])), "bytes_per_launch_avg": rs_b,
                "bytes_per_launch": [rs_b]}
    tmp = torch.empty((W, w.ld), dtype=torch.int16, device=dev)
    add_mix_reference(roofline, best_reference(x, w.ld // 8, W, tmp, w.ld // 8, 1, M // 8),
                      f"read {W} rows, write 1")
    # the all-gather's mix: one row of M read, all W rows of M written (the
    # outputs are recomputed by the step below)
    ag_ref, ag_shape = best_reference(x, w.ld // 8, 1, tmp, w.ld // 8, W, M // 8)
    del tmp
    extra = {"all_gather_rank_gbs": round(gbs[1], 1), "all_gather_ring_gbs": round(gbs[2], 1),
             "all_gather_rank_frac": round(gbs[1] / HBM_PEAK_GBS, 4),
             "all_gather_ring_frac": round(gbs[2] / HBM_PEAK_GBS, 4),
             "all_gather_launch_ms": {"rank": round(reg[1], 4), "ring": round(reg[2], 4)},
             "all_gather_traffic": traffic_from_profile("rs_ag_allgather", w.name),
             "all_gather_roofline": {
                 "kernel": "k_ag_vec", "bound": "hbm",
                 "achieved": round(2 * ag_b / ((reg[1] + reg[2]) / 1e3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                 "unit": "GB/s", "frac": round(2 * ag_b / ((reg[1] + reg[2]) / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                 "launch_ms_avg": round((reg[1] + reg[2]) / 2, 4), "timing": REGION_TIMING,
                 "bytes_per_launch": [ag_b, ag_b],
                 "traffic": traffic_from_profile("rs_ag_allgather", w.name),
                 "access_mix_reference_gbs": round(ag_ref, 1),
                 "frac_of_access_mix_reference": round(2 * ag_b / ((reg[1] + reg[2]) / 1e3) / 1e9 / ag_ref, 4),
                 "access_mix_reference": (f"read 1 row, write {W}, xor only: the best of "
                                          f"{len(REFERENCE_SHAPES)} launch shapes ({ag_shape})"),
                 "what": "the two all-gathers (rank and ring order), the step's larger share of time"},
             "all_gather_gbs_with_events": {"rank": round(ev[1], 1), "ring": round(ev[2], 1)}}
    step()
    torch.cuda.synchronize()
    del x
    torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu_baseline:
        parity, cpu, allc = rs_ag_oracle(w, sh, out, out_ring, ld_sh)
        extra["parity"] = parity
        extra["cpu_oracle_all_threads"] = allc
    return {"name": w.name, "ms": ms_step, "value": (rs_b + 2 * ag_b) / (ms_step / 1e3) / 1e9,
            "roofline": roofline, "extra": extra, "dtype": "bf16", "cpu": cpu}


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
    ring_ms = region_launch_ms(torch, args, lambda: dc.dc_reduce_scatter_ring(W, 0, x, w.ld, sh, ld_sh, M, 1), 1)
    ring_gbs = rs_b / (ring_ms / 1e3) / 1e9
    log(f"[bench] rs_ring back to back: {ring_ms:.4f} ms, {ring_gbs:.1f} GB/s")
    roofline = {"bound": "hbm", "achieved": round(ring_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ring_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile("schedules_w8", w.name),
                "kernel": "k_rs_ring", "launch_ms_avg": round(ring_ms, 4), "timing": REGION_TIMING,
                "per_launch_events": per_launch_events(gbs["rs_ring"], float(kern[1])),
                "bytes_per_launch_avg": rs_b, "bytes_per_launch": [rs_b]}
    tmp = torch.empty((W, w.ld), dtype=torch.int16, device=dev)
    add_mix_reference(roofline, best_reference(x, w.ld // 8, W, tmp, w.ld // 8, 1, M // 8),
                      f"read {W} rows, write 1")
    del tmp
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
    torch.cuda.synchronize()
    cpu = None
    if not args.no_cpu_baseline:
        cpu, extra["cpu_oracle_all_threads"], extra["parity"] = schedules_oracle(w, sh, x, ld_sh)
    del x
    return {"name": w.name, "ms": ms_step, "value": sum(byts) / (ms_step / 1e3) / 1e9,
            "roofline": roofline, "extra": extra, "dtype": "bf16", "cpu": cpu}


def schedules_oracle(w, sh_ring, x, ld_sh):
    """The ring-order reduce-scatter shards against the oracle on every
    element, and the oracle's ring-order reduce-scatter timing (one thread
    on a quarter of the shard columns, all threads on all, medians of 3)."""
    import concurrent.futures
    import oracle
    from oracle import columns as OC
    W, M, dtype = w.W, w.M, w.dtype
    L = M // W
    hin = OC.host_rows(dtype, w.value_seed, 0, w.scale, W, 0, M)
    hin = np.ascontiguousarray(hin[:, :M])
    k = OC.nthreads()
    blk = 1 << 18

    def ring_cols(cols, threads):
        # shard s column k folds column s*L + k of every row in ring order;
        # blocks of k run the oracle's ring reduce-scatter on the W-row slab of
        # those columns of every shard (the same per-column operands)
        out = np.zeros((W, cols), hin.dtype)

        def run(s0):
            m = min(blk, cols - s0)
            sub = np.empty((W, W * m), hin.dtype)
            for q in range(W):
                sub[:, q * m:(q + 1) * m] = hin[:, q * L + s0:q * L + s0 + m]
            o = np.zeros((W, m), hin.dtype)
            oracle.reduce_scatter_ring(W, dtype, sub, o, W * m, 1)
            out[:, s0:s0 + m] = o
        with concurrent.futures.ThreadPoolExecutor(threads) as p:
            list(p.map(run, range(0, cols, blk)))
        return out
    tp, want = _median3(lambda: ring_cols(L, k))
    t1, _ = _median3(lambda: ring_cols(L // 4, 1))
    got = _gpu_cols(sh_ring, 0, L, dtype)
    bad = int(np.count_nonzero(got != want))
    parity = {"columns_checked": int(L), "elements_checked": int(got.size), "mismatches": bad,
              "outputs": "ring-order reduce-scatter shards"}
    rs_b = W * M * 2 + M * 2
    base = {"value": round(rs_b / 4 / t1 / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the ring-order reduce-scatter over the first quarter of every shard, "
                      f"oracle.c on one thread, median of 3 runs of {t1:.2f} s"}
    allc = {"value": round(rs_b / tp / 1e9, 4), "unit": "GB/s", "threads": k,
            "seconds_median": round(tp, 3), "sample": "the whole ring-order reduce-scatter"}
    log(f"[bench] schedules parity: {bad} mismatches; cpu oracle one thread {base['value']} GB/s")
    return base, allc, parity


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
    ex.fetch_metadata()
    flat = ex.d_flat[:w.P].cpu().numpy()
    plans = []
    for bk in w.buckets:
        t = dc.tasks_array([(k.offset, k.numel, k.param, k.comm) for k in bk.tasks])
        pieces, seg = dc.dc_plan_relayout(W, t, len(t), flat, ex.h_psize, w.P)
        tiles = dc.dc_plan_relayout_tiles(0, bk.col, bk.numel, pieces, len(pieces), int(seg[-1]))
        plans.append((torch.from_numpy(pieces.view(np.uint8).copy()).to(dev), len(pieces), seg,
                      torch.from_numpy(tiles).to(dev), len(tiles)))
    maxn = max(int(p[2][-1]) for p in plans)
    maxseg = max(int(max(p[2][1:] - p[2][:-1])) for p in plans)
    ld_r, ld_s = wl.round_up(maxn, 64), wl.round_up(maxseg, 64)
    relaid = torch.empty((W, ld_r), dtype=torch.int16, device=dev)
    shards = torch.empty((W, ld_s), dtype=torch.int16, device=dev)
    nb = len(w.buckets)
    # per bucket: W rows read and written, the piece table, and with a tile
    # plan 8 bytes per tile record
    rl_b = [2 * W * int(p[2][-1]) * b + 32 * p[1] + (0 if args.searched else 8 * p[4]) for p in plans]
    rs_b = [W * int(p[2][-1]) * b + int(p[2][-1]) * b for p in plans]

    def step(tm=None):
        for k, bk in enumerate(w.buckets):
            d_pieces, npc, seg, d_tiles, ntiles = plans[k]
            if tm: tm.ev[2 * k][0].record()
            if args.searched:
                dc.dc_relayout_bucket(W, 0, x, ld, relaid, ld_r, bk.col, bk.numel, d_pieces, npc,
                                      int(seg[-1]))
            else:
                dc.dc_relayout_bucket_planned(W, 0, x, ld, relaid, ld_r, bk.col, bk.numel, d_pieces,
                                              npc, int(seg[-1]), d_tiles, ntiles)
            if tm: tm.ev[2 * k][1].record(); tm.ev[2 * k + 1][0].record()
            dc.dc_reduce_scatter_v(W, 0, relaid, ld_r, shards, ld_s, seg, w.pre_div)
            if tm: tm.ev[2 * k + 1][1].record()

    ms_step, kern_all = run_timed(torch, args, step, 2 * nb)
    kern = kern_all.mean(axis=0)
    rl_gbs = sum(rl_b) / (kern[0::2].sum() / 1e3) / 1e9
    ev_rs_gbs = sum(rs_b) / (kern[1::2].sum() / 1e3) / 1e9

    def rs_only():
        for k in range(nb):
            dc.dc_reduce_scatter_v(W, 0, relaid, ld_r, shards, ld_s, plans[k][2], w.pre_div)

    rs_ms = region_launch_ms(torch, args, rs_only, 1)
    rs_gbs = sum(rs_b) / (rs_ms / 1e3) / 1e9

    def rl_only():
        for k, bk in enumerate(w.buckets):
            d_pieces, npc, seg, d_tiles, ntiles = plans[k]
            if args.searched:
                dc.dc_relayout_bucket(W, 0, x, ld, relaid, ld_r, bk.col, bk.numel, d_pieces, npc,
                                      int(seg[-1]))
            else:
                dc.dc_relayout_bucket_planned(W, 0, x, ld, relaid, ld_r, bk.col, bk.numel, d_pieces,
                                              npc, int(seg[-1]), d_tiles, ntiles)

    ev_rl_gbs = rl_gbs
    rl_ms = region_launch_ms(torch, args, rl_only, 1)
    rl_gbs = sum(rl_b) / (rl_ms / 1e3) / 1e9
    log(f"[bench] relayout + reduce-scatter-v: step {ms_step:.3f} ms; relayout {rl_gbs:.1f} GB/s back to "
        f"back ({rl_ms:.3f} ms), {ev_rl_gbs:.1f} with events; reduce-scatter-v {rs_gbs:.1f} GB/s back to "
        f"back ({rs_ms:.3f} ms), {ev_rs_gbs:.1f} GB/s with events ({kern[1::2].sum():.3f} ms)")
    roofline = {"bound": "hbm", "achieved": round(rs_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(rs_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile("relayout_rs_w8", w.name), "kernel": "k_rs_v",
                "launch_ms_avg": round(rs_ms / nb, 4), "timing": REGION_TIMING,
                "per_launch_events": per_launch_events(ev_rs_gbs, float(kern[1::2].mean())),
                "bytes_per_launch_avg": int(np.mean(rs_b)),
                "bytes_per_launch": [int(b) for b in rs_b]}
    extra = {"relayout": ("searched: each tile looks up its pieces" if args.searched else
                          "planned: per-bucket tile plans built once on the host"),
             "relayout_gbs": round(rl_gbs, 1), "relayout_ms": round(rl_ms, 4),
             "reduce_scatter_v_ms": round(rs_ms, 4),
             "relayout_roofline": {
                 "kernel": "k_relayout" if args.searched else "k_relayout_planned", "bound": "hbm",
                 "achieved": round(rl_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(rl_gbs / HBM_PEAK_GBS, 4), "launch_ms_avg": round(rl_ms / nb, 4),
                 "timing": REGION_TIMING,
                 "per_launch_events": per_launch_events(ev_rl_gbs, float(kern[0::2].mean())),
                 "bytes_per_launch": [int(b) for b in rl_b],
                 "traffic": None if args.searched else traffic_from_profile("relayout_rs_relayout", w.name),
                 "what": "the relayouts, the step's larger share of time, timed back to back"}}
    # references at the largest relaid bucket: reduce-scatter-v reads W rows and
    # writes one row's worth; the relayout reads and writes all W rows (the
    # input slab is not used after the timed steps)
    nvec = maxn // 8
    add_mix_reference(roofline, best_reference(relaid, ld_r // 8, W, x, ld // 8, 1, nvec),
                      f"read {W} rows, write 1")
    rl_ref, rl_shape = best_reference(x, ld // 8, W, relaid, ld_r // 8, W, nvec)
    extra["relayout_access_mix_reference_gbs"] = round(rl_ref, 1)
    extra["relayout_frac_of_access_mix_reference"] = round(rl_gbs / rl_ref, 4)
    extra["relayout_access_mix_reference"] = f"read {W} rows, write {W}, xor only, at {rl_shape}"
    return {"name": w.name, "ms": ms_step, "value": (sum(rl_b) + sum(rs_b)) / (ms_step / 1e3) / 1e9,
            "roofline": roofline, "extra": extra, "dtype": "bf16", "cpu": None}


# ---------------------------------------------------------------------------
# Host and reference figures
# ---------------------------------------------------------------------------

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
    """Host facts next to the figures: CPU model, threads, sockets, memory."""
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
    return info


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

FLUSH_WORKLOADS = {"owner_w8": ("owner_flush_w8", "owner"), "allreduce_w8": ("owner_flush_w8", "allreduce"),
                   "zero2_w8": ("owner_flush_w8", "zero2"),
                   "layered_w8": ("owner_flush_w8_layered", "owner"),
                   "layered_allreduce_w8": ("owner_flush_w8_layered", "allreduce"),
                   "mixed": ("mixed_flush_w16", "owner"), "zero2_mixed": ("mixed_flush_w16", "zero2"),
                   "tiny": ("tiny_flush", "owner")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="owner_w8",
                    choices=list(FLUSH_WORKLOADS) + ["deferred", "rs_ag", "schedules_w8",
                                                     "relayout_rs_w8", "fused_w8", "fused_mixed"])
    ap.add_argument("--ga", type=int, default=8)
    ap.add_argument("--fused", action="store_true",
                    help="deferred workload: report the step with the last accumulate fused into "
                         "the reduce as the line's value")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle: no parity check and no CPU baseline")
    ap.add_argument("--no-deferred", action="store_true",
                    help="headline run: leave out the deferred-reduce step in detail.deferred")
    ap.add_argument("--searched", action="store_true",
                    help="flush, fused and relayout workloads: run without tile plans (each "
                         "tile searches the task or piece table) instead of with the per-bucket "
                         "tile plans")
    ap.add_argument("--load-sample-s", type=float, default=1.5,
                    help="flush workloads: seconds of steps run while rocm-smi samples the GPU's "
                         "clocks and power (0: no sample, e.g. under a profiler)")
    ap.add_argument("--bucket-numel", type=int, default=0,
                    help="flush workloads but tiny: bucket capacity in elements (default: the "
                         "workload's 52,428,800); the same gradient, packed into buckets of "
                         "this size")
    ap.add_argument("--probe", action="store_true",
                    help="flush workloads: print the probe line of each of the first 20 flushes "
                         "(the executor's reduce_probe), as they are issued")
    args = ap.parse_args()
    if args.bucket_numel and (args.workload not in FLUSH_WORKLOADS or args.workload == "tiny"
                              or args.bucket_numel < 1):
        print("--bucket-numel takes a positive size and applies to the 402.8M and mixed flush "
              "workloads only", file=sys.stderr)
        sys.exit(2)
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
    parity_bad = 0
    if args.workload in FLUSH_WORKLOADS:
        fn, mode = FLUSH_WORKLOADS[args.workload]
        w = getattr(wl, fn)(**({"capacity": args.bucket_numel} if args.bucket_numel else {}))
        r = bench_flush(args, w, mode)
        ms, value, roof, extra = r["ms"], r["value"], r["roofline"], r["extra"]
        if not extra.get("device_plans", {}).get("records_equal_host", True):
            parity_bad += 1
        name, dtype = w.name, wl.DTYPE_NAME[w.dtype]
        metric = METRIC.format(W=w.W)
        config = {"workload": name, "W": w.W, "elements": w.total, "buckets": len(w.buckets),
                  "tasks_per_bucket": [len(b.tasks) for b in w.buckets],
                  "bucket_capacity": w.capacity,
                  "mode": {"owner": "reduce_to_owner", "allreduce": "allreduce", "zero2": "zero2"}[mode],
                  "pre_div": w.pre_div, "step": "owner map + every bucket flush",
                  "flush": ("searched: each tile looks up its tasks" if args.searched else
                            "planned: per-bucket tile plans built once at init on the host"),
                  "step_bytes": r["step_bytes"]}
        if not args.no_cpu_baseline:
            # every column when the slab is a few GB (the 402.8M W=8 workloads),
            # else the first two buckets
            whole = w.W * w.total * w.elem_bytes() < 16e9
            parity, cpu, allc = flush_oracle(w, r["y"], mode, init="zero",
                                             max_buckets=None if whole else 2)
            extra["parity"] = parity
            extra["cpu_oracle_all_threads"] = allc
            parity_bad += parity["mismatches"]
        del r
        torch.cuda.empty_cache()
        if args.workload == "owner_w8" and not args.no_deferred:
            d = bench_deferred(args, args.ga, check=not args.no_cpu_baseline)
            extra["deferred"] = d
            parity_bad += d.get("parity", {}).get("mismatches", 0)
    elif args.workload in ("fused_w8", "fused_mixed"):
        w = wl.owner_flush_w8() if args.workload == "fused_w8" else wl.mixed_flush_w16()
        r = bench_flush_buffers(args, w)
        ms, value, roof, extra = r["ms"], r["value"], r["roofline"], r["extra"]
        name, dtype = w.name, wl.DTYPE_NAME[w.dtype]
        metric = "fused copy-in/copy-out " + METRIC.format(W=w.W)
        config = {"workload": name, "W": w.W, "elements": w.total, "buckets": len(w.buckets),
                  "mode": "copy-in/copy-out fused flush into per-rank grad buffers",
                  "flush": ("searched: each tile looks up its tasks" if args.searched else
                            "planned: per-bucket tile plans built once at registration"),
                  "pre_div": w.pre_div, "step": "owner map + every bucket flush",
                  "step_bytes": r["step_bytes"]}
    elif args.workload == "deferred":
        d = bench_deferred(args, args.ga, check=not args.no_cpu_baseline)
        key = "fused" if args.fused else "unfused"
        name, dtype = d["workload"], "f32"
        ms, value, roof = d[key]["ms_per_step"], d[key]["value"], d[key]["roofline"]
        cpu = d.pop("cpu_baseline", None)
        extra = d
        parity_bad += d.get("parity", {}).get("mismatches", 0)
        metric = ("gradient-accumulation step GB/s (bytes read+written/time; K accumulates + one "
                  "cross-replica reduce) and % of MI355X HBM peak, W=4")
        config = {"workload": name, "W": 4, "K": args.ga, "step": d[key]["step"]}
    else:
        fns = {"relayout_rs_w8": bench_relayout_rs, "schedules_w8": bench_schedules, "rs_ag": bench_rs_ag}
        r = fns[args.workload](args)
        name, ms, value, roof, extra, dtype, cpu = (r["name"], r["ms"], r["value"], r["roofline"],
                                                   r["extra"], r["dtype"], r["cpu"])
        parity_bad += extra.get("parity", {}).get("mismatches", 0)
        metric, step = {
            "relayout_rs_w8": ("relayout + reduce-scatter-v GB/s (bytes read+written/time) and % of "
                               "MI355X HBM peak, W=8", "relayout by destination + reduce-scatter-v "
                                                       "of every bucket"),
            "schedules_w8": ("collective-schedule GB/s (bytes read+written/time) and % of MI355X HBM "
                             "peak, W=8", "reduce-scatter rank + ring order, all-gather "
                                          "ring/bidir/rd step executors"),
            "rs_ag": ("reduce-scatter + all-gather GB/s (bytes read+written/time) and % of MI355X "
                      "HBM peak, W=8", "reduce-scatter + all-gather rank + all-gather ring")}[args.workload]
        config = {"workload": name, "W": 8, "step": step}
    roof["copy_reference_gbs"] = calib
    line = {"metric": metric,
            "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic (seeded SplitMix64 Irwin-Hall gradients, random-init shapes)",
            "config": config, "roofline": roof, "cpu_baseline": cpu, "detail": extra,
            "system": system_info()}
    print(json.dumps(line), flush=True)
    if parity_bad:
        log(f"[bench] PARITY FAILURE: {parity_bad} output elements differ from the oracle (or the "
            f"device-built plans from the host's)")
        sys.exit(PARITY_EXIT)


if __name__ == "__main__":
    main()
