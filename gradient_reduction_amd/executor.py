"""ZeRO-1 (and ZeRO-2) bucket-flush executor over one GPU's [W, M] gradient slab.

DeepSpeed issue "[REQUEST] DeepCompile ZeRO-1: reduce-to-owner instead of
AllReduce": at init the owner map is built from the partition lists and the
qualifying ratio is reported; every bucket flush then reduces each task to its
owner (reduce_to_owner on) or to every rank (off, the default), and the probe
reports one line per flush for the first 20 flushes (reduce_probe).  With
zero2=True every element goes to the rank whose partition holds it (the
issue's ZeRO-2 follow-up); the probe describes the ZeRO-1 paths only.

register_buffers + flush_buffers run the flush with copy-in and copy-out
fused in: each rank's gradient is read from its own buffer and the sum lands
in the grad buffers of the ranks that keep one, with no bucket in between.

plan() builds each bucket's flush plan once on the host (dc_plan_flush: the
tasks each tile of the flush grid overlaps and, for a tile inside one task,
the rows its sums go to), or on the device (dc_plan_flush_device, the same
records); flush() then launches dc_flush_bucket_planned, the same sums with
no per-tile search.

torch supplies device memory and the stream; every step runs in libdc.so.
"""
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import dc

PROBE_FLUSHES = 20


@dataclass
class BucketSpec:
    col: int                                  # first slab column
    numel: int
    tasks: Sequence[Tuple[int, int, int, int]]  # (offset, numel, param, comm)


class Zero1FlushExecutor:
    def __init__(self, W: int, dtype: int, numel: Sequence[int], group_begin: Sequence[int],
                 group_parts: Sequence[int], group_comm_size: Sequence[int],
                 group_rank_to_global: Sequence[Sequence[int]], comms: Sequence[Tuple[int, int]],
                 buckets: Sequence[BucketSpec], pre_div: int, reduce_to_owner: bool = False,
                 reduce_probe: bool = False, device: str = "cuda", log=print,
                 zero2: bool = False):
        import torch
        self.torch = torch
        self.W, self.dtype, self.pre_div = W, dtype, pre_div
        self.reduce_to_owner, self.reduce_probe = reduce_to_owner, reduce_probe
        self.zero2 = zero2
        self.log = log
        self.P = len(numel)
        self.G = len(group_parts)
        self.group_begin = list(group_begin)
        self.group_parts = list(group_parts)
        self.group_comm_size = list(group_comm_size)
        self.group_rank_to_global = np.asarray(group_rank_to_global, np.int32).reshape(self.G, W)
        self.comms = dc.comms_array(comms)
        self.buckets = list(buckets)
        self.flushes = 0
        dev = torch.device(device)
        self.pids_capacity = self.P + sum(p - 1 for p in self.group_parts)
        self.d_numel = torch.tensor(list(numel), dtype=torch.int64, device=dev)
        self.d_flat = torch.empty(max(self.P, 1), dtype=torch.int64, device=dev)
        self.d_part_size = torch.empty(self.G, dtype=torch.int64, device=dev)
        self.d_pid_off = torch.empty(self.P + 1, dtype=torch.int32, device=dev)
        self.d_pids = torch.empty(max(self.pids_capacity, 1), dtype=torch.int32, device=dev)
        self.d_owner = torch.empty(max(self.P, 1), dtype=torch.int32, device=dev)
        self.d_counts = torch.empty(2 * self.G, dtype=torch.int32, device=dev)
        # one device task table for all buckets, bucket b at rows [t_begin[b], t_begin[b+1])
        self.h_tasks = [dc.tasks_array(b.tasks) for b in self.buckets]
        for b, t in zip(self.buckets, self.h_tasks):
            dc.dc_validate_tasks(W, t, len(t), b.numel, self.P, self.comms, len(self.comms))
        self.t_begin = np.concatenate([[0], np.cumsum([len(t) for t in self.h_tasks])]).astype(int)
        allt = np.concatenate(self.h_tasks) if self.h_tasks else np.zeros(0, dc.TASK_DTYPE)
        raw = torch.from_numpy(allt.view(np.uint8).copy())
        self.d_tasks = raw.to(dev) if len(allt) else torch.empty(32, dtype=torch.uint8, device=dev)
        self.h_owner: Optional[np.ndarray] = None
        self.d_tiles = None        # flush plans (plan()), one table for all buckets
        self.tile_begin = None
        self.root_tiles = None
        # ZeRO-2: the partition size of each param's group, 0 for groups on
        # another communicator (they keep AllReduce), from dc_param_part_size
        self.d_psize = torch.zeros(max(self.P, 1), dtype=torch.int64, device=dev)
        self._h_psize: Optional[np.ndarray] = None

    def build_owner_map(self, stream=None) -> None:
        """Partition lists and owner map on the device (no host
        synchronization); in ZeRO-2 mode also every param's partition size."""
        dc.dc_partition_ids(self.W, self.P, self.d_numel, self.G, self.group_begin,
                            self.group_parts, self.d_flat, self.d_part_size, self.d_pid_off,
                            self.d_pids, self.pids_capacity, stream)
        dc.dc_build_owner_map(self.W, self.P, self.d_pid_off, self.d_pids, self.pids_capacity,
                              self.G, self.group_begin, self.group_comm_size,
                              self.group_rank_to_global, self.d_owner, self.d_counts, stream)
        if self.zero2:
            dc.dc_param_part_size(self.W, self.P, self.G, self.group_begin, self.group_comm_size,
                                  self.group_rank_to_global, self.d_part_size, self.d_psize,
                                  stream)

    def fetch_metadata(self) -> None:
        """Copy the owner map and partition lists to the host (synchronizes);
        the probe and the ratio report use them."""
        self.h_owner = self.d_owner[:self.P].cpu().numpy()
        self.h_pid_off = self.d_pid_off.cpu().numpy()
        self.h_pids = self.d_pids[:int(self.h_pid_off[-1])].cpu().numpy()
        self.h_counts = self.d_counts.cpu().numpy()
        self._h_psize = self.d_psize[:self.P].cpu().numpy()

    @property
    def h_psize(self) -> np.ndarray:
        """Host copy of every param's ZeRO-2 partition size (fetched, with a
        synchronization, on first use after build_owner_map)."""
        if self._h_psize is None:
            self._h_psize = self.d_psize[:self.P].cpu().numpy()
        return self._h_psize

    def ratio_line(self) -> str:
        owners = int(self.h_counts[0::2].sum())
        return f"DeepCompile reduce_to_owner: {owners}/{self.P} gradients reduce to one rank"

    def task_table(self, b: int) -> int:
        return self.d_tasks.data_ptr() + 32 * int(self.t_begin[b])

    def plan(self, on_device: bool = False, stream=None) -> None:
        """Plan every bucket's flush on the host (dc_plan_flush: per tile, the
        tasks it overlaps and, for a tile inside one task, its rows), from
        the owner map (or the ZeRO-2 partition sizes), and keep the plans on
        the device; flush() then takes the planned path.  Synchronizes: call
        it at init, after build_owner_map, not while a graph is captured.
        on_device: the same plans from dc_plan_flush_device, straight from
        the device task table and owner map (no host copies); one
        synchronization reads back the root counts, which pick each planned
        launch's shape."""
        if on_device:
            self._plan_on_device(stream)
            return
        torch = self.torch
        if self.h_owner is None:
            self.fetch_metadata()
        flat = self.d_flat[:self.P].cpu().numpy() if self.zero2 else None
        recs, self.root_tiles = [], []
        for b, bk in enumerate(self.buckets):
            t = self.h_tasks[b]
            if self.zero2:
                tiles, roots = dc.dc_plan_flush(self.W, self.dtype, bk.col, bk.numel, t, len(t), None,
                                                flat, self.h_psize, self.P, self.comms,
                                                len(self.comms))
            else:
                owner = self.h_owner if self.reduce_to_owner else None
                tiles, roots = dc.dc_plan_flush(self.W, self.dtype, bk.col, bk.numel, t, len(t),
                                                owner, None, None, self.P, self.comms,
                                                len(self.comms))
            recs.append(tiles)
            self.root_tiles.append(roots)
        self.tile_begin = np.concatenate([[0], np.cumsum([len(r) for r in recs])]).astype(int)
        allr = np.concatenate(recs) if recs else np.zeros(0, dc.TILE_DTYPE)
        raw = torch.from_numpy(allr.view(np.uint8).copy()) if len(allr) else torch.zeros(16, dtype=torch.uint8)
        self.d_tiles = raw.to(self.d_tasks.device)

    def _plan_on_device(self, stream=None) -> None:
        torch = self.torch
        dev = self.d_tasks.device
        counts = [dc.dc_plan_flush_device(self.W, self.dtype, bk.col, bk.numel, self.task_table(b),
                                          len(bk.tasks), None, None, None, self.P, self.comms,
                                          len(self.comms), None, 0)
                  for b, bk in enumerate(self.buckets)]
        self.tile_begin = np.concatenate([[0], np.cumsum(counts)]).astype(int)
        self.d_tiles = torch.empty(16 * max(int(self.tile_begin[-1]), 1), dtype=torch.uint8, device=dev)
        roots = torch.empty(max(len(self.buckets), 1), dtype=torch.int64, device=dev)
        if self.zero2:
            owner, flat, psize = None, self.d_flat, self.d_psize
        else:
            owner, flat, psize = (self.d_owner if self.reduce_to_owner else None), None, None
        for b, bk in enumerate(self.buckets):
            dc.dc_plan_flush_device(self.W, self.dtype, bk.col, bk.numel, self.task_table(b),
                                    len(bk.tasks), owner, flat, psize, self.P, self.comms,
                                    len(self.comms), self.d_tiles.data_ptr() + 16 * int(self.tile_begin[b]),
                                    counts[b], roots.data_ptr() + 8 * b, stream)
        torch.cuda.synchronize()
        self.root_tiles = [int(v) for v in roots.cpu().numpy()[:len(self.buckets)]]

    def flush(self, b: int, slab_in, ld_in: int, slab_out, ld_out: int, stream=None) -> None:
        bk = self.buckets[b]
        if self.d_tiles is not None:
            nt = int(self.tile_begin[b + 1] - self.tile_begin[b])
            tp = self.d_tiles.data_ptr() + 16 * int(self.tile_begin[b])
            if self.zero2:
                dc.dc_flush_bucket_planned(self.W, self.dtype, slab_in, ld_in, slab_out, ld_out,
                                           bk.col, bk.numel, self.task_table(b), len(bk.tasks), None,
                                           self.d_flat, self.d_psize, self.P, self.comms,
                                           len(self.comms), self.pre_div, tp, nt,
                                           self.root_tiles[b], stream)
            else:
                owner = self.d_owner if self.reduce_to_owner else None
                dc.dc_flush_bucket_planned(self.W, self.dtype, slab_in, ld_in, slab_out, ld_out,
                                           bk.col, bk.numel, self.task_table(b), len(bk.tasks), owner,
                                           None, None, self.P, self.comms, len(self.comms),
                                           self.pre_div, tp, nt, self.root_tiles[b], stream)
        elif self.zero2:
            dc.dc_flush_bucket_zero2(self.W, self.dtype, slab_in, ld_in, slab_out, ld_out, bk.col,
                                     bk.numel, self.task_table(b), len(bk.tasks), self.d_flat,
                                     self.d_psize, self.P, self.comms, len(self.comms),
                                     self.pre_div, stream)
        else:
            owner = self.d_owner if self.reduce_to_owner else None
            dc.dc_flush_bucket(self.W, self.dtype, slab_in, ld_in, slab_out, ld_out, bk.col,
                               bk.numel, self.task_table(b), len(bk.tasks), owner, self.P,
                               self.comms, len(self.comms), self.pre_div, stream)
        if self.reduce_probe and not self.zero2 and self.flushes < PROBE_FLUSHES:
            self.log(self.probe_line(b, self.flushes))
        self.flushes += 1

    # -- relayout by destination rank + reduce-scatter-v ------------------------

    def plan_relayout(self, planned=True) -> None:
        """The reduce-scatter alternative of the flush ([DS] "Describe
        alternatives"): per bucket, the relayout's pieces and segment starts
        (dc_plan_relayout, from the ZeRO-2 flat offsets and partition sizes:
        build_owner_map must have run in ZeRO-2 mode) and, with planned, its
        tile plan (dc_plan_relayout_tiles on the host, or with
        planned="device" dc_plan_relayout_tiles_device), kept on the device.
        relayout_reduce_scatter() then runs the path.  Synchronizes."""
        torch = self.torch
        if not self.zero2:
            raise ValueError("plan_relayout needs the executor in ZeRO-2 mode (zero2=True)")
        dev = self.d_tasks.device
        flat = self.d_flat[:self.P].cpu().numpy()
        self.rl = []
        for b, bk in enumerate(self.buckets):
            t = self.h_tasks[b]
            pieces, seg = dc.dc_plan_relayout(self.W, t, len(t), flat, self.h_psize, self.P)
            n = int(seg[-1])
            d_pieces = (torch.from_numpy(pieces.view(np.uint8).copy()).to(dev) if len(pieces)
                        else None)
            d_tiles, ntiles = None, 0
            if planned == "device":
                ntiles = dc.dc_plan_relayout_tiles_device(self.dtype, bk.col, bk.numel, None,
                                                          len(pieces), n, None, 0)
                d_tiles = torch.empty(max(ntiles, 1), dtype=torch.int64, device=dev)
                dc.dc_plan_relayout_tiles_device(self.dtype, bk.col, bk.numel, d_pieces, len(pieces),
                                                 n, d_tiles, ntiles)
            elif planned:
                tiles = dc.dc_plan_relayout_tiles(self.dtype, bk.col, bk.numel, pieces, len(pieces), n)
                ntiles = len(tiles)
                d_tiles = torch.from_numpy(tiles).to(dev) if ntiles else None
            self.rl.append((d_pieces, len(pieces), seg, d_tiles, ntiles if planned else -1))
        torch.cuda.synchronize()

    def relayout_sizes(self, b: int) -> Tuple[int, int]:
        """(relaid columns, longest segment) of bucket b: the relaid slab
        needs ld >= the first, the shards ld >= the second."""
        seg = self.rl[b][2]
        return int(seg[-1]), int(max(seg[1:] - seg[:-1])) if len(seg) > 1 else 0

    def relayout_reduce_scatter(self, b: int, slab_in, ld_in: int, relaid, ld_relaid: int, shards,
                                ld_shards: int, stream=None) -> None:
        """Bucket b relaid by destination rank into `relaid` ([W, ld_relaid])
        and reduced by reduce-scatter-v into `shards` ([W, ld_shards]): row q
        of the shards holds partition q's sums, the values the ZeRO-2 flush
        writes to row q."""
        bk = self.buckets[b]
        d_pieces, npieces, seg, d_tiles, ntiles = self.rl[b]
        n = int(seg[-1])
        if ntiles >= 0:
            dc.dc_relayout_bucket_planned(self.W, self.dtype, slab_in, ld_in, relaid, ld_relaid, bk.col,
                                          bk.numel, d_pieces, npieces, n, d_tiles, ntiles, stream)
        else:
            dc.dc_relayout_bucket(self.W, self.dtype, slab_in, ld_in, relaid, ld_relaid, bk.col,
                                  bk.numel, d_pieces, npieces, n, stream)
        dc.dc_reduce_scatter_v(self.W, self.dtype, relaid, ld_relaid, shards, ld_shards, seg,
                               self.pre_div, stream)

    # -- copy-in and copy-out fused into the flush ------------------------------

    def holders(self, b: int) -> np.ndarray:
        """[n_tasks, W] bool for bucket b: rank r keeps a gradient buffer for
        the task's param (dc_holders: its partition holds part of it, in
        every block of a sub-communicator).  These are the ranks the copy-out
        writes and the probe's `kept` counts."""
        if self.h_owner is None:
            self.fetch_metadata()
        t = self.h_tasks[b]
        return dc.dc_holders(self.W, t, len(t), self.P, self.h_pid_off, self.h_pids, self.comms,
                             len(self.comms))

    def register_buffers(self, in_addr: np.ndarray, out_addr: np.ndarray, planned=True) -> None:
        """in_addr, out_addr: [W, P] device addresses of rank r's gradient of
        param p and of its grad buffer (0 = empty buffer).  A task's slice
        starts at its position within its param (the params' tasks in bucket
        order).  Task coordinates are re-laid at 128-byte steps: buffers that
        start on a 128-byte boundary then move as whole vectors with every
        wave's accesses on whole cache lines.  Tables are validated on the
        host and kept on the device; with planned (the default) each bucket's
        tile plan (dc_plan_flush_buffers) is built here too, and flush_buffers
        launches the planned kernel.  planned="device": the same plans from
        dc_plan_flush_buffers_device, built on the device from the uploaded
        task tables."""
        torch = self.torch
        W = self.W
        eb = 2 if self.dtype == dc.DC_BF16 else 4
        step = 128 // eb
        in_addr = np.asarray(in_addr, np.uint64).reshape(W, self.P)
        out_addr = np.asarray(out_addr, np.uint64).reshape(W, self.P)
        seen = np.zeros(self.P, np.int64)
        tasks, ins, outs, self.buf_extent, self.buf_begin = [], [], [], [], [0]
        plans, self.buf_tile_begin = [], [0]
        for b, bk in enumerate(self.buckets):
            pos = 0
            rows = []
            tin = np.zeros((len(bk.tasks), W), np.uint64)
            tout = np.zeros((len(bk.tasks), W), np.uint64)
            for k, (_, numel, param, comm) in enumerate(bk.tasks):
                rows.append((pos, numel, param, comm))
                skip = np.uint64(int(seen[param]) * eb)
                tin[k] = in_addr[:, param] + skip
                tout[k] = np.where(out_addr[:, param] != 0, out_addr[:, param] + skip, 0)
                seen[param] += numel
                pos = -(-(pos + numel) // step) * step
            t = dc.tasks_array(rows)
            extent = int(rows[-1][0] + rows[-1][1]) if rows else 0
            dc.dc_validate_buffer_tasks(W, self.dtype, t, len(t), extent, self.comms,
                                        len(self.comms), tin.ravel(), tout.ravel())
            tasks.append(t)
            ins.append(tin.ravel())
            outs.append(tout.ravel())
            self.buf_extent.append(extent)
            self.buf_begin.append(self.buf_begin[-1] + len(t))
            if planned == "device":
                n = dc.dc_plan_flush_buffers_device(W, self.dtype, extent, None, len(t), self.comms,
                                                    len(self.comms), None, 0)
                self.buf_tile_begin.append(self.buf_tile_begin[-1] + n)
            elif planned:
                pl = dc.dc_plan_flush_buffers(W, self.dtype, extent, t, len(t), self.comms,
                                              len(self.comms))
                plans.append(pl)
                self.buf_tile_begin.append(self.buf_tile_begin[-1] + len(pl))
        dev = self.d_tasks.device
        allt = np.concatenate(tasks) if tasks else np.zeros(0, dc.TASK_DTYPE)
        self.d_btasks = torch.from_numpy(allt.view(np.uint8).copy()).to(dev) if len(allt) else None
        self.d_bin = torch.from_numpy(np.concatenate(ins).view(np.int64)).to(dev)
        self.d_bout = torch.from_numpy(np.concatenate(outs).view(np.int64)).to(dev)
        self.d_btiles = None
        if planned == "device":
            self.d_btiles = torch.empty(16 * max(int(self.buf_tile_begin[-1]), 1), dtype=torch.uint8,
                                        device=dev)
            for b in range(len(self.buckets)):
                n = int(self.buf_tile_begin[b + 1] - self.buf_tile_begin[b])
                k = self.buf_begin[b + 1] - self.buf_begin[b]
                if n == 0:
                    continue
                dc.dc_plan_flush_buffers_device(
                    W, self.dtype, self.buf_extent[b], self.d_btasks.data_ptr() + 32 * self.buf_begin[b],
                    k, self.comms, len(self.comms),
                    self.d_btiles.data_ptr() + 16 * int(self.buf_tile_begin[b]), n)
            torch.cuda.synchronize()   # the plans are ready for a flush on any stream
        elif planned:
            allp = np.concatenate(plans) if plans else np.zeros(0, dc.TILE_DTYPE)
            raw = allp.view(np.uint8).copy() if len(allp) else np.zeros(16, np.uint8)
            self.d_btiles = torch.from_numpy(raw).to(dev)

    def flush_buffers(self, b: int, stream=None) -> None:
        n = len(self.buckets[b].tasks)
        if n == 0:
            return
        t0 = self.buf_begin[b]
        if self.d_btiles is not None:
            p0 = self.buf_tile_begin[b]
            dc.dc_flush_bucket_buffers_planned(
                self.W, self.dtype, self.buf_extent[b], self.d_btasks.data_ptr() + 32 * t0, n,
                self.d_bin.data_ptr() + 8 * t0 * self.W, self.d_bout.data_ptr() + 8 * t0 * self.W,
                self.comms, len(self.comms), self.pre_div, self.d_btiles.data_ptr() + 16 * p0,
                self.buf_tile_begin[b + 1] - p0, stream)
        else:
            dc.dc_flush_bucket_buffers(self.W, self.dtype, self.buf_extent[b],
                                       self.d_btasks.data_ptr() + 32 * t0, n,
                                       self.d_bin.data_ptr() + 8 * t0 * self.W,
                                       self.d_bout.data_ptr() + 8 * t0 * self.W,
                                       self.comms, len(self.comms), self.pre_div, stream)
        self.flushes += 1

    # -- one step as a HIP graph --------------------------------------------------

    def capture_step(self, slab_in=None, ld_in: int = 0, slab_out=None, ld_out: int = 0,
                     fused: bool = False):
        """Record one step (owner map + every bucket flush, or every fused
        flush) as a HIP graph; `graph.replay()` re-issues it with one launch.
        The graph keeps the pointers, sizes and tables given here, so replay
        it on the same buffers.  No call in the step allocates, synchronizes
        or clears memory, so every kernel records as a plain kernel node.
        The probe is not printed from a graph."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        probe, self.reduce_probe = self.reduce_probe, False
        flushes = self.flushes
        try:
            with torch.cuda.graph(g):
                self.build_owner_map()
                for b in range(len(self.buckets)):
                    if fused:
                        self.flush_buffers(b)
                    else:
                        self.flush(b, slab_in, ld_in, slab_out, ld_out)
        finally:
            self.reduce_probe = probe
            self.flushes = flushes
        return g

    def probe(self, b: int):
        if self.h_owner is None:
            self.fetch_metadata()
        t = self.h_tasks[b]
        owner = self.h_owner if self.reduce_to_owner else None
        return dc.dc_probe_flush(self.W, self.dtype, t, len(t), owner, self.P, self.h_pid_off,
                                 self.h_pids, self.comms, len(self.comms), self.pre_div)

    def probe_line(self, b: int, flush_no: int, rank: int = 0) -> str:
        pr = self.probe(b)
        name = "BFloat16" if self.dtype == dc.DC_BF16 else "Float"
        red = pr.reduced_elems
        disc = 100.0 * pr.discarded[rank] / red if red else 0.0
        oe = 100.0 * pr.owner_elems / red if red else 0.0
        return (f"[dc-probe][r{rank}] flushReduceBucket #{flush_no} dtype={name} "
                f"tasks={pr.tasks} reduced_elems={red} kept_elems={pr.kept[rank]} "
                f"discarded={disc:.1f}% pre_div={self.pre_div} owner_tasks={pr.owner_tasks} "
                f"owner_elems={pr.owner_elems} ({oe:.1f}%)")


def from_workload(w, reduce_to_owner: bool, reduce_probe: bool = False, device: str = "cuda",
                  log=print, zero2: bool = False) -> Zero1FlushExecutor:
    """Executor for a synthetic flush workload description (duck-typed: the
    fields of synth.workloads.FlushWorkload)."""
    buckets = [BucketSpec(b.col, b.numel, [(t.offset, t.numel, t.param, t.comm) for t in b.tasks])
               for b in w.buckets]
    comm_sizes = [w.comms[c].size for c in w.group_comm]
    return Zero1FlushExecutor(
        w.W, w.dtype, w.numel, w.group_begin, w.group_parts(), comm_sizes,
        w.group_rank_to_global(), [(c.size, c.stride) for c in w.comms], buckets, w.pre_div,
        reduce_to_owner=reduce_to_owner, reduce_probe=reduce_probe, device=device, log=log,
        zero2=zero2)
