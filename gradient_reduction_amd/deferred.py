"""Gradient accumulation with the data-parallel reduce deferred to update().

MaxText PR "Defer the data-parallel gradient all-reduce to update() under
gradient accumulation": each replica accumulates its own micro-batch
gradients locally (What), and one cross-replica reduce runs at update() on the
accumulated sums instead of one per micro-batch; the accumulator lives across
the micro-batches of a step and can be saved and restored mid-step
(What else had to change, accumulator lifetime).

W replicas are the rows of [W, ld] fp32 slabs on one GPU.  Marshalling only:
every step runs in libdc.so (dc_accumulate, dc_deferred_reduce,
dc_accumulate_reduce); torch supplies the memory and the stream.
"""
from . import dc


class DeferredReducer:
    def __init__(self, W: int, M: int, ld: int = 0, device: str = "cuda"):
        """W replicas of M fp32 gradient elements each; the accumulator is a
        [W, ld] slab (ld defaults to M rounded up to 64 elements)."""
        import torch
        self.torch = torch
        self.W, self.M = W, M
        self.ld = ld if ld else max(64, -(-M // 64) * 64)
        if self.ld < M:
            raise ValueError(f"ld={self.ld} < M={M}")
        self.acc = torch.empty((W, self.ld), dtype=torch.float32, device=device)
        self.micro_batches = 0

    def accumulate(self, x, ld_x: int, stream=None) -> None:
        """Add one micro-batch: acc[r] += x[r] on every replica row (the first
        micro-batch of a step starts from +0)."""
        dc.dc_accumulate(self.W, x, ld_x, self.acc, self.ld, self.M, 1 if self.micro_batches == 0 else 0,
                         stream)
        self.micro_batches += 1

    def reduce(self, out, ld_out: int, out_rows: int = 1, last=None, ld_last: int = 0,
               keep_acc: bool = False, stream=None) -> None:
        """update(): the cross-replica fold of the accumulators into
        out[0..out_rows) (1: one reduced copy, W: every replica gets it).
        With `last`, that final micro-batch is accumulated in the same pass
        (dc_accumulate_reduce); keep_acc also writes it to the accumulator.
        The next accumulate() starts a new step."""
        if last is None:
            if self.micro_batches == 0:
                raise RuntimeError("reduce() before any accumulate() in this step")
            dc.dc_deferred_reduce(self.W, self.acc, self.ld, out, ld_out, self.M, out_rows, stream)
        else:
            dc.dc_accumulate_reduce(self.W, last, ld_last, self.acc, self.ld,
                                    1 if self.micro_batches == 0 else 0, 1 if keep_acc else 0, out,
                                    ld_out, out_rows, self.M, stream)
        self.micro_batches = 0

    def state_dict(self) -> dict:
        """The accumulator's state mid-step: a copy of the slab's M columns
        and the micro-batch count."""
        return {"acc": self.acc[:, :self.M].clone(), "micro_batches": self.micro_batches}

    def load_state_dict(self, state: dict) -> None:
        acc = state["acc"]
        if tuple(acc.shape) != (self.W, self.M):
            raise ValueError(f"accumulator of shape {tuple(acc.shape)}, expected {(self.W, self.M)}")
        self.acc[:, :self.M].copy_(acc)
        self.micro_batches = int(state["micro_batches"])
