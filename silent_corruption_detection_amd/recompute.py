"""Recompute audit for activation checkpointing.

AEGIS review page ("Safeguarding LLM Training at Scale"), section "core
method", item 4: training already recomputes activations to save memory, and
a deterministic recomputation must reproduce the original bit for bit, so
fingerprints of the original and of the recomputed result are compared and
any difference is a confirmed fault (in either run's compute path, or in the
saved input the recomputation starts from).  Placing the fingerprint at the
end of a recomputed segment covers the whole segment with one comparison.

`RecomputeAudit.wrap(fn, k)` returns the function to hand to
`torch.utils.checkpoint.checkpoint` for segment k.  The first call of segment
k in a step (the forward pass) stores the row of its output; the second (the
recomputation in backward) scans the recomputed output, compares it with the
stored row on the device and counts a difference.  Every scan is
`sdc_fingerprint_tensor`: asynchronous on the current stream, no plan upload,
no host synchronisation.  `result()` is the step's one synchronisation.

The recomputation must run the whole segment: use `use_reentrant=True`, or
make the non-reentrant `checkpoint` calls of the forward pass inside
`torch.utils.checkpoint.set_checkpoint_early_stop(False)` (early stopping ends
the recomputation as soon as the saved tensors are rebuilt, before the
segment's output exists; the setting is read when `checkpoint` is called).
A segment that was not recomputed is reported in `result()["not_recomputed"]`.
"""
import torch

from . import (COL_ALL, rows_numpy, sdc_fingerprint_diff, sdc_fingerprint_tensor,
               sdc_tensor_ws_bytes)


class RecomputeAudit:
    def __init__(self, n_segments, device="cuda", col_mask=COL_ALL):
        if n_segments < 1:
            raise ValueError("need at least one segment")
        self.n = n_segments
        self.col_mask = col_mask
        dev = torch.device(device)
        self.original = torch.zeros((n_segments, 4), dtype=torch.int64, device=dev)
        self.recomputed = torch.zeros_like(self.original)
        self.mismatch = torch.zeros(n_segments, dtype=torch.int32, device=dev)
        self.calls = [0] * n_segments
        self._ws = {}  # one scan workspace per stream: calls on a stream run in order

    def _workspace(self, t):
        st = torch.cuda.current_stream(t.device)
        need = sdc_tensor_ws_bytes(t)
        ws = self._ws.get(st.cuda_stream)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 1 << 16), dtype=torch.uint8, device=t.device)
            self._ws[st.cuda_stream] = ws
        return ws

    def begin_step(self):
        """Start a step: clears the counters (a fill kernel on the current stream)."""
        self.mismatch.zero_()
        self.calls = [0] * self.n

    def wrap(self, fn, k):
        """fn(*args) -> tensor, as segment k of a checkpointed model."""
        if not 0 <= k < self.n:
            raise IndexError(f"segment {k} out of range 0..{self.n - 1}")

        def run(*args, **kwargs):
            out = fn(*args, **kwargs)
            self.record(k, out)
            return out
        return run

    def record(self, k, out):
        if not isinstance(out, torch.Tensor):
            raise TypeError(f"segment {k} must return one tensor, got {type(out).__name__}")
        c = self.calls[k]
        t = out.detach()
        if c == 0:
            sdc_fingerprint_tensor(t, out=self.original[k:k + 1], ws=self._workspace(t))
        elif c == 1:
            sdc_fingerprint_tensor(t, out=self.recomputed[k:k + 1], ref=self.original[k:k + 1],
                                   mismatch=self.mismatch[k:k + 1], col_mask=self.col_mask,
                                   ws=self._workspace(t))
        else:
            raise RuntimeError(f"segment {k} ran {c + 1} times in one step (call begin_step())")
        self.calls[k] = c + 1

    def result(self):
        """After backward (synchronises): segments whose recomputation differed
        from the original, segments not recomputed, and for each mismatch the
        single-bit-flip localisation of the two rows when there is one."""
        mism = self.mismatch.cpu().tolist()
        bad = [k for k in range(self.n) if mism[k]]
        hints = {}
        if bad:
            d = sdc_fingerprint_diff(self.original, self.recomputed, col_mask=self.col_mask)
            hints = {k: h for k, h in zip(d["indices"], d["hints"]) if k in bad}
        return {"mismatched": bad,
                "not_recomputed": [k for k in range(self.n) if self.calls[k] == 1],
                "not_run": [k for k in range(self.n) if self.calls[k] == 0],
                "hints": hints}

    def rows(self):
        """Host uint64 copies of the original and recomputed rows."""
        return rows_numpy(self.original), rows_numpy(self.recomputed)
