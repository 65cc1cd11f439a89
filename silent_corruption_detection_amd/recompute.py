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
k in a step (the forward pass) stores the rows of its outputs (a tensor, or a
tuple of up to `outputs` tensors); the second (the recomputation in
backward) scans the recomputed outputs, compares them with the stored rows
on the device and counts differences.  Every scan is
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

from . import (COL_ALL, _current_stream_handle, rows_numpy, sdc_fingerprint_diff, sdc_fingerprint_tensor,
               sdc_tensor_ws_bytes)


class RecomputeAudit:
    """Fingerprints of each checkpointed segment's outputs (up to `outputs`
    tensors per segment), stored at forward time and compared on the device
    when backward recomputes them."""

    def __init__(self, n_segments, device="cuda", col_mask=COL_ALL, outputs=1):
        if n_segments < 1 or outputs < 1:
            raise ValueError("need at least one segment and one output per segment")
        self.n = n_segments
        self.outputs = outputs
        self.col_mask = col_mask
        dev = torch.device(device)
        # row k * outputs + j: output j of segment k
        self.original = torch.zeros((n_segments * outputs, 4), dtype=torch.int64, device=dev)
        self.recomputed = torch.zeros_like(self.original)
        self.mismatch = torch.zeros(n_segments, dtype=torch.int32, device=dev)
        # one-row views made once: slicing a view costs about a microsecond,
        # a sixth of a call's host time
        self._original_rows = self.original.split(1)
        self._recomputed_rows = self.recomputed.split(1)
        self._mismatch_at = self.mismatch.split(1)
        self.calls = [0] * n_segments
        self._ws = {}  # one scan workspace per stream: calls on a stream run in order

    def _workspace(self, t):
        # The size is asked for only when t is larger than every tensor the
        # stream's workspace has served: a workspace of at least 64 KiB holds
        # the partial rows of any tensor below the tensor-wide split, and
        # above it the need grows with the size.  (Were one too small, the
        # scan would take a workspace of its own for that call.)
        key = _current_stream_handle(t.device)
        nbytes = t.numel() * t.element_size()
        entry = self._ws.get(key)
        if entry is None or nbytes > entry[1]:
            need = sdc_tensor_ws_bytes(t)
            ws = entry[0] if entry is not None else None
            if ws is None or ws.numel() < need:
                ws = torch.empty(max(need, 1 << 16), dtype=torch.uint8, device=t.device)
            entry = self._ws[key] = (ws, max(nbytes, entry[1] if entry is not None else 0))
        return entry[0]

    def begin_step(self):
        """Start a step: clears the counters (a fill kernel on the current stream)."""
        self.mismatch.zero_()
        self.calls = [0] * self.n

    def wrap(self, fn, k):
        """fn(*args) -> a tensor, or a tuple/list of tensors (None entries are
        skipped), as segment k of a checkpointed model."""
        if not 0 <= k < self.n:
            raise IndexError(f"segment {k} out of range 0..{self.n - 1}")

        def run(*args, **kwargs):
            out = fn(*args, **kwargs)
            self.record(k, out)
            return out
        return run

    def record(self, k, out):
        outs = (out,) if isinstance(out, torch.Tensor) else out
        if not isinstance(outs, (tuple, list)) or len(outs) > self.outputs or not all(
                o is None or isinstance(o, torch.Tensor) for o in outs):
            raise TypeError(f"segment {k} must return a tensor or up to {self.outputs} tensors")
        c = self.calls[k]
        if c > 1:
            raise RuntimeError(f"segment {k} ran {c + 1} times in one step (call begin_step())")
        for j, o in enumerate(outs):
            if o is None:
                continue
            t = o.detach()
            r = k * self.outputs + j
            if c == 0:
                sdc_fingerprint_tensor(t, out=self._original_rows[r], ws=self._workspace(t))
            else:
                sdc_fingerprint_tensor(t, out=self._recomputed_rows[r], ref=self._original_rows[r],
                                       mismatch=self._mismatch_at[k], col_mask=self.col_mask,
                                       ws=self._workspace(t))
        self.calls[k] = c + 1

    def result(self):
        """After backward (synchronises): segments whose recomputation differed
        from the original, segments not recomputed or not run, for each
        mismatched segment the outputs that differ, and the single-bit-flip
        localisation of its first differing output when there is one."""
        mism = self.mismatch.cpu().tolist()
        bad = [k for k in range(self.n) if mism[k]]
        hints, outs = {}, {}
        if bad:
            d = sdc_fingerprint_diff(self.original, self.recomputed, col_mask=self.col_mask)
            for r, h in zip(d["indices"], d["hints"]):
                k, j = divmod(r, self.outputs)
                if k in bad:
                    outs.setdefault(k, []).append(j)
                    hints.setdefault(k, h)
        return {"mismatched": bad,
                "not_recomputed": [k for k in range(self.n) if self.calls[k] == 1],
                "not_run": [k for k in range(self.n) if self.calls[k] == 0],
                "outputs": outs, "hints": hints}

    def rows(self):
        """Host uint64 copies of the original and recomputed rows."""
        return rows_numpy(self.original), rows_numpy(self.recomputed)
