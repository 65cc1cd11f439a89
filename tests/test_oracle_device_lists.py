"""The streaming oracle driver (oracle/device_lists.py) gives the oracle's own
rows, tensor by tensor, for lists with missing, empty and strided tensors of
several types (host tensors here; on a GPU the same code copies through
pinned buffers)."""
import numpy as np
import torch

import oracle as O
from oracle.device_lists import rows_of_device_tensors


def test_streamed_rows_are_the_oracles_rows():
    g = torch.Generator().manual_seed(3)
    ts = [torch.randn(1000, generator=g), None, torch.empty(0, dtype=torch.float16),
          torch.randn(37, 5, generator=g).to(torch.bfloat16).t(),
          torch.randint(-100, 100, (4097,), generator=g, dtype=torch.int16),
          torch.randn(3, generator=g, dtype=torch.float64)]
    rows, st = rows_of_device_tensors(ts, threads=3, inflight_bytes=5000)
    codes = [O.F32, None, O.F16, O.BF16, O.U16, O.F64]
    for k, (t, c) in enumerate(zip(ts, codes)):
        if t is None or t.numel() == 0:
            assert rows[k].tolist() == [0, 0, 0, 0]
        else:
            want = O.fingerprint(t.contiguous().reshape(-1).view(torch.uint8).numpy(), c)
            assert rows[k].tolist() == list(want), k
    assert st["bytes"] == 4000 + 185 * 2 + 4097 * 2 + 24
    assert st["elements"] == 1000 + 185 + 4097 + 3
    assert st["threads"] == 3 and st["wall_s"] >= st["max_call_s"] >= 0
