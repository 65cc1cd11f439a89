"""Stored fingerprint tables (silent_corruption_detection_amd/table.py): the
rows and the description of the list survive a save/load round trip bit for
bit, and loading refuses a table that does not belong to the live list.
Rows here are the oracle's (host); the GPU round trip is in
test_gpu_configs.py."""
import numpy as np
import pytest
import torch

import oracle as O
from silent_corruption_detection_amd.table import load_table, save_table

CODE = {torch.float32: O.F32, torch.bfloat16: O.BF16, torch.float16: O.F16}


def rows_of(ts):
    r = np.zeros((len(ts), 4), dtype=np.uint64)
    for k, t in enumerate(ts):
        if t is not None:
            r[k] = O.fingerprint(t.contiguous().view(torch.uint8).numpy(), CODE[t.dtype])
    return torch.from_numpy(r.view(np.int64))


def test_round_trip_and_checks(tmp_path):
    g = torch.Generator().manual_seed(1)
    one = [torch.randn(33, 7, generator=g), torch.randn(5, generator=g).to(torch.bfloat16), None,
           torch.empty(0, dtype=torch.float16)]
    ts = one + [t.clone() if t is not None else None for t in one]   # two replicas
    rows = rows_of(ts)
    rows[4 + 1, 0] = -1          # patterns above 2^63 survive as uint64
    p = str(tmp_path / "table")
    save_table(p, rows, ts, R=2, names=["a", "b", "c", "d"])
    back, meta = load_table(p, tensors=ts)
    assert torch.equal(back, rows) and back.dtype == torch.int64
    assert meta["R"] == 2 and meta["T"] == 4 and [d["name"] for d in meta["tensors"]] == list("abcd")
    assert meta["tensors"][0] == {"name": "a", "dtype": "float32", "numel": 231, "shape": [33, 7]}
    assert meta["tensors"][2]["dtype"] is None
    # refused: another list, another dtype or size, another widening mode, a different replica
    with pytest.raises(ValueError):
        load_table(p, tensors=ts[:4])
    bad = list(ts)
    bad[1] = bad[1].float()
    with pytest.raises(ValueError):
        load_table(p, tensors=bad)
    bad = list(ts)
    bad[0] = bad[0][:30]
    with pytest.raises(ValueError):
        load_table(p, tensors=bad)
    with pytest.raises(ValueError):
        load_table(p, signed=True)
    bad = list(ts)
    bad[5] = bad[5].float()
    with pytest.raises(ValueError):
        save_table(p, rows, bad, R=2)
    with pytest.raises(ValueError):
        save_table(p, rows[:3], ts, R=2)
