"""Stored fingerprint tables: the rows of a scan saved beside a checkpoint and
loaded back after a restore, so the restored weights can be checked against
the state that was saved (AWS Machine Learning Blog, "Detecting and recovering
from silent data corruption on Amazon SageMaker HyperPod", sections "Fault
scenarios" -- the weight check run right after a restore -- and "Check 3").

A table is two files: ``<path>.npy``, the uint64 rows as an [R, T, 4] array
(replica-major; columns sum, wsum, xorsum, nonfinite), and ``<path>.json``,
which describes the list the rows belong to (per tensor: name, dtype, numel,
shape; the replica count and whether 2-/4-byte patterns were sign-extended).
Loading checks the files against each other and, when given, against the live
tensor list, so a table is never compared with a different list.  Host-side
file handling only: the rows come from the scan, the comparison is
sdc_fingerprint_diff.
"""
import json

import numpy as np
import torch

FORMAT = "sdc-fingerprint-table"
VERSION = 1
COLUMNS = ["sum", "wsum", "xorsum", "nonfinite"]


def _describe(tensors, names):
    out = []
    for k, t in enumerate(tensors):
        nm = names[k] if names is not None else str(k)
        if t is None:
            out.append({"name": nm, "dtype": None, "numel": 0, "shape": None})
        else:
            out.append({"name": nm, "dtype": str(t.dtype).replace("torch.", ""),
                        "numel": int(t.numel()), "shape": list(t.shape)})
    return out


def save_table(path, rows, tensors, R=1, names=None, signed=False):
    """Writes the [R*T, 4] rows (an int64 tensor holding the uint64 patterns,
    device or host, as the scans return them) of the replica-major list
    `tensors` (R*T entries, None allowed; names: T names or None) to
    <path>.npy and <path>.json."""
    n = len(tensors)
    if R < 1 or n % R:
        raise ValueError(f"{n} tensors are not {R} replicas of one list")
    T = n // R
    if names is not None and len(names) != T:
        raise ValueError(f"{len(names)} names for {T} tensors per replica")
    if not isinstance(rows, torch.Tensor) or rows.dtype != torch.int64 or tuple(rows.shape) != (n, 4):
        raise ValueError(f"rows must be an int64 [{n}, 4] tensor")
    arr = rows.detach().cpu().numpy().view(np.uint64).reshape(R, T, 4)
    meta = {"format": FORMAT, "version": VERSION, "columns": COLUMNS, "R": R, "T": T,
            "signed": bool(signed),
            "tensors": _describe(tensors[:T], names if names is not None else None)}
    for r in range(1, R):  # every replica must have the first one's shapes and types
        if _describe(tensors[r * T:(r + 1) * T], names) != meta["tensors"]:
            raise ValueError(f"replica {r} differs in shape or type from replica 0")
    np.save(path + ".npy", arr, allow_pickle=False)
    with open(path + ".json", "w") as f:
        json.dump(meta, f, indent=1)


def load_table(path, tensors=None, device=None, signed=None):
    """(rows, meta): the stored rows as an int64 [R*T, 4] tensor (on `device`,
    default the host) and the sidecar.  With `tensors` (the live list, R*T
    entries) every tensor's dtype and numel must match the sidecar; with
    `signed`, so must the widening mode.  Raises ValueError on any mismatch."""
    with open(path + ".json") as f:
        meta = json.load(f)
    if meta.get("format") != FORMAT or meta.get("version") != VERSION:
        raise ValueError(f"{path}.json is not a fingerprint table of version {VERSION}")
    arr = np.load(path + ".npy", allow_pickle=False)
    R, T = int(meta["R"]), int(meta["T"])
    if arr.dtype != np.uint64 or arr.shape != (R, T, 4) or len(meta["tensors"]) != T:
        raise ValueError(f"{path}.npy does not hold {R} x {T} rows of uint64")
    if signed is not None and bool(signed) != bool(meta["signed"]):
        raise ValueError("the table was taken in the other widening mode")
    if tensors is not None:
        if len(tensors) != R * T:
            raise ValueError(f"the list has {len(tensors)} tensors, the table {R * T}")
        for k, t in enumerate(tensors):
            d = meta["tensors"][k % T]
            got = (None, 0) if t is None else (str(t.dtype).replace("torch.", ""), int(t.numel()))
            if got != (d["dtype"], d["numel"]):
                raise ValueError(f"tensor {k} ({d['name']}): stored {d['dtype']}[{d['numel']}], "
                                 f"live {got[0]}[{got[1]}]")
    rows = torch.from_numpy(arr.reshape(R * T, 4).view(np.int64).copy())
    if device is not None:
        rows = rows.to(device)
    return rows, meta
