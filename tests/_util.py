"""Test helpers: host copies of device tensors and oracle rows for them.

Oracle calls over a list run in a thread pool, one plain oracle call per
tensor (ctypes releases the GIL); the oracle itself is unchanged.
"""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle as O

CODE = {torch.float32: O.F32, torch.bfloat16: O.BF16, torch.float16: O.F16,
        torch.float64: O.F64, torch.uint8: O.U8, torch.int8: O.U8, torch.bool: O.U8,
        torch.float8_e4m3fn: O.FP8_E4M3, torch.float8_e5m2: O.FP8_E5M2,
        torch.float8_e4m3fnuz: O.FP8_E4M3FNUZ, torch.float8_e5m2fnuz: O.FP8_E5M2FNUZ,
        torch.int16: O.U16, torch.int32: O.U32, torch.int64: O.U64}
THREADS = int(os.environ.get("SDC_TEST_THREADS", "16"))


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def host_bytes(t):
    """Raw bytes of a device tensor as a host uint8 numpy array."""
    if t is None:
        return None
    return t.detach().reshape(-1).view(torch.uint8).cpu().numpy()


def oracle_rows(tensors, threads=THREADS, flags=0):
    """uint64 [n, 4] oracle rows of a list of device tensors (None allowed)."""
    def one(t):
        if t is None:
            return (0, 0, 0, 0)
        return O.fingerprint(host_bytes(t), CODE[t.dtype], flags)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        rows = list(ex.map(one, tensors))
    return np.array(rows, dtype=np.uint64).reshape(-1, 4)


def oracle_nonfinite(tensors, threads=THREADS):
    def one(t):
        if t is None:
            return 0
        c, _ = O.nonfinite_list([host_bytes(t)], [CODE[t.dtype]])
        return int(c[0])
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return np.array(list(ex.map(one, tensors)), dtype=np.uint64)


def oracle_sqnorms(tensors, threads=THREADS):
    def one(t):
        return 0.0 if t is None else O.sqnorm(host_bytes(t), CODE[t.dtype])
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(one, tensors))


def assert_sq_close(gpu, ref, numels):
    """Squared sums of non-negative terms: |gpu - ref| <= 2 (n + 1) 2^-53 ref;
    NaN and Inf must match exactly."""
    import math
    for k, (g, r, n) in enumerate(zip(list(gpu), ref, numels)):
        if math.isfinite(r):
            assert abs(g - r) <= (2 * n + 2) * 2.0 ** -53 * r, (k, n, g, r)
        else:
            assert (math.isnan(g) and math.isnan(r)) or g == r, (k, n, g, r)


def assert_rows_equal(gpu, ref, names=None):
    gpu = np.asarray(gpu, dtype=np.uint64).reshape(-1, 4)
    ref = np.asarray(ref, dtype=np.uint64).reshape(-1, 4)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    bad = np.nonzero((gpu != ref).any(axis=1))[0]
    if bad.size:
        k = int(bad[0])
        nm = names[k] if names else k
        raise AssertionError(f"{bad.size} rows differ; first {nm}: gpu {gpu[k].tolist()} "
                             f"oracle {ref[k].tolist()}")
