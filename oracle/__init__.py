"""Oracle for the integrity scan -- TEST INFRASTRUCTURE ONLY.

A ctypes view of ``libsdc_oracle.so`` (plain single-threaded C, see
``sdc_oracle.h``).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It works on host
(numpy) buffers only and never touches the HIP library.

Parity status: every function here is pinned -- by ``tests/test_oracle_pins.py``
(closed forms, invariants, brute force, library routines, the pages' worked
example and fault table) and ``tests/test_ring.py`` (the pages' ring-audit
scenarios, brute force); none is "parity unpinned".
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16, F16, F64, U8, FP8_E4M3, FP8_E5M2, FP8_E4M3FNUZ, FP8_E5M2FNUZ, U16, U32, U64 = range(12)
ESIZE = {F32: 4, BF16: 2, F16: 2, F64: 8, U8: 1, FP8_E4M3: 1, FP8_E5M2: 1, FP8_E4M3FNUZ: 1,
         FP8_E5M2FNUZ: 1, U16: 2, U32: 4, U64: 8}
SIGNED = 1
COL_SUM, COL_WSUM, COL_XOR, COL_NONFINITE, COL_ALL = 1, 2, 4, 8, 15
U64MAX = (1 << 64) - 1

ROW_DTYPE = np.dtype([("sum", "<u8"), ("wsum", "<u8"), ("xorsum", "<u8"), ("nonfinite", "<u8")])


class Row(ctypes.Structure):
    _fields_ = [("sum", ctypes.c_uint64), ("wsum", ctypes.c_uint64),
                ("xorsum", ctypes.c_uint64), ("nonfinite", ctypes.c_uint64)]


class Majority(ctypes.Structure):
    _fields_ = [("diverged", ctypes.c_int32), ("has_majority", ctypes.c_int32),
                ("n_diff", ctypes.c_uint64), ("first_diff", ctypes.c_uint64),
                ("first_no_majority", ctypes.c_uint64)]


class FlipHint(ctypes.Structure):
    _fields_ = [("index", ctypes.c_uint64), ("bit", ctypes.c_int32), ("dir", ctypes.c_int32)]


_lib = None


def lib():
    """Load the oracle library, building it with gcc if it is not there yet."""
    global _lib
    if _lib is None:
        path = os.environ.get("SDC_ORACLE_LIB")  # e.g. the sanitizer build
        if not path:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        L = ctypes.CDLL(path)
        P, U64, U32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32
        L.oracle_element_size.argtypes = [U32]
        L.oracle_element_size.restype = U32
        L.oracle_is_nonfinite.argtypes = [U64, U32]
        L.oracle_is_nonfinite.restype = ctypes.c_int
        L.oracle_fingerprint.argtypes = [P, U64, U32, P]
        L.oracle_fingerprint_ex.argtypes = [P, U64, U32, U32, P]
        L.oracle_fingerprint_list.argtypes = [P, P, P, U64, P]
        L.oracle_nonfinite_list.argtypes = [P, P, P, U64, P, P]
        L.oracle_majority_compare.argtypes = [P, U32, U64, U32, P, P, P]
        L.oracle_flip_hint.argtypes = [P, P, P]
        L.oracle_fingerprint_diff.argtypes = [P, P, U64, U32, P, P, U64, P]
        L.oracle_value.argtypes = [U64, U32]
        L.oracle_value.restype = ctypes.c_double
        L.oracle_sqnorm.argtypes = [P, U64, U32, P]
        L.oracle_sqnorm.restype = ctypes.c_int
        L.oracle_sqnorm_flag.argtypes = [ctypes.c_double]
        L.oracle_sqnorm_flag.restype = ctypes.c_int
        L.oracle_ring_pairs.argtypes = [P, U32, U64, U32, P]
        L.oracle_ring_localize.argtypes = [P, U32, U32, P, P]
        L.oracle_confirm_verdict.argtypes = [P, P, P, P, U64, P]
        for f in ("oracle_fingerprint", "oracle_fingerprint_ex", "oracle_fingerprint_list", "oracle_nonfinite_list",
                  "oracle_majority_compare", "oracle_flip_hint", "oracle_fingerprint_diff",
                  "oracle_ring_pairs", "oracle_ring_localize", "oracle_confirm_verdict"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle call failed with code {rc}")


def _host_bytes(a):
    """A C-contiguous numpy view of host data (the caller keeps it alive)."""
    a = np.ascontiguousarray(a)
    return a, (a.ctypes.data if a.size else None)


def fingerprint(data, dtype, flags=0):
    """Row (S, W, X, NF) of one tensor given as a host numpy array of raw
    elements (any numpy dtype; its bytes are read; None = a missing tensor)."""
    out = Row()
    if data is None:
        _check(lib().oracle_fingerprint_ex(None, 0, dtype, flags, ctypes.byref(out)))
    else:
        arr, ptr = _host_bytes(data)
        numel = arr.nbytes // ESIZE[dtype]
        _check(lib().oracle_fingerprint_ex(ptr, numel, dtype, flags, ctypes.byref(out)))
    return (out.sum, out.wsum, out.xorsum, out.nonfinite)


def fingerprint_list(arrays, dtypes):
    """Rows of a list of host arrays (None allowed) as a structured array."""
    n = len(arrays)
    keep = []
    ptrs = (ctypes.c_void_p * max(n, 1))()
    numels = np.zeros(max(n, 1), dtype=np.uint64)
    dts = np.zeros(max(n, 1), dtype=np.uint32)
    for k, (a, dt) in enumerate(zip(arrays, dtypes)):
        dts[k] = dt
        if a is None:
            ptrs[k] = None
            continue
        arr, ptr = _host_bytes(a)
        keep.append(arr)
        ptrs[k] = ptr
        numels[k] = arr.nbytes // ESIZE[dt]
    rows = np.zeros(max(n, 1), dtype=ROW_DTYPE)
    _check(lib().oracle_fingerprint_list(ctypes.cast(ptrs, ctypes.c_void_p), numels.ctypes.data,
                                         dts.ctypes.data, n, rows.ctypes.data))
    return rows[:n]


def nonfinite_list(arrays, dtypes):
    n = len(arrays)
    keep = []
    ptrs = (ctypes.c_void_p * max(n, 1))()
    numels = np.zeros(max(n, 1), dtype=np.uint64)
    dts = np.zeros(max(n, 1), dtype=np.uint32)
    for k, (a, dt) in enumerate(zip(arrays, dtypes)):
        dts[k] = dt
        if a is None:
            continue
        arr, ptr = _host_bytes(a)
        keep.append(arr)
        ptrs[k] = ptr
        numels[k] = arr.nbytes // ESIZE[dt]
    counts = np.zeros(max(n, 1), dtype=np.uint64)
    total = ctypes.c_uint64(0)
    _check(lib().oracle_nonfinite_list(ctypes.cast(ptrs, ctypes.c_void_p), numels.ctypes.data,
                                       dts.ctypes.data, n, counts.ctypes.data,
                                       ctypes.byref(total)))
    return counts[:n], total.value


def as_rows(table):
    """Structured ROW_DTYPE array from an (..., 4) uint64 array or a structured one."""
    t = np.asarray(table)
    if t.dtype == ROW_DTYPE:
        return np.ascontiguousarray(t)
    t = np.ascontiguousarray(t.astype(np.uint64, copy=False).reshape(-1, 4))
    return t.view(ROW_DTYPE).reshape(-1)


def majority_compare(table, R, T, col_mask=COL_ALL):
    """Strict-majority comparison of a replica-major table of R*T rows."""
    rows = as_rows(table)
    assert rows.size == R * T
    res = Majority()
    suspect = np.zeros(max(R, 1), dtype=np.uint8)
    status = np.zeros(max(T, 1), dtype=np.uint8)
    _check(lib().oracle_majority_compare(rows.ctypes.data, R, T, col_mask, ctypes.byref(res),
                                         suspect.ctypes.data, status.ctypes.data))
    return {"diverged": bool(res.diverged), "has_majority": bool(res.has_majority),
            "n_diff": res.n_diff, "first_diff": res.first_diff,
            "first_no_majority": res.first_no_majority,
            "suspects": [r for r in range(R) if suspect[r]] if res.has_majority else None,
            "suspect_flags": suspect[:R].copy(), "tensor_status": status[:T].copy()}


def flip_hint(a, b):
    ra, rb = Row(*[int(v) for v in a]), Row(*[int(v) for v in b])
    h = FlipHint()
    _check(lib().oracle_flip_hint(ctypes.byref(ra), ctypes.byref(rb), ctypes.byref(h)))
    return (h.index, h.bit, h.dir)


def fingerprint_diff(a, b, col_mask=COL_ALL, cap=None):
    ra, rb = as_rows(a), as_rows(b)
    assert ra.size == rb.size
    T = ra.size
    cap = T if cap is None else cap
    idx = np.zeros(max(cap, 1), dtype=np.uint64)
    hints = (FlipHint * max(cap, 1))()
    n = ctypes.c_uint64(0)
    _check(lib().oracle_fingerprint_diff(ra.ctypes.data if T else None,
                                         rb.ctypes.data if T else None, T, col_mask,
                                         ctypes.byref(n), idx.ctypes.data, cap,
                                         ctypes.cast(hints, ctypes.c_void_p)))
    m = min(n.value, cap)
    return {"n_diff": n.value, "indices": [int(i) for i in idx[:m]],
            "hints": [(hints[i].index, hints[i].bit, hints[i].dir) for i in range(m)]}


VERDICTS = {1: "replayer computed wrong", 2: "persistent", 3: "transient", 4: "unclear",
            5: "unattributable"}


def ring_pairs(table, n, offset):
    """Mismatch flags of the n ring pairs of an [n, 2, width] uint64 table."""
    t = np.ascontiguousarray(np.asarray(table, dtype=np.uint64).reshape(n, 2, -1))
    width = t.shape[2]
    out = np.zeros(n, dtype=np.uint8)
    _check(lib().oracle_ring_pairs(t.ctypes.data if t.size else None, n, width, offset,
                                   out.ctypes.data))
    return out


def ring_localize(mismatch, n, offset):
    m = np.ascontiguousarray(np.asarray(mismatch, dtype=np.uint8))
    cul = np.zeros(n, dtype=np.uint8)
    amb = np.zeros(n, dtype=np.uint8)
    _check(lib().oracle_ring_localize(m.ctypes.data, n, offset, cul.ctypes.data, amb.ctypes.data))
    return cul, amb


def confirm_verdict(witness, retry, original, replay):
    """Verdict code of a confirmation (see VERDICTS) from the witness GPU's
    replay, the target's retry, the target's original result and the
    replayer's replay."""
    arrs = [np.ascontiguousarray(np.asarray(a, dtype=np.uint64).reshape(-1))
            for a in (witness, retry, original, replay)]
    width = arrs[0].size
    v = ctypes.c_int32(0)
    _check(lib().oracle_confirm_verdict(*[a.ctypes.data if width else None for a in arrs], width,
                                        ctypes.byref(v)))
    return v.value


def value(x, dtype):
    return lib().oracle_value(int(x), dtype)


def sqnorm(data, dtype):
    """sum of squared element values (double, index order) of a host array."""
    out = ctypes.c_double(0.0)
    if data is None:
        _check(lib().oracle_sqnorm(None, 0, dtype, ctypes.byref(out)))
    else:
        arr, ptr = _host_bytes(data)
        _check(lib().oracle_sqnorm(ptr, arr.nbytes // ESIZE[dtype], dtype, ctypes.byref(out)))
    return out.value


def sqnorm_flag(sq):
    return bool(lib().oracle_sqnorm_flag(float(sq)))
