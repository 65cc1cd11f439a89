"""The oracle over device tensors -- TEST INFRASTRUCTURE ONLY (used by tests/
and by bench.py's cpu_baseline leg).

Streams a list of device tensors to the host and runs the unmodified
single-threaded oracle (``oracle.fingerprint``, one call per whole tensor) on
a pool of host threads.  The main thread copies tensor after tensor into
pinned host buffers (synchronous copies, so their time is measured on their
own); each copied tensor goes to the pool at once, so copies overlap the
oracle's work on earlier tensors.  Host memory is bounded by the bytes of
tensors copied but not yet fingerprinted.  Nothing here computes any part of
a fingerprint: the rows are the oracle's.
"""
import threading
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import fingerprint

_CODE_OF = {}


def _code(t):
    import torch
    import oracle as O
    if not _CODE_OF:
        _CODE_OF.update({torch.float32: O.F32, torch.bfloat16: O.BF16, torch.float16: O.F16,
                         torch.float64: O.F64, torch.uint8: O.U8, torch.int8: O.U8,
                         torch.bool: O.U8, torch.float8_e4m3fn: O.FP8_E4M3,
                         torch.float8_e5m2: O.FP8_E5M2, torch.float8_e4m3fnuz: O.FP8_E4M3FNUZ,
                         torch.float8_e5m2fnuz: O.FP8_E5M2FNUZ, torch.int16: O.U16,
                         torch.int32: O.U32, torch.int64: O.U64})
    return _CODE_OF[t.dtype]


def rows_of_device_tensors(tensors, threads=16, inflight_bytes=24 << 30, flags=0):
    """(rows, stats): the oracle's uint64 [n, 4] rows of a list of device
    tensors (None: a missing tensor; host tensors are copied into ordinary
    host memory) in logical row-major element order, and
    timing statistics:
      threads   worker threads that ran oracle calls
      bytes     bytes fingerprinted; elements: elements fingerprinted
      wall_s    wall time from the first copy to the last row
      d2h_s     time the main thread spent in device-to-host copies
      busy_s    sum over the oracle calls of their durations (CPU seconds)
      max_call_s  the longest single oracle call
    """
    import torch
    n = len(tensors)
    rows = np.zeros((n, 4), dtype=np.uint64)
    lock = threading.Condition()
    state = {"inflight": 0, "busy": 0.0, "max_call": 0.0}

    def work(k, host, code, nb):
        t0 = time.perf_counter()
        r = fingerprint(host.numpy(), code, flags)
        dt = time.perf_counter() - t0
        rows[k] = r
        with lock:
            state["inflight"] -= nb
            state["busy"] += dt
            state["max_call"] = max(state["max_call"], dt)
            lock.notify_all()

    d2h = 0.0
    nbytes = nel = 0
    futures = []
    t_start = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for k, t in enumerate(tensors):
            if t is None or t.numel() == 0:
                continue  # the zero row
            nb = t.numel() * t.element_size()
            with lock:
                while state["inflight"] > 0 and state["inflight"] + nb > inflight_bytes:
                    lock.wait()
                state["inflight"] += nb
            src = t.detach().contiguous().reshape(-1).view(torch.uint8)
            host = torch.empty(nb, dtype=torch.uint8, pin_memory=t.is_cuda)
            t0 = time.perf_counter()
            host.copy_(src)
            d2h += time.perf_counter() - t0
            nbytes += nb
            nel += t.numel()
            futures.append(ex.submit(work, k, host, _code(t), nb))
        for f in futures:
            f.result()
    wall = time.perf_counter() - t_start
    del futures
    try:
        torch._C._host_emptyCache()  # return the pinned staging buffers
    except AttributeError:
        pass
    return rows, {"threads": threads, "bytes": nbytes, "elements": nel, "wall_s": wall,
                  "d2h_s": d2h, "busy_s": state["busy"], "max_call_s": state["max_call"]}
