"""sdc_fingerprint_tensor_noalloc (the single-tensor scan without a workspace:
partial rows in the library's static device array) against
sdc_fingerprint_tensor (the same scan with a caller workspace) and the
oracle, through the C ABI: two calls in a row, the second on a smaller tensor,
so the second reuses the array the first left behind.  Also the device
compare, and the size limit (rejected before anything is queued)."""
import ctypes

import numpy as np
import pytest
import torch

import silent_corruption_detection_amd as sdc
from _util import assert_rows_equal, oracle_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


class _T(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("numel", ctypes.c_uint64),
                ("dtype", ctypes.c_uint32), ("flags", ctypes.c_uint32)]


def _abi():
    lib = ctypes.CDLL(sdc.LIB_PATH)
    V, U64, U32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32
    lib.sdc_fingerprint_tensor_noalloc.argtypes = [V, U64, V, U32, V, V, V]
    lib.sdc_fingerprint_tensor_noalloc.restype = ctypes.c_int32
    return lib


def _noalloc(lib, t, code, out, item_bytes=0, ref=None, mismatch=None, mask=sdc.COL_ALL):
    desc = _T(t.data_ptr(), t.numel(), code, 0)
    s = torch.cuda.current_stream()
    return lib.sdc_fingerprint_tensor_noalloc(
        ctypes.byref(desc), item_bytes, ref.data_ptr() if ref is not None else None, mask,
        out.data_ptr(), mismatch.data_ptr() if mismatch is not None else None, s.cuda_stream)


def test_noalloc_matches_the_workspace_scan_twice_in_a_row():
    lib = _abi()
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    # first: 300 MiB of bf16 (the tensor-wide split, one item per CU); second:
    # a smaller fp32 tensor at a misaligned start (deep/short split, a head)
    big = torch.empty(150 << 20, dtype=torch.float32, device=DEV).normal_(0, 1, generator=g)
    big = big.to(torch.bfloat16)
    small_base = torch.empty(3_000_001, dtype=torch.float32, device=DEV).normal_(0, 0.02, generator=g)
    small = small_base[1:]
    cases = [(big, sdc.BF16), (small, sdc.F32)]
    ref = oracle_rows(cases[0][0:1] + cases[1][0:1])
    out = torch.full((2, 4), -1, dtype=torch.int64, device=DEV)
    want = torch.empty((2, 4), dtype=torch.int64, device=DEV)
    torch.cuda.synchronize()
    for k, (t, code) in enumerate(cases):
        say(f"case noalloc call {k}: numel {t.numel()} dtype {t.dtype}")
        assert _noalloc(lib, t, code, out[k]) == 0
        sdc.sdc_fingerprint_tensor(t, out=want[k:k + 1])
        torch.cuda.synchronize()
        assert torch.equal(out[k], want[k])
    assert_rows_equal(sdc.rows_numpy(out), ref)
    # explicit item sizes, both calls again (reusing the array once more)
    for k, (t, code) in enumerate(cases):
        for ib in (1 << 20, 65536):
            if t.numel() * t.element_size() // ib > 8000:
                continue
            o = torch.full((4,), -1, dtype=torch.int64, device=DEV)
            assert _noalloc(lib, t, code, o, item_bytes=ib) == 0
            torch.cuda.synchronize()
            assert np.array_equal(sdc.rows_numpy(o)[0], ref[k]), (k, ib)


def test_noalloc_compare_and_limit():
    lib = _abi()
    g = torch.Generator(device=DEV)
    g.manual_seed(78)
    t = torch.empty(5_000_000, dtype=torch.float32, device=DEV).normal_(0, 0.02, generator=g)
    stored = torch.empty(4, dtype=torch.int64, device=DEV)
    assert _noalloc(lib, t, sdc.F32, stored) == 0
    mis = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.empty(4, dtype=torch.int64, device=DEV)
    assert _noalloc(lib, t, sdc.F32, out, ref=stored, mismatch=mis) == 0
    torch.cuda.synchronize()
    assert int(mis.item()) == 0 and torch.equal(out, stored)
    t.view(torch.int32)[123_457] ^= 1 << 9
    assert _noalloc(lib, t, sdc.F32, out, ref=stored, mismatch=mis) == 0
    torch.cuda.synchronize()
    assert int(mis.item()) == 1
    assert np.array_equal(sdc.rows_numpy(out)[0], oracle_rows([t])[0])
    # more work items than the static array holds: rejected, nothing queued
    mis.zero_()
    torch.cuda.synchronize()
    assert _noalloc(lib, t, sdc.F32, out, item_bytes=16) == -7
    # the binding's form of the call
    o2 = torch.empty(4, dtype=torch.int64, device=DEV)
    sdc.sdc_fingerprint_tensor_noalloc(t, o2)
    torch.cuda.synchronize()
    assert torch.equal(o2, out)


def test_noalloc_under_graph_capture():
    # the callers it is for: two calls (a tensor-wide split with a compare, and a
    # smaller tensor) captured into a graph, replayed with eager work and a
    # data change in between; every replay equals the eager scans and the oracle
    import workloads as W
    lib = _abi()
    g = torch.Generator(device=DEV)
    g.manual_seed(79)
    big = torch.empty(40_000_003, dtype=torch.float32, device=DEV).normal_(0, 1, generator=g)
    small = torch.empty(777_777, dtype=torch.float32, device=DEV).normal_(0, 1, generator=g)
    small = small.to(torch.bfloat16)
    ref = sdc.sdc_fingerprint_tensor(big).clone()
    out = torch.empty((2, 4), dtype=torch.int64, device=DEV)
    mis = torch.zeros(1, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()

    def work():
        mis.zero_()
        assert _noalloc(lib, big, sdc.F32, out[0], ref=ref, mismatch=mis) == 0
        assert _noalloc(lib, small, sdc.BF16, out[1]) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("case noalloc graph capture")
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()
    expect = oracle_rows([big, small])
    for rep in range(4):
        if rep == 2:   # a flip in the big tensor: the compare must report it
            W.flip_bit(big, 123_457, 5)
            expect = oracle_rows([big, small])
        out.fill_(-1)
        torch.cuda.synchronize()
        say(f"case noalloc graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        got = sdc.rows_numpy(out).copy()
        torch.randn(1 << 20, device=DEV).sum().item()   # eager work between replays
        eager = np.concatenate([sdc.rows_numpy(sdc.sdc_fingerprint_tensor(big)),
                                sdc.rows_numpy(sdc.sdc_fingerprint_tensor(small))])
        torch.cuda.synchronize()
        assert np.array_equal(got, eager)
        assert_rows_equal(got, expect)
        assert int(mis.item()) == (1 if rep >= 2 else 0)
