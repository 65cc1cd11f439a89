"""The C-ABI library loads and exports every declared symbol; host-only entry
points (sizing, validation, status strings) behave as documented.  No GPU:
nothing here launches a kernel or touches device memory."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions(header):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(sdc_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions(os.path.join(ROOT, "include", "sdc.h"))
    for required in ("sdc_fingerprint", "sdc_fingerprint_plan", "sdc_plan_build", "sdc_plan_bytes",
                     "sdc_nonfinite", "sdc_majority_compare", "sdc_fingerprint_diff"):
        assert required in names


def test_library_exports_every_declared_symbol():
    import silent_corruption_detection_amd as sdc
    lib = ctypes.CDLL(sdc.LIB_PATH)
    for name in declared_functions(os.path.join(ROOT, "include", "sdc.h")):
        assert hasattr(lib, name), name


def test_oracle_exports_every_declared_symbol():
    import oracle
    lib = oracle.lib()
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "oracle", "sdc_oracle.h")).read(), flags=re.S)
    names = set(re.findall(r"\b(oracle_[a-z_0-9]+)\s*\(", text))
    assert len(names) >= 8
    for name in names:
        assert hasattr(lib, name), name


def test_status_and_version():
    import silent_corruption_detection_amd as sdc
    assert sdc.sdc_abi_version() == 2
    assert sdc.sdc_status_string(0) == "ok"
    for code in range(-7, 0):
        assert sdc.sdc_status_string(code) not in ("ok", "unknown status")
    assert sdc.sdc_status_string(-99) == "unknown status"


class _T(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("numel", ctypes.c_uint64),
                ("dtype", ctypes.c_uint32), ("flags", ctypes.c_uint32)]


def plan_bytes(descs, item_bytes=0):
    import silent_corruption_detection_amd as sdc
    lib = ctypes.CDLL(sdc.LIB_PATH)
    arr = (_T * max(len(descs), 1))(*[_T(*d) for d in descs])
    out = ctypes.c_uint64(0)
    rc = lib.sdc_plan_bytes(arr, ctypes.c_uint64(len(descs)), ctypes.c_uint64(item_bytes),
                            ctypes.byref(out))
    return rc, out.value


def test_plan_bytes_host_only():
    # Sizing reads only the descriptors (pointer values are never dereferenced).
    rc, b0 = plan_bytes([])
    assert rc == 0 and b0 >= 64
    rc, b1 = plan_bytes([(0x10000, 1000, 0, 0)])
    assert rc == 0 and b1 >= 64 + 32
    # 4 MiB of fp32 split into 64 KiB items: 64 items of 32 bytes each + one cleared row
    rc, b2 = plan_bytes([(0x10000, 1 << 20, 0, 0)], item_bytes=65536)
    assert rc == 0 and b2 >= 64 + 64 * 32 + 4
    # None / empty tensors need no items, only a cleared row
    rc, b3 = plan_bytes([(None, 0, 0, 0), (0x10000, 0, 1, 0)])
    assert rc == 0


def test_fingerprint_ws_bytes_is_the_automatic_plan_size():
    import numpy as np
    import silent_corruption_detection_amd as sdc
    lib = ctypes.CDLL(sdc.LIB_PATH)
    rng = np.random.default_rng(8)
    for n in (0, 1, 7, 300, 5000):
        descs = [(0x7F0000000000 + int(rng.integers(0, 1 << 20)) * 16, int(rng.integers(0, 3_000_000)),
                  int(rng.integers(0, 3)), 0) for _ in range(n)]
        arr = (_T * max(n, 1))(*[_T(*d) for d in descs])
        out = ctypes.c_uint64(0)
        assert lib.sdc_fingerprint_ws_bytes(arr, ctypes.c_uint64(n), ctypes.byref(out)) == 0
        assert plan_bytes(descs) == (0, out.value)
    assert lib.sdc_fingerprint_ws_bytes(None, ctypes.c_uint64(1), ctypes.byref(out)) == -1


@pytest.mark.parametrize("desc,item_bytes,code", [
    ((0x10000, 10, 99, 0), 0, -2),     # unknown dtype
    ((0x10001, 10, 3, 0), 0, -3),      # fp64 pointer not 8-byte aligned
    ((0x10001, 10, 0, 0), 0, -3),      # fp32 pointer not 4-byte aligned
    ((0x10001, 10, 1, 0), 0, -3),      # bf16 pointer odd
    ((0x10000, 10, 0, 2), 0, -1),      # only SDC_FLAG_SIGNED is a flag
    ((0x10000, 10, 0, 0), 24, -1),     # item size not a multiple of 16
    ((0x10000, 10, 0, 0), 8 << 20, -1),  # item size above 4 MiB
    ((0x10000, 1 << 62, 0, 0), 0, -7),  # too many elements
    ((0x10000, 1 << 59, 3, 0), 0, -7),  # fp64: 2^62 bytes (below 2^62 elements)
    ((0x10000, (1 << 60) - 1, 0, 0), 4 << 20, -7),  # fp32, just under 2^62 bytes: too many items
])
def test_plan_validation_errors(desc, item_bytes, code):
    rc, _ = plan_bytes([desc], item_bytes)
    assert rc == code


def test_workspace_sizing():
    import silent_corruption_detection_amd as sdc
    assert sdc.sdc_majority_ws_bytes(3, 100) > 0
    # the workspace holds a 24-byte record (index + flip hint) per reported row,
    # and at most T rows can differ, so a cap above T counts as T
    assert sdc.sdc_diff_ws_bytes(5000, 1000) >= sdc.sdc_diff_ws_bytes(5000, 0) + 24 * 1000 - 256
    assert sdc.sdc_diff_ws_bytes(100, 10) >= 16 + 24 * 10
    assert sdc.sdc_diff_ws_bytes(100, 1000) == sdc.sdc_diff_ws_bytes(100, 100)
    assert sdc.sdc_diff_ws_bytes(100, (1 << 58) - 1) == sdc.sdc_diff_ws_bytes(100, 100)
    with pytest.raises(sdc.SdcError):
        sdc.sdc_majority_ws_bytes(0, 10)


def tensor_ws_bytes(desc, item_bytes=0):
    import silent_corruption_detection_amd as sdc
    lib = ctypes.CDLL(sdc.LIB_PATH)
    t = _T(*desc)
    out = ctypes.c_uint64(0)
    rc = lib.sdc_tensor_ws_bytes(ctypes.byref(t), ctypes.c_uint64(item_bytes), ctypes.byref(out))
    return rc, out.value


def one_tensor_plan_items(desc, item_bytes):
    import silent_corruption_detection_amd as sdc
    lib = ctypes.CDLL(sdc.LIB_PATH)
    arr = (_T * 1)(_T(*desc))
    need = ctypes.c_uint64(0)
    assert lib.sdc_plan_bytes(arr, ctypes.c_uint64(1), ctypes.c_uint64(item_bytes),
                              ctypes.byref(need)) == 0
    buf = (ctypes.c_ubyte * need.value)()

    info = sdc._PlanInfo()
    assert lib.sdc_plan_pack_host(arr, ctypes.c_uint64(1), ctypes.c_uint64(item_bytes), buf,
                                  ctypes.c_uint64(need.value), ctypes.byref(info)) == 0
    return info.n_items, info.total_bytes


DESCS = [(0x10000, 1, 0, 0), (0x10004, 1000, 0, 0), (0x10002, 3 << 20, 1, 0),
         (0x10000, 5 << 30, 1, 1), (0x10008, 12345678, 3, 0), (0x10003, 7777777, 4, 0),
         (0x10000, (64 << 20) - 1, 1, 0), (0x10002, 64 << 20, 2, 0), (0x10004, 300 << 20, 0, 0),
         (0x10001, (1 << 30) + 7, 4, 0)]


@pytest.mark.parametrize("desc", DESCS)
@pytest.mark.parametrize("item_bytes", [16, 4096, 65536, 1 << 20, 4 << 20])
def test_tensor_ws_bytes_match_the_plan_split(desc, item_bytes):
    # the single-tensor scan splits a tensor exactly as a one-tensor plan does
    if desc[1] * 8 // item_bytes > 1 << 22:
        pytest.skip("plan image too large for a host test")
    rc, ws = tensor_ws_bytes(desc, item_bytes)
    assert rc == 0
    assert ws == 32 * one_tensor_plan_items(desc, item_bytes)[0]


def tensor_split(desc, item_bytes, cus):
    import silent_corruption_detection_amd as sdc
    lib = ctypes.CDLL(sdc.LIB_PATH)
    t = _T(*desc)
    n, ib = ctypes.c_uint64(0), ctypes.c_uint64(0)
    rc = lib.sdc_tensor_split_host(ctypes.byref(t), ctypes.c_uint64(item_bytes), ctypes.c_uint32(cus),
                                   ctypes.byref(n), ctypes.byref(ib))
    return rc, n.value, ib.value


def auto_tensor_item_bytes(nbytes, cus=256):
    # tensors of at least 128 MiB: a multiple of `cus` items (one per CU per
    # pass; at most 256 CUs are used) of at most 4 MiB; smaller ones: about
    # 1024 items within [64 KiB, 1 MiB]; item sizes are multiples of 4 KiB
    r4k = lambda b: -(-b // 4096) * 4096
    c = max(1, min(cus, 256))
    if nbytes >= 128 << 20:
        passes = -(-nbytes // (c * (4 << 20)))
        return r4k(-(-nbytes // (c * passes)))
    return min(max(r4k(max(nbytes // 1024, 1)), 64 << 10), 1 << 20)


ESZ = {0: 4, 1: 2, 2: 2, 3: 8, 4: 1}


@pytest.mark.parametrize("desc", DESCS)
@pytest.mark.parametrize("cus", [256, 80, 32, 1, 304])
def test_tensor_automatic_item_size(desc, cus):
    # the split on a device with `cus` compute units (the full MI355X: 256; a
    # CPX partition: 32), and the workspace bound that holds for all of them
    nbytes = desc[1] * ESZ[desc[2]]
    ib = auto_tensor_item_bytes(nbytes, cus)
    assert ib % 4096 == 0 and ib <= 4 << 20
    rc, n_split, ib_split = tensor_split(desc, 0, cus)
    assert rc == 0 and ib_split == ib
    n_items, total = one_tensor_plan_items(desc, ib)
    assert total == nbytes and n_split == n_items
    assert tensor_ws_bytes(desc)[1] >= 32 * n_items
    c = max(1, min(cus, 256))
    if nbytes >= 128 << 20:  # one item per CU per pass, at most 4 MiB each
        passes = -(-nbytes // (c * (4 << 20)))
        assert c * passes - c < n_items <= c * passes + 1
    else:  # the workspace is exact below the wide split
        assert tensor_ws_bytes(desc)[1] == 32 * n_items


@pytest.mark.parametrize("desc", DESCS)
def test_tensor_ws_bound_covers_every_cu_count(desc):
    ws = tensor_ws_bytes(desc)[1]
    nbytes = desc[1] * ESZ[desc[2]]
    worst = max(tensor_split(desc, 0, c)[1] for c in range(1, 257))
    assert 32 * worst <= ws <= 32 * max(worst, -(-nbytes // (4 << 20)) + 257)


def test_tensor_ws_small_below_the_wide_split_and_growing_above():
    # what the recompute audit's workspace cache relies on: with the automatic
    # split, 64 KiB holds the partial rows of any tensor below 128 MiB, and
    # above it the bound never falls as the tensor grows
    sizes = {s for k in range(1, 28) for s in (1 << k, (1 << k) + 7, 3 << (k - 1))}
    sizes |= {(m << 20) + d for m in range(127, 4097, 61) for d in (-8, 0, 8)}
    for dtype, es in ESZ.items():
        for align in (0, es):
            prev = 0
            for nbytes in sorted(sizes):
                rc, ws = tensor_ws_bytes((0x100000 + (align if es > 1 else 0), nbytes // es, dtype, 0))
                assert rc == 0
                if nbytes // es * es < 128 << 20:
                    assert ws <= 1 << 16, (dtype, nbytes)
                else:
                    assert ws >= prev, (dtype, nbytes)
                    prev = ws


def test_tensor_split_explicit_item_size_ignores_cus():
    for cus in (1, 32, 256):
        assert tensor_split((0x10002, 3 << 20, 1, 0), 65536, cus) == (0, 96, 65536)
    assert tensor_split((0x10000, 10, 0, 0), 0, 0)[0] == -1


@pytest.mark.parametrize("desc,item_bytes,code", [
    ((0x10000, 10, 99, 0), 0, -2), ((0x10001, 10, 0, 0), 0, -3), ((0x10000, 10, 0, 2), 0, -1),
    ((0x10000, 1 << 62, 0, 0), 0, -7), ((0x10000, 1 << 59, 3, 0), 0, -7),
    ((0x10000, 10, 0, 0), 24, -1),
    ((0x10000, 10, 0, 0), 8 << 20, -1)])
def test_tensor_ws_bytes_errors(desc, item_bytes, code):
    assert tensor_ws_bytes(desc, item_bytes)[0] == code


def test_tensor_ws_bytes_empty_and_missing():
    assert tensor_ws_bytes((None, 100, 0, 0)) == (0, 32)
    assert tensor_ws_bytes((0x10000, 0, 2, 0)) == (0, 32)


@pytest.mark.parametrize("buf,nbytes,ws,ws_bytes,out,code", [
    (0x10000, 6, 0x30000, 8, 0x20000, -1),           # not a whole number of 32-bit words
    (0x10000, 16, 0x30000, 8, None, -1),             # no output
    (0x10000, 16, None, 8, 0x20000, -1),             # no workspace
    (None, 16, 0x30000, 8, 0x20000, -1),             # no buffer
    (0x10004, 16, 0x30000, 8, 0x20000, -3),          # buffer not 16-byte aligned
    (0x10000, 16, 0x30004, 8, 0x20000, -3),          # workspace not 8-byte aligned
    (0x10000, (1 << 20) + 16, 0x30000, 8, 0x20000, -4),   # two chunks need 16 bytes
    (0x10000, 1 << 62, 0x30000, 8, 0x20000, -7)])    # more chunks than a grid holds
def test_read_sum_argument_checks(buf, nbytes, ws, ws_bytes, out, code):
    # every case returns before any HIP call (the pointers are never dereferenced)
    import silent_corruption_detection_amd as sdc
    lib = ctypes.CDLL(sdc.LIB_PATH)
    V, U64 = ctypes.c_void_p, ctypes.c_uint64
    lib.sdc_read_sum.argtypes = [V, U64, V, U64, V, V]
    lib.sdc_read_sum.restype = ctypes.c_int32
    assert lib.sdc_read_sum(buf, nbytes, ws, ws_bytes, out, None) == code


def test_read_sum_ws_bytes():
    import silent_corruption_detection_amd as sdc
    MIB = 1 << 20
    for nbytes, chunks in ((0, 1), (4, 1), (MIB, 1), (MIB + 4, 1), (MIB + 16, 2), (32 << 30, 32768)):
        assert sdc.sdc_read_sum_ws_bytes(nbytes) == 8 * chunks
    with pytest.raises(sdc.SdcError):
        sdc.sdc_read_sum_ws_bytes(1 << 62)
