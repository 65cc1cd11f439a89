"""Host logic of the plan (CPU, no GPU): the work list built by
sdc_plan_pack_host covers every element of every tensor exactly once, keeps
every item inside its tensor, aligns every item boundary inside a tensor to
16 bytes, respects the item-size bounds the kernels' accumulators rely on,
and keeps the wave-item, whole-tensor and split/slot bookkeeping consistent.
Pointer values here are synthetic (never dereferenced)."""
import ctypes

import numpy as np
import pytest

import silent_corruption_detection_amd as sdc

ES = {0: 4, 1: 2, 2: 2, 3: 8, 4: 1, 5: 1, 6: 1, 7: 1, 8: 1, 9: 2, 10: 4, 11: 8}
WHOLE = 0x100
WAVE_BODY_VECS = 512
ITEM_MAX = 4 << 20


class _T(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("numel", ctypes.c_uint64),
                ("dtype", ctypes.c_uint32), ("flags", ctypes.c_uint32)]


def pack(descs, item_bytes):
    lib = ctypes.CDLL(sdc.LIB_PATH)
    arr = (_T * max(len(descs), 1))(*[_T(*d) for d in descs])
    nbytes = ctypes.c_uint64(0)
    assert lib.sdc_plan_bytes(arr, ctypes.c_uint64(len(descs)), ctypes.c_uint64(item_bytes),
                              ctypes.byref(nbytes)) == 0
    buf = (ctypes.c_uint8 * nbytes.value)()
    info = sdc._PlanInfo()
    rc = lib.sdc_plan_pack_host(arr, ctypes.c_uint64(len(descs)), ctypes.c_uint64(item_bytes), buf,
                                ctypes.c_uint64(nbytes.value), ctypes.byref(info))
    assert rc == 0
    img = np.frombuffer(bytes(buf), dtype=np.uint8)
    return img, info, nbytes.value


def parse(img, info):
    hdr = img[:64].view(np.uint64)
    it = np.dtype([("addr", "<u8"), ("start", "<u8"), ("len", "<u4"), ("row", "<u4"),
                   ("slot", "<u4"), ("df", "<u4")])
    items = img[64:64 + 32 * info.n_items].view(it)
    so = 64 + 32 * info.n_items
    split = img[so:so + 16 * info.n_split].view(np.uint32).reshape(-1, 4)
    return hdr, items, split


def check_plan(descs, item_bytes):
    img, info, nbytes = pack(descs, item_bytes)
    hdr, items, split = parse(img, info)
    assert int(hdr[1]) == len(descs) == info.n_tensors
    assert int(hdr[2]) == info.n_items and int(hdr[3]) == info.n_split
    assert int(hdr[4]) == info.n_slots and int(hdr[7]) == info.n_small
    assert info.plan_bytes == nbytes
    ib = info.item_bytes
    assert ib % 16 == 0 and 16 <= ib <= ITEM_MAX
    n_block = info.n_items - info.n_small
    by_row = {}
    for i, x in enumerate(items):
        by_row.setdefault(int(x["row"]), []).append((i, x))
    total = 0
    for k, (ptr, numel, dt, _) in enumerate(descs):
        es = ES[dt]
        has = ptr is not None and numel > 0
        its = by_row.get(k, [])
        if not has:
            assert not its
            continue
        total += numel * es
        its.sort(key=lambda p: int(p[1]["start"]))
        pos = 0
        for idx, x in its:
            assert int(x["start"]) == pos, (k, pos, x)
            assert int(x["addr"]) == ptr + pos * es
            assert int(x["df"]) & 0xFF == dt
            assert bool(int(x["df"]) & 0x200) == bool(descs[k][3] & 1)
            ln = int(x["len"])
            assert ln > 0
            if pos > 0:
                assert int(x["addr"]) % 16 == 0  # interior boundaries are aligned
            assert ln * es <= ib + 16 and ln * es <= ITEM_MAX + 16
            pos += ln
        assert pos == numel  # exact cover, no overlap
        whole = len(its) == 1
        for idx, x in its:
            assert bool(int(x["df"]) & WHOLE) == whole
            if idx >= n_block:  # wave item: whole tensor with a short body
                assert whole
                h = 0 if ptr % 16 == 0 else min(numel, (16 - ptr % 16) // es)
                assert (numel - h) * es // 16 <= WAVE_BODY_VECS
    assert total == info.total_bytes
    # split table: missing/empty tensors (count 0) and multi-item tensors
    srows = {int(r[0]): (int(r[1]), int(r[2])) for r in split}
    assert len(srows) == info.n_split
    used = np.zeros(info.n_slots, dtype=np.int64)
    for k, (ptr, numel, dt, _) in enumerate(descs):
        its = by_row.get(k, [])
        has = ptr is not None and numel > 0
        if not has:
            assert srows[k] == (0, 0)
        elif len(its) > 1:
            first, count = srows[k]
            assert count == len(its)
            slots = sorted(int(x["slot"]) for _, x in its)
            assert slots == list(range(first, first + count))
            used[first:first + count] += 1
        else:
            assert k not in srows
    assert np.all(used == 1)
    return info


@pytest.mark.parametrize("item_bytes", [0, 16, 48, 4096, 65536, 1 << 20, 4 << 20])
def test_random_lists_are_covered_exactly(item_bytes):
    rng = np.random.default_rng(item_bytes + 1)
    base = 0x7F0000000000
    descs = []
    for k in range(300):
        dt = int(rng.integers(0, 12))
        es = ES[dt]
        r = rng.random()
        if r < 0.05:
            descs.append((None, 0, dt, 0))
            continue
        numel = int(rng.integers(0, 20)) if r < 0.3 else int(np.exp(rng.uniform(0, np.log(3e6))))
        if item_bytes == 16:
            numel = min(numel, 20000)  # keep the item list small
        ptr = base + int(rng.integers(0, 1 << 20)) * 16 + int(rng.integers(0, 16 // es)) * es
        descs.append((ptr, numel, dt, int(rng.integers(0, 2))))
    info = check_plan(descs, item_bytes)
    assert info.n_items > 0


def test_wave_items_and_block_items_split_at_8k():
    base = 0x7F0000000000
    descs = [(base, 4096, 1, 0),          # 8 KiB bf16 aligned: a wave item
             (base + 2, 4096, 1, 0),      # misaligned: head 7, body 4089 -> 511 vectors + tail
             (base + 16, 4104, 1, 0),     # 513 vectors: a workgroup item
             (base, 2048, 0, 0),          # 8 KiB fp32
             (base, 2049, 0, 0),          # 512 vectors + a 1-element tail
             (base, 2052, 0, 0),          # 513 vectors: a workgroup item
             (base, 1, 2, 0)]
    img, info, _ = pack(descs, 0)
    _, items, _ = parse(img, info)
    n_block = info.n_items - info.n_small
    wave_rows = sorted(int(x["row"]) for x in items[n_block:])
    assert wave_rows == [0, 1, 3, 4, 6]
    check_plan(descs, 0)


def test_auto_item_size_policy():
    base = 0x7F0000000000
    big = [(base, 70_553_706_496 // 723, 1, 0)] * 723     # a 141 GB list
    assert check_plan(big, 0).item_bytes == 1 << 20
    small = [(base, 1000, 0, 0)] * 10
    assert check_plan(small, 0).item_bytes == 64 << 10
