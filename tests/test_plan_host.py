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
FULL_BODY_VECS = 512   # a wave item scanned by a whole wave: body <= 8 KiB
HALF_BODY_VECS = 256   # by half a wave: body <= 4 KiB
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
            h = 0 if ptr % 16 == 0 else min(numel, (16 - ptr % 16) // es)
            body = (numel - h) * es // 16
            if idx >= info.n_items - info.n_half:    # half-wave item
                assert whole and body <= HALF_BODY_VECS
            elif idx >= n_block:                     # full-wave item
                assert whole and HALF_BODY_VECS < body <= FULL_BODY_VECS
            elif whole:                              # workgroup item of a whole tensor
                assert body > FULL_BODY_VECS
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


def test_wave_item_classes():
    # aligned body <= 256 vectors (4 KiB): half a wave; <= 512 (8 KiB): a wave
    base = 0x7F0000000000
    descs = [(base, 2048, 1, 0),          # 4 KiB bf16 aligned: half wave
             (base + 2, 2048, 1, 0),      # misaligned: head 7, body 2041 -> 255 vectors + tail
             (base + 16, 2056, 1, 0),     # 257 vectors: a wave
             (base, 1024, 0, 0),          # 4 KiB fp32: half wave
             (base, 1025, 0, 0),          # 256 vectors + a 1-element tail: half wave
             (base, 1028, 0, 0),          # 257 vectors: a wave
             (base, 1, 2, 0),             # half wave
             (base, 4096, 1, 0),          # 8 KiB: a wave
             (base, 4104, 1, 0),          # 513 vectors: a workgroup item
             (base, 2049, 0, 0)]          # 512 vectors + tail: a wave
    img, info, _ = pack(descs, 0)
    _, items, _ = parse(img, info)
    n_block = info.n_items - info.n_small
    n_full = info.n_small - info.n_half
    full_rows = sorted(int(x["row"]) for x in items[n_block:n_block + n_full])
    half_rows = sorted(int(x["row"]) for x in items[n_block + n_full:])
    assert half_rows == [0, 1, 3, 4, 6]
    assert full_rows == [2, 5, 7, 9]
    check_plan(descs, 0)


def test_wave_items_are_grouped_by_type():
    # each class of wave items is stored grouped by element type (stable within a type)
    base = 0x7F0000000000
    dts = [0, 1, 2, 1, 0, 2, 2, 1, 0, 0]
    sizes = [100, 3000, 3000, 100, 1500, 100, 3000, 100, 1500, 100]   # half / full classes
    descs = [(base + (1 << 16) * k, n, dt, 0) for k, (dt, n) in enumerate(zip(dts, sizes))]
    img, info, _ = pack(descs, 0)
    _, items, _ = parse(img, info)
    n_block = info.n_items - info.n_small
    n_full = info.n_small - info.n_half
    for lo, hi in ((n_block, n_block + n_full), (n_block + n_full, info.n_items)):
        got = [(int(x["df"]) & 0xFF, int(x["row"])) for x in items[lo:hi]]
        assert got == sorted(got)
    assert n_full == 5 and info.n_half == 5
    check_plan(descs, 0)


def test_auto_item_size_policy():
    base = 0x7F0000000000
    big = [(base, 70_553_706_496 // 723, 1, 0)] * 723     # a 141 GB list
    assert check_plan(big, 0).item_bytes == 1 << 20
    small = [(base, 1000, 0, 0)] * 10
    assert check_plan(small, 0).item_bytes == 64 << 10
