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
# wave items of class c are scanned by 64 >> c lanes: aligned body <= 512 >> c vectors
CLASS_BODY_VECS = [512, 256, 128, 64]
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


def class_of(info, idx):
    """Wave-item class of plan item idx (items of class 0..3 follow the workgroup items)."""
    start = info.n_items - info.n_small
    for c in range(4):
        start += info.n_wave[c]
        if idx < start:
            return c
    raise AssertionError("not a wave item")


def check_plan(descs, item_bytes):
    img, info, nbytes = pack(descs, item_bytes)
    hdr, items, split = parse(img, info)
    assert int(hdr[1]) == len(descs) == info.n_tensors
    assert int(hdr[2]) == info.n_items and int(hdr[3]) == info.n_split
    assert int(hdr[4]) == info.n_slots and int(hdr[7]) == info.n_small
    assert sum(info.n_wave) == info.n_small
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
            if idx >= n_block:                       # wave item: the narrowest class that fits
                assert whole
                c = class_of(info, idx)
                assert body <= CLASS_BODY_VECS[c]
                assert c == 3 or body > CLASS_BODY_VECS[c + 1]
            elif whole:                              # workgroup item of a whole tensor
                assert body > CLASS_BODY_VECS[0]
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


def flat_list(rng, n, base=0x7F0000000000, gap_max=3, dts=(0, 1, 2), max_numel=65536):
    """Tensors carved back to back from one flat buffer at element-aligned
    offsets (plus random gaps of up to gap_max bytes), like gradient-bucket views."""
    descs, off = [], 0
    for _ in range(n):
        dt = int(rng.choice(dts))
        es = ES[dt]
        numel = min(max_numel, int(np.exp(rng.uniform(0, np.log(max_numel + 1)))))
        off += int(rng.integers(0, gap_max + 1))
        off = -(-off // es) * es
        descs.append((base + off, numel, dt, int(rng.integers(0, 2))))
        off += numel * es
    return descs


@pytest.mark.parametrize("item_bytes", [0, 4096, 1 << 20])
def test_flat_buffer_lists_are_covered_exactly(item_bytes):
    # neighbouring tensors share 16-byte vectors; each is still covered
    # exactly by its own items, whose heads and tails are read element-wise
    rng = np.random.default_rng(item_bytes + 7)
    check_plan(flat_list(rng, 2000, dts=(0, 1, 2, 3, 4, 5, 9, 10, 11)), item_bytes)
    check_plan(flat_list(rng, 1000, max_numel=3), item_bytes)


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
    # aligned body <= 64 vectors (1 KiB): 8 lanes; <= 128: 16; <= 256: 32; <= 512 (8 KiB): 64
    base = 0x7F0000000000
    descs = [(base, 2048, 1, 0),          # 4 KiB bf16 aligned: 256 vectors, class 1
             (base + 2, 2048, 1, 0),      # misaligned: head 7, body 2041 -> 255 vectors + tail: 1
             (base + 16, 2056, 1, 0),     # 257 vectors: class 0
             (base, 1024, 0, 0),          # 4 KiB fp32: class 1
             (base, 1025, 0, 0),          # 256 vectors + a 1-element tail: class 1
             (base, 1028, 0, 0),          # 257 vectors: class 0
             (base, 1, 2, 0),             # no body: class 3
             (base, 4096, 1, 0),          # 8 KiB: class 0
             (base, 4104, 1, 0),          # 513 vectors: a workgroup item
             (base, 2049, 0, 0),          # 512 vectors + tail: class 0
             (base, 256, 0, 0),           # 64 vectors: class 3
             (base, 257, 0, 0),           # 64 vectors + tail: class 3
             (base, 260, 0, 0),           # 65 vectors: class 2
             (base + 1, 2048, 4, 0),      # u8, head 15, body 2033 B -> 127 vectors + tail: 2
             (base, 1024, 1, 0)]          # 2 KiB = 128 vectors: class 2
    img, info, _ = pack(descs, 0)
    _, items, _ = parse(img, info)
    n_block = info.n_items - info.n_small
    rows = [sorted(int(items[i]["row"]) for i in range(n_block, info.n_items) if class_of(info, i) == c)
            for c in range(4)]
    assert rows == [[2, 5, 7, 9], [0, 1, 3, 4], [12, 13, 14], [6, 10, 11]]
    check_plan(descs, 0)


def test_wave_items_are_grouped_by_type():
    # each class of wave items is stored grouped by element type (stable within a type)
    base = 0x7F0000000000
    dts = [0, 1, 2, 1, 0, 2, 2, 1, 0, 0]
    sizes = [100, 3000, 3000, 100, 1500, 100, 3000, 100, 1500, 100]
    descs = [(base + (1 << 16) * k, n, dt, 0) for k, (dt, n) in enumerate(zip(dts, sizes))]
    img, info, _ = pack(descs, 0)
    _, items, _ = parse(img, info)
    lo = info.n_items - info.n_small
    for c in range(4):
        hi = lo + info.n_wave[c]
        got = [(int(x["df"]) & 0xFF, int(x["row"])) for x in items[lo:hi]]
        assert got == sorted(got)
        lo = hi
    assert list(info.n_wave) == [5, 0, 0, 5]
    check_plan(descs, 0)


def test_auto_item_size_policy():
    base = 0x7F0000000000
    big = [(base, 70_553_706_496 // 723, 1, 0)] * 723     # a 141 GB list
    assert check_plan(big, 0).item_bytes == 1 << 20
    small = [(base, 1000, 0, 0)] * 10
    assert check_plan(small, 0).item_bytes == 64 << 10
