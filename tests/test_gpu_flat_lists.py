"""Lists of tensors that lie back to back in one flat buffer (the layout of
gradient-bucket views) against the oracle, element by element.

The lists are views carved from one device byte buffer of random bits (so
every NaN/Inf encoding and every sign pattern occurs), at element-aligned
offsets with gaps of 0..15 bytes, so tensor boundaries fall at every byte
offset inside 16-byte vectors and between tensors of different element
types, and neighbouring tensors share vectors; tensors of 1 element to
256 KiB; long clusters of 1..3-element tensors; and missing, empty, large,
overlapping and far-away tensors in between.  The NaN/Inf-count and
squared-norm scans of the same plans are checked too.
"""
import numpy as np
import pytest
import torch

import oracle as O
import silent_corruption_detection_amd as sdc
from _util import CODE, assert_rows_equal, assert_sq_close, oracle_sqnorms, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
ALL = [torch.float32, torch.bfloat16, torch.float16, torch.float64, torch.uint8,
       torch.float8_e4m3fn, torch.float8_e5m2, torch.float8_e4m3fnuz, torch.float8_e5m2fnuz,
       torch.int16, torch.int32, torch.int64]


def carve(seed, n, dtypes, max_numel, gap_max=15, lead=0, nbytes_cap=None):
    """(flat buffer, host copy, [(offset, numel, dtype)]) of n tensors."""
    rng = np.random.default_rng(seed)
    layout, off = [], lead
    for _ in range(n):
        dt = dtypes[int(rng.integers(0, len(dtypes)))]
        es = torch.empty(0, dtype=dt).element_size()
        numel = max(1, min(max_numel, int(np.exp(rng.uniform(0, np.log(max_numel + 1))))))
        off += int(rng.integers(0, gap_max + 1))
        off = -(-off // es) * es
        layout.append((off, numel, dt))
        off += numel * es
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    buf = torch.randint(0, 256, (off + 64,), dtype=torch.uint8, device=DEV, generator=g)
    return buf, layout


def views(buf, layout):
    return [buf[o:o + n * torch.empty(0, dtype=dt).element_size()].view(dt) for o, n, dt in layout]


def oracle_of(buf, layout, flags=0):
    h = buf.cpu().numpy()
    out = np.zeros((len(layout), 4), dtype=np.uint64)
    for k, (o, n, dt) in enumerate(layout):
        if n:
            es = torch.empty(0, dtype=dt).element_size()
            out[k] = O.fingerprint(h[o:o + n * es], CODE[dt], flags)
    return out


def scan(ts, **kw):
    plan = sdc.sdc_plan_build(ts, **kw)
    rows = sdc.rows_numpy(sdc.sdc_fingerprint_plan(plan))
    torch.cuda.synchronize()
    return plan, rows


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("ib", [0, 1 << 20])
def test_flat_buffer_all_types(seed, ib):
    buf, layout = carve(seed, 3000, ALL, 65536)
    ts = views(buf, layout)
    say(f"case flat list all types seed={seed} item_bytes={ib}")
    plan, rows = scan(ts, item_bytes=ib)
    ref = oracle_of(buf, layout)
    assert_rows_equal(rows, ref)
    # the page's sign-extended mode over the same list
    _, srows = scan(ts, item_bytes=ib, signed=True)
    assert_rows_equal(srows, oracle_of(buf, layout, O.SIGNED))
    counts, total = sdc.sdc_nonfinite(plan)
    torch.cuda.synchronize()
    assert counts.cpu().numpy().astype(np.uint64).tolist() == ref[:, 3].tolist()
    assert int(total.item()) == int(ref[:, 3].sum())


@pytest.mark.parametrize("dts", [(torch.float32, torch.bfloat16, torch.float16),
                                 (torch.float16, torch.uint8), (torch.float64, torch.int16),
                                 (torch.bfloat16,), (torch.float8_e4m3fn, torch.int32)])
def test_boundaries_at_every_offset(dts):
    # tensors of 1..40 elements back to back: every boundary position inside a
    # vector, every pair of neighbouring types, lead offsets 0..15
    for lead in range(16):
        buf, layout = carve(100 + lead, 400, list(dts), 40, gap_max=3, lead=lead)
        ts = views(buf, layout)
        plan, rows = scan(ts)
        assert_rows_equal(rows, oracle_of(buf, layout))


def test_tiny_clusters_and_mixed_sizes():
    # clusters of 1..3-element tensors between large ones (random bits, rich
    # in NaN/Inf)
    rng = np.random.default_rng(9)
    layout, off = [], 0
    for blk in range(40):
        if blk % 2:
            for _ in range(int(rng.integers(50, 400))):
                dt = [torch.bfloat16, torch.float32, torch.uint8][int(rng.integers(0, 3))]
                es = torch.empty(0, dtype=dt).element_size()
                off = -(-off // es) * es
                n = int(rng.integers(1, 4))
                layout.append((off, n, dt))
                off += n * es
        else:
            dt = [torch.bfloat16, torch.float16, torch.float32][blk % 3]
            es = torch.empty(0, dtype=dt).element_size()
            off = -(-off // es) * es
            n = int(rng.integers(1, (256 << 10) // es + 1))
            layout.append((off, n, dt))
            off += n * es
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
    buf = torch.randint(0, 256, (off + 64,), dtype=torch.uint8, device=DEV, generator=g)
    ts = views(buf, layout)
    plan, rows = scan(ts, item_bytes=1 << 20)
    assert_rows_equal(rows, oracle_of(buf, layout))


def test_missing_empty_large_and_overlapping_neighbours():
    buf, layout = carve(21, 600, [torch.float32, torch.bfloat16, torch.float16], 5000)
    ts = views(buf, layout)
    other = torch.randn(1 << 20, device=DEV)
    ts[50] = None                                   # missing
    ts[100] = ts[100][:0]                           # empty
    ts[150] = other                                 # far away (and 4 MiB)
    ts[200] = ts[199]                               # the same tensor again (overlaps)
    ts[250] = ts[249][1:]                           # overlapping view
    ts[300] = other[:1000]                          # far away small
    plan, rows = scan(ts)
    ref = np.zeros((len(ts), 4), dtype=np.uint64)
    for k, t in enumerate(ts):
        if t is not None and t.numel():
            ref[k] = O.fingerprint(t.contiguous().view(torch.uint8).cpu().numpy(), CODE[t.dtype])
    assert_rows_equal(rows, ref)
    sq, total, flag = sdc.sdc_sqnorm(plan)
    torch.cuda.synchronize()
    assert_sq_close(sq.cpu().tolist(), oracle_sqnorms(ts), [0 if t is None else t.numel() for t in ts])


def test_repeated_scans_and_one_shot():
    buf, layout = carve(31, 2000, [torch.float32, torch.bfloat16, torch.float16], 65536)
    ts = views(buf, layout)
    plan = sdc.sdc_plan_build(ts)
    out = torch.full((len(ts), 4), -1, dtype=torch.int64, device=DEV)
    ref = oracle_of(buf, layout)
    for _ in range(3):
        sdc.sdc_fingerprint_plan(plan, out)
        torch.cuda.synchronize()
        assert_rows_equal(sdc.rows_numpy(out), ref)
        out.fill_(-1)
    assert_rows_equal(sdc.rows_numpy(sdc.sdc_fingerprint(ts)), ref)
