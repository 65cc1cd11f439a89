"""The asynchronous entry points on non-default streams, concurrently on two
streams, and captured into a HIP graph (through torch.cuda.CUDAGraph) and
replayed several times with eager work and data changes between replays.
Every result is checked against the oracle or against the same call made
eagerly; no call inside the graph synchronises or allocates device memory in
the library.
"""
import numpy as np
import pytest
import torch

import oracle as O
import silent_corruption_detection_amd as sdc
import workloads as W
from _util import assert_rows_equal, oracle_nonfinite, oracle_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def mixed_list(seed):
    """Wave items, whole workgroup items and split tensors, three dtypes, a
    misaligned view, and NaN/Inf values."""
    g = gen(seed)
    out = []
    for n, dt in ((100, torch.float32), (3_000, torch.bfloat16), (40_000, torch.float16),
                  (2_500_001, torch.float32), (7_000_003, torch.bfloat16), (1, torch.float16)):
        t = torch.empty(n + 3, dtype=torch.float32, device=DEV).normal_(0, 0.02, generator=g)
        out.append(t.to(dt)[1:n + 1])   # misaligned start for 2-byte types
    W.write_pattern(out[3], 17, 0x7FC00000)
    W.write_pattern(out[4], 1_000_000, 0xFF80)
    return out


# item sizes of the plans and single-tensor scans: automatic (short launch
# shape for these lists), and 1 MiB (the wide shapes: one workgroup per CU
# through a dynamic-LDS reservation, for the plans and the single tensors)
ITEMS = [0, 1 << 20]


@pytest.mark.parametrize("ib", ITEMS)
def test_two_streams_concurrently(ib):
    a, b = mixed_list(1), mixed_list(2)
    pa, pb = sdc.sdc_plan_build(a, item_bytes=ib), sdc.sdc_plan_build(b, item_bytes=ib)
    if ib:
        assert pa.total_bytes // pa.n_items >= 512 << 10
    oa = torch.empty((len(a), 4), dtype=torch.int64, device=DEV)
    ob = torch.empty_like(oa)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    say(f"case two streams item_bytes={ib}")
    for _ in range(5):
        with torch.cuda.stream(s1):
            sdc.sdc_fingerprint_plan(pa, oa)
        with torch.cuda.stream(s2):
            sdc.sdc_fingerprint_plan(pb, ob)
    torch.cuda.synchronize()
    assert_rows_equal(sdc.rows_numpy(oa), oracle_rows(a))
    assert_rows_equal(sdc.rows_numpy(ob), oracle_rows(b))
    # single-tensor scans on both streams, each with its own reused workspace
    ta, tb = a[4], b[3]
    wa = torch.empty(sdc.sdc_tensor_ws_bytes(ta, item_bytes=ib), dtype=torch.uint8, device=DEV)
    wb = torch.empty(sdc.sdc_tensor_ws_bytes(tb, item_bytes=ib), dtype=torch.uint8, device=DEV)
    ra = torch.empty((1, 4), dtype=torch.int64, device=DEV)
    rb = torch.empty_like(ra)
    for _ in range(5):
        with torch.cuda.stream(s1):
            sdc.sdc_fingerprint_tensor(ta, out=ra, ws=wa, item_bytes=ib)
        with torch.cuda.stream(s2):
            sdc.sdc_fingerprint_tensor(tb, out=rb, ws=wb, item_bytes=ib)
    torch.cuda.synchronize()
    assert_rows_equal(sdc.rows_numpy(ra), oracle_rows([ta]))
    assert_rows_equal(sdc.rows_numpy(rb), oracle_rows([tb]))


@pytest.mark.parametrize("ib", ITEMS)
def test_graph_capture_and_replay(ib):
    ts = mixed_list(3)
    big = ts[4]
    plan = sdc.sdc_plan_build(ts, item_bytes=ib)
    n = len(ts)
    rows = torch.empty((n, 4), dtype=torch.int64, device=DEV)
    counts = torch.empty(n, dtype=torch.int64, device=DEV)
    total = torch.empty(1, dtype=torch.int64, device=DEV)
    sq = torch.empty(n, dtype=torch.float64, device=DEV)
    sq_total = torch.empty(1, dtype=torch.float64, device=DEV)
    flag = torch.empty(1, dtype=torch.int32, device=DEV)
    ws = torch.empty(sdc.sdc_tensor_ws_bytes(big, item_bytes=ib), dtype=torch.uint8, device=DEV)
    ref = sdc.sdc_fingerprint_tensor(big).clone()
    one = torch.empty((1, 4), dtype=torch.int64, device=DEV)
    mis = torch.zeros(1, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()

    def work():
        mis.zero_()
        sdc.sdc_fingerprint_plan(plan, rows)
        sdc.sdc_nonfinite(plan, counts, total)
        sdc.sdc_sqnorm(plan, sq, sq_total, flag)
        sdc.sdc_fingerprint_tensor(big, out=one, ref=ref, mismatch=mis, ws=ws, item_bytes=ib)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say(f"case graph capture item_bytes={ib}")
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()

    for rep in range(4):
        if rep == 2:   # change the data between replays: a flip in the big tensor
            W.flip_bit(big, 123_457, 5)
        for x in (rows, counts, total, sq, sq_total, flag, one):   # stale outputs
            x.fill_(-1) if x.dtype != torch.float64 else x.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"case graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = (sdc.rows_numpy(rows).copy(), counts.cpu().clone(), int(total.item()),
               sq.cpu().clone(), float(sq_total.item()), int(flag.item()), sdc.rows_numpy(one).copy(),
               int(mis.item()))
        # eager work between replays, then the same calls made eagerly
        torch.randn(1 << 20, device=DEV).sum().item()
        e_rows = sdc.rows_numpy(sdc.sdc_fingerprint_plan(plan)).copy()
        e_counts, e_total = sdc.sdc_nonfinite(plan)
        e_sq, e_sqt, e_flag = sdc.sdc_sqnorm(plan)
        e_one = sdc.rows_numpy(sdc.sdc_fingerprint_tensor(big)).copy()
        torch.cuda.synchronize()
        assert np.array_equal(got[0], e_rows)
        assert_rows_equal(got[0], oracle_rows(ts))
        assert torch.equal(got[1], e_counts.cpu()) and got[2] == int(e_total.item())
        assert got[1].numpy().astype(np.uint64).tolist() == oracle_nonfinite(ts).tolist()
        assert np.array_equal(got[3].numpy().view(np.uint64), e_sq.cpu().numpy().view(np.uint64))
        assert (np.isnan(got[4]) and np.isnan(float(e_sqt.item()))) or got[4] == float(e_sqt.item())
        assert got[5] == int(e_flag.item()) == 1    # the list holds a NaN
        assert np.array_equal(got[6], e_one)
        assert got[7] == (1 if rep >= 2 else 0)


def test_strided_inputs_scanned_on_a_side_stream():
    # The binding makes contiguous copies of strided inputs (and allocates
    # the workspace and output) on the current stream; a scan on another
    # stream must still read the finished copies.  The copies are made right
    # after a long kernel on the current stream, so a side stream that did not
    # wait would run ahead of them.
    g = gen(11)
    base = [torch.empty((2048, 3000), dtype=torch.float32, device=DEV).normal_(0, 0.02, generator=g),
            torch.empty((777, 4096), dtype=torch.bfloat16, device=DEV).normal_(0, 0.02, generator=g)]
    views = [base[0].t(), base[1][:, ::3], base[0][5:, 1::2].t()]
    assert not any(v.is_contiguous() for v in views)
    ref = oracle_rows([v.contiguous() for v in views])
    big = torch.empty(1 << 28, dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"case strided side stream rep={rep}")
        big.add_(1.0)  # keeps the current stream busy while the copies are enqueued behind it
        rows = sdc.sdc_fingerprint(views, stream=side)
        one = [sdc.sdc_fingerprint_tensor(v, stream=side) for v in views]
        side.synchronize()
        assert_rows_equal(sdc.rows_numpy(rows), ref)
        assert_rows_equal(np.concatenate([sdc.rows_numpy(o) for o in one]), ref)
    torch.cuda.synchronize()
