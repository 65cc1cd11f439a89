"""GPU tests of the plan-free single-tensor scan and the recompute audit built
on it (AEGIS review page, section "core method", item 4: fingerprints of an
original and its deterministic recomputation, compared bit for bit).

- sdc_fingerprint_tensor rows equal the oracle's for every element type, both
  widening modes, sizes across several items with ragged tails and every
  misaligned start; the device compare counts exactly the rows that differ
  from the reference under each column mask.
- The audit on a small random-init checkpointed MLP (fp32 and bf16): a clean
  step has no mismatch and its rows equal the oracle's rows of the captured
  outputs; a bit flipped in a saved segment input between forward and
  backward (the page's case of a corrupted saved intermediate) is reported
  for exactly that segment; a bit flipped in one segment's recomputed output
  is reported for that segment with the flipped element and bit.
"""
import numpy as np
import pytest
import torch
import torch.utils.checkpoint as cp

import oracle as O
import silent_corruption_detection_amd as sdc
from silent_corruption_detection_amd.recompute import RecomputeAudit
import workloads as W
from _util import CODE, assert_rows_equal, host_bytes, oracle_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
TYPES = [torch.float32, torch.bfloat16, torch.float16, torch.float64, torch.uint8,
         torch.float8_e4m3fn, torch.float8_e5m2fnuz, torch.int16, torch.int32, torch.int64]


def gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def carve(buf, offset, n, dtype):
    es = torch.empty(0, dtype=dtype).element_size()
    return buf[offset:offset + n * es].view(dtype)


def one_row(t, signed=False):
    r = sdc.sdc_fingerprint_tensor(t, signed=signed)
    torch.cuda.synchronize()
    return sdc.rows_numpy(r)


@pytest.mark.parametrize("dtype", TYPES, ids=[str(t).split(".")[1] for t in TYPES])
def test_tensor_rows_match_the_oracle(dtype):
    es = torch.empty(0, dtype=dtype).element_size()
    for n in (1, 7, 8, 9, 4097, 65537, 1_000_003, 9_000_011):
        raw = torch.randint(0, 256, (n * es + 16,), dtype=torch.uint8, device=DEV, generator=gen(n))
        for off in sorted({0, es, 16 - es}):
            t = carve(raw, off, n, dtype)
            for signed in (False, True):
                say(f"case tensor dtype={dtype} n={n} off={off} signed={signed}")
                ref = oracle_rows([t], flags=O.SIGNED if signed else 0)
                assert_rows_equal(one_row(t, signed), ref)


def test_tensor_rows_do_not_depend_on_the_item_size():
    g = gen(3)
    for dtype, n, off in ((torch.bfloat16, 5_000_003, 6), (torch.float32, 2_000_001, 4),
                          (torch.uint8, 3_333_333, 5), (torch.float64, 700_001, 8)):
        es = torch.empty(0, dtype=dtype).element_size()
        buf = torch.randint(0, 256, (n * es + 16,), dtype=torch.uint8, device=DEV, generator=g)
        t = carve(buf, off, n, dtype)
        ref = oracle_rows([t])
        for ib in (0, 16, 48, 4096, 65536, 1 << 20, 4 << 20):
            say(f"case tensor items dtype={dtype} item_bytes={ib}")
            r = sdc.sdc_fingerprint_tensor(t, item_bytes=ib)
            torch.cuda.synchronize()
            assert_rows_equal(sdc.rows_numpy(r), ref)


def test_tensor_automatic_split_around_128_mib():
    # tensors of at least 128 MiB are cut into one item per CU (the tensor-wide
    # launch shape), smaller ones into about 1024 items: rows equal the oracle's
    # on both sides of the threshold, with misaligned starts and ragged tails
    g = gen(7)
    for dtype, nbytes, off in ((torch.float32, 128 << 20, 4), (torch.float32, (128 << 20) - 4, 0),
                               (torch.bfloat16, 300 << 20, 6), (torch.uint8, (128 << 20) + 1, 3)):
        es = torch.empty(0, dtype=dtype).element_size()
        buf = torch.randint(0, 256, (nbytes + 16,), dtype=torch.uint8, device=DEV, generator=g)
        t = carve(buf, off, nbytes // es, dtype)
        say(f"case tensor automatic split dtype={dtype} bytes={nbytes} off={off}")
        assert_rows_equal(one_row(t), oracle_rows([t]))
        del buf, t


def test_tensor_empty_missing_and_large():
    assert one_row(torch.empty(0, device=DEV)).tolist() == [[0, 0, 0, 0]]
    # a 2 GiB bf16 tensor (the Llama-70B embedding's size) equals the list scan's row
    g = gen(5)
    t = torch.empty(128256 * 8192, dtype=torch.bfloat16, device=DEV).normal_(0, 0.02, generator=g)
    plan = sdc.sdc_plan_build([t])
    a = sdc.rows_numpy(sdc.sdc_fingerprint_plan(plan))
    # the whole tensor against the oracle (2.1 GB, one oracle call), and the
    # list scan of the same tensor
    say("case tensor 2 GiB bf16: oracle over the whole tensor")
    ref = oracle_rows([t])
    assert_rows_equal(one_row(t), ref)
    assert_rows_equal(a, ref)
    # and a slice that spans items and a ragged tail
    s = t[:3_000_001]
    assert_rows_equal(one_row(s), oracle_rows([s]))
    del t, plan


def test_tensor_caller_workspace_too_small_or_empty():
    # a caller workspace smaller than the tensor's split needs, or an empty
    # one, is replaced for that call (the library refuses it before queuing
    # anything); the row and the compare are those of a right-sized one
    g = gen(17)
    t = torch.empty(5_000_003, dtype=torch.float32, device=DEV).normal_(0, 1, generator=g)
    ref = oracle_rows([t])
    need = sdc.sdc_tensor_ws_bytes(t)
    assert need > 64
    good = torch.tensor(ref.view(np.int64), device=DEV)
    mis = torch.zeros(1, dtype=torch.int32, device=DEV)
    for nb in (0, 32, need - 32, need):
        ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
        say(f"case tensor caller workspace of {nb} bytes (needs {need})")
        out = torch.full((1, 4), -1, dtype=torch.int64, device=DEV)
        sdc.sdc_fingerprint_tensor(t, out=out, ws=ws)
        assert_rows_equal(sdc.rows_numpy(out), ref)
        sdc.sdc_fingerprint_tensor(t, out=out, ref=good, mismatch=mis, ws=ws)
        torch.cuda.synchronize()
        assert mis.item() == 0
    with pytest.raises(ValueError):  # a workspace on the host is refused, not replaced
        sdc.sdc_fingerprint_tensor(t, ws=torch.empty(need, dtype=torch.uint8))


def test_audit_workspace_across_the_wide_split():
    # the audit asks for a workspace size only when a larger tensor comes:
    # outputs that grow past 128 MiB and shrink again all give the oracle's rows
    g = gen(19)
    sizes = [1_000_003, (128 << 20) // 4 + 5, 7_777_777, (300 << 20) // 4 + 1, (128 << 20) // 4 - 9]
    ts = [torch.empty(n, dtype=torch.float32, device=DEV).normal_(0, 1, generator=g) for n in sizes]
    audit = RecomputeAudit(len(ts), device=DEV)
    audit.begin_step()
    for k, t in enumerate(ts):
        say(f"case audit workspace segment {k} numel={t.numel()}")
        audit.record(k, t)
    for k, t in enumerate(ts):   # the recomputation: same tensors
        audit.record(k, t)
    res = audit.result()
    assert res["mismatched"] == [] and res["not_recomputed"] == []
    orig, again = audit.rows()
    ref = oracle_rows(ts)
    assert_rows_equal(orig, ref)
    assert_rows_equal(again, ref)
    del ts


def test_tensor_compare_counts_and_masks():
    g = gen(9)
    t = torch.empty(300_001, dtype=torch.float32, device=DEV).normal_(0, 1, generator=g)
    good = sdc.sdc_fingerprint_tensor(t).clone()
    mis = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.empty((1, 4), dtype=torch.int64, device=DEV)
    for _ in range(3):
        sdc.sdc_fingerprint_tensor(t, out=out, ref=good, mismatch=mis)
    torch.cuda.synchronize()
    assert int(mis.item()) == 0 and torch.equal(out, good)
    # each column of the reference perturbed in turn: counted under masks that include it
    for col in range(4):
        bad = good.clone()
        bad[0, col] += 1
        for mask in (1, 2, 4, 8, 3, 15):
            mis.zero_()
            sdc.sdc_fingerprint_tensor(t, out=out, ref=bad, mismatch=mis, col_mask=mask)
            torch.cuda.synchronize()
            assert int(mis.item()) == int(bool(mask & (1 << col))), (col, mask)
    # a flip in the data: counted, and the flip localised from the two rows
    idx, bit = 123_457, 22
    W.flip_bit(t, idx, bit)
    mis.zero_()
    sdc.sdc_fingerprint_tensor(t, out=out, ref=good, mismatch=mis)
    d = sdc.sdc_fingerprint_diff(good, out)
    assert int(mis.item()) == 1 and d["indices"] == [0] and d["hints"][0][:2] == (idx, bit)


def test_tensor_rejects_bad_arguments():
    t = torch.ones(10, device=DEV)
    row = torch.zeros((1, 4), dtype=torch.int64, device=DEV)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        sdc.sdc_fingerprint_tensor(t, ref=row)                 # a compare needs a counter
    for mask in (0, 16, 31):
        with pytest.raises(sdc.SdcError):
            sdc.sdc_fingerprint_tensor(t, ref=row, mismatch=cnt, col_mask=mask)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 0


# ---- the audit on a checkpointed model --------------------------------------------

class Block(torch.nn.Module):
    def __init__(self, d):
        super().__init__()
        self.lin = torch.nn.Linear(d, d)
        self.norm = torch.nn.LayerNorm(d)

    def forward(self, x):
        return self.norm(torch.nn.functional.gelu(self.lin(x)))


def make_model(d, n, dtype, seed):
    torch.manual_seed(seed)
    return torch.nn.ModuleList([Block(d) for _ in range(n)]).to(device=DEV, dtype=dtype)


def run_step(model, x, audit, reentrant, faults=None, corrupt=None, capture=None):
    """One forward + backward with every block checkpointed.  faults[k](out, call)
    may change block k's output; corrupt(inputs) runs between forward and
    backward; capture collects (k, call, output copy)."""
    audit.begin_step()
    calls = [0] * len(model)
    inputs = []

    def seg(k):
        def f(h):
            out = model[k](h)
            c = calls[k]
            calls[k] += 1
            if faults and k in faults:
                faults[k](out, c)
            if capture is not None:
                capture.append((k, c, out.detach().clone()))
            return out
        return audit.wrap(f, k)

    h = x
    # the setting is taken when checkpoint() runs, so it wraps the forward pass
    with cp.set_checkpoint_early_stop(False):
        for k in range(len(model)):
            inputs.append(h)
            h = cp.checkpoint(seg(k), h, use_reentrant=reentrant)
    loss = h.float().pow(2).mean()
    if corrupt:
        corrupt(inputs)
    loss.backward()
    return audit.result()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("reentrant", [True, False])
def test_clean_step_has_no_mismatch_and_rows_match_the_oracle(dtype, reentrant):
    n, d = 4, 512
    model = make_model(d, n, dtype, seed=1)
    x = torch.randn(2048, d, device=DEV, dtype=dtype, generator=gen(2)).requires_grad_(True)
    audit = RecomputeAudit(n)
    cap = []
    say(f"case audit clean dtype={dtype} reentrant={reentrant}")
    res = run_step(model, x, audit, reentrant, capture=cap)
    assert res["mismatched"] == [] and res["not_recomputed"] == [] and res["not_run"] == []
    orig, rec = audit.rows()
    assert np.array_equal(orig, rec)
    first = {k: t for k, c, t in cap if c == 0}
    assert_rows_equal(orig, oracle_rows([first[k] for k in range(n)]))
    # the next step starts clean
    res = run_step(model, x, audit, reentrant)
    assert res["mismatched"] == []


@pytest.mark.parametrize("reentrant", [True, False])
def test_corrupted_saved_input_is_caught_in_its_segment(reentrant):
    n, d = 4, 512
    model = make_model(d, n, torch.float32, seed=3)
    x = torch.randn(1024, d, device=DEV, generator=gen(4)).requires_grad_(True)
    audit = RecomputeAudit(n)

    def corrupt(inputs):
        # a silent bit flip in the saved input of block 2 (no autograd version bump)
        W.flip_bit(inputs[2].data, 77_777, 27)
    say(f"case audit saved-input flip reentrant={reentrant}")
    res = run_step(model, x, audit, reentrant, corrupt=corrupt)
    assert res["mismatched"] == [2]


def test_flip_in_a_recomputed_output_is_localised():
    n, d = 3, 256
    model = make_model(d, n, torch.float32, seed=5)
    x = torch.randn(512, d, device=DEV, generator=gen(6)).requires_grad_(True)
    audit = RecomputeAudit(n)
    idx, bit = 4_321, 9

    def fault(out, call):
        if call == 1:  # only the recomputation goes wrong (a transient fault)
            W.flip_bit(out.data.reshape(-1), idx, bit)
    say("case audit recompute-output flip")
    res = run_step(model, x, audit, reentrant=True, faults={1: fault})
    assert res["mismatched"] == [1]
    i, b, _ = res["hints"][1]
    assert (i, b) == (idx, bit)


def test_segments_with_several_outputs():
    # a segment returning (hidden, residual): each output has its own row; a
    # flip in the recomputed residual is reported for that segment and output
    n, d = 3, 256
    model = make_model(d, n, torch.float32, seed=8)
    x = torch.randn(512, d, device=DEV, generator=gen(9)).requires_grad_(True)
    audit = RecomputeAudit(n, outputs=2)
    calls = [0] * n

    def seg(k):
        def f(h, r):
            out = model[k](h)
            res = r + out
            if k == 1 and calls[k] == 1:   # the recomputation of segment 1 goes wrong
                W.flip_bit(res.data.reshape(-1), 777, 3)
            calls[k] += 1
            return out, res
        return audit.wrap(f, k)

    audit.begin_step()
    h, r = x, torch.zeros_like(x)
    for k in range(n):
        h, r = cp.checkpoint(seg(k), h, r, use_reentrant=True)
    (h.float().pow(2).mean() + r.float().pow(2).mean()).backward()
    res = audit.result()
    assert res["mismatched"] == [1] and res["outputs"] == {1: [1]}
    assert res["hints"][1][:2] == (777, 3)
    orig, rec = audit.rows()
    assert np.array_equal(np.delete(orig, 3, axis=0), np.delete(rec, 3, axis=0))
