"""The pages' injected weight faults, end to end on the GPU (AWS blog post,
sections "Fault scenarios" and "Compare by fingerprint"; fixture
tests/golden/fault_kinds.json): each fault is applied to one of three replicas
of a small GPT-style parameter list, and then
  - the GPU rows equal the oracle's;
  - the strict-majority compare names exactly the faulted replica, under all
    four columns and under the pages' own two columns (sum, weighted sum);
  - the plain sum alone catches the fault exactly when the fixture says so
    (a swap and a +-4096 compensating change leave it unchanged: that is
    what the weighted sum is for);
  - the diff against a clean replica names exactly the faulted tensor, and a
    single bit flip is localised to its element and bit.
And the worked example of section "Step 1" (one weight on three replicas,
fixture tests/golden/worked_example.json) computed on the GPU: the update
lands on the same bits everywhere; a wrong local gradient changes every copy
alike (the majority cannot see it, and being finite the NaN/Inf check passes
it); a weight corrupted on one replica after the step is named.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
import silent_corruption_detection_amd as sdc
import workloads as W
from _util import assert_rows_equal, oracle_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
HERE = os.path.dirname(os.path.abspath(__file__))
CASES = json.load(open(os.path.join(HERE, "golden", "fault_kinds.json")))["cases"]


def replicas(dtype, seed):
    shapes = W.gpt_shapes(d=256, layers=2, vocab=1000)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    base = [torch.empty(s, dtype=torch.float32, device=DEV).normal_(0, 0.02, generator=g).to(dtype)
            for _, s, _ in shapes]
    return [[t.clone() for t in base] for _ in range(3)]


def apply(case, t, rng):
    """Applies the fixture's fault kind to tensor t in place; returns the
    flipped (index, bit) for bit flips, else None."""
    flat = t.view(-1)
    n = flat.numel()
    if case["kind"] == "bit_flip":
        i = int(rng.integers(0, n))
        W.flip_bit(flat, i, case["bit"])
        return i, case["bit"]
    ints = flat.view(torch.int32 if t.element_size() == 4 else torch.int16)
    i, j = (int(x) for x in rng.choice(n, size=2, replace=False))
    if case["kind"] == "swap":
        while bool(ints[i] == ints[j]):
            j = int(rng.integers(0, n))
        a, b = ints[i].clone(), ints[j].clone()
        ints[i], ints[j] = b, a
    elif case["kind"] == "add_pair":
        ints[i] += case["delta"]
        ints[j] -= case["delta"]
    else:
        raise ValueError(case["kind"])
    return None


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_page_fault_kinds(case):
    dtype = {"f32": torch.float32, "bf16": torch.bfloat16}[case["dtype"]]
    rng = np.random.default_rng(len(case["name"]))
    reps = replicas(dtype, seed=7)
    T = len(reps[0])
    bad_r, bad_k = 2, int(rng.integers(1, T))
    while reps[bad_r][bad_k].numel() < 2:
        bad_k = int(rng.integers(1, T))
    say(f"case fault {case['name']} replica {bad_r} tensor {bad_k}")
    flip = apply(case, reps[bad_r][bad_k], rng)
    tensors = [t for r in reps for t in r]
    plan = sdc.sdc_plan_build(tensors)
    out = sdc.sdc_fingerprint_plan(plan)
    torch.cuda.synchronize()
    assert_rows_equal(sdc.rows_numpy(out), oracle_rows(tensors))
    for mask in (sdc.COL_ALL, sdc.COL_SUM | sdc.COL_WSUM):
        res = sdc.sdc_majority_compare(out, 3, T, col_mask=mask)
        assert res["suspects"] == [bad_r] and res["n_diff"] == 1 and res["first_diff"] == bad_k
    only_sum = sdc.sdc_majority_compare(out, 3, T, col_mask=sdc.COL_SUM)
    assert only_sum["diverged"] == case["plain_sum_changes"]
    only_w = sdc.sdc_majority_compare(out, 3, T, col_mask=sdc.COL_WSUM)
    assert only_w["diverged"] == case["weighted_sum_changes"]
    faulted = out[bad_r * T:(bad_r + 1) * T].contiguous()
    d = sdc.sdc_fingerprint_diff(out[:T].contiguous(), faulted)
    assert d["n_diff"] == 1 and d["indices"] == [bad_k]
    if flip is not None:
        assert d["hints"][0][:2] == flip
    else:
        assert d["hints"][0][1] == -1   # not a single bit flip


def test_worked_example_on_the_gpu():
    # AWS blog post, "Step 1: Detect with three checks in your training loop":
    # one weight on three replicas (fixture tests/golden/worked_example.json)
    g = json.load(open(os.path.join(HERE, "golden", "worked_example.json")))
    R, lr = g["replicas"], g["learning_rate"]

    def dp_step(grads):
        # the all-reduce averages once, in rank order; every replica applies it
        acc = torch.zeros(1, dtype=torch.float32, device=DEV)
        for x in grads:
            acc = acc + torch.tensor([x], dtype=torch.float32, device=DEV)
        avg = acc / R
        return [torch.tensor([w], dtype=torch.float32, device=DEV) - lr * avg
                for w in g["weight_at_start"]]

    def scan(ws):
        plan = sdc.sdc_plan_build(ws)
        out = sdc.sdc_fingerprint_plan(plan)
        torch.cuda.synchronize()
        return out

    w1 = dp_step(g["local_gradient"])
    bits = [int(t.view(torch.int32).item()) & 0xFFFFFFFF for t in w1]
    assert bits == [int(np.array([v], dtype=np.float32).view(np.uint32)[0])
                    for v in g["weight_after_step"]]
    clean = scan(w1)
    assert_rows_equal(sdc.rows_numpy(clean), oracle_rows(w1))
    assert not sdc.sdc_majority_compare(clean, R, 1)["diverged"]
    # a wrong local gradient reaches every replica: the copies still agree
    bad = list(g["local_gradient"])
    bad[g["faulty_local_gradient"]["replica"]] = g["faulty_local_gradient"]["value"]
    w_bad = dp_step(bad)
    t_bad = scan(w_bad)
    assert not sdc.sdc_majority_compare(t_bad, R, 1)["diverged"]
    assert sdc.sdc_fingerprint_diff(clean, t_bad)["n_diff"] == R   # but every copy changed
    # the wrong gradient is finite: the NaN/Inf check passes it
    grads = [torch.tensor([x], dtype=torch.float32, device=DEV) for x in bad]
    _, _, flag = sdc.sdc_sqnorm(sdc.sdc_plan_build(grads))
    assert int(flag.item()) == 0
    # a weight corrupted on one replica after the step: that replica is named
    W.flip_bit(w1[2], 0, 22)
    res = sdc.sdc_majority_compare(scan(w1), R, 1)
    assert res["diverged"] and res["suspects"] == [2]
