"""Ring replay audit table logic ("Check 2: Ring replay, before the optimizer
step" and "Fault scenarios" of the AWS blog post).

CPU: the oracle reproduces the pages' printed pairs, culprits and confirmation
verdicts (tests/golden/ring_scenarios.json) from a model of each injected
fault, its localisation matches a Counter-based brute force, and the
library's host-only localisation equals the oracle's.  GPU: the compare and
confirmation kernels equal the oracle on random tables and on the scenarios.
"""
import itertools
import json
import os
from collections import Counter

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FIX = json.load(open(os.path.join(GOLDEN, "ring_scenarios.json")))
WIDTH = 9  # loss bits + two fingerprint rows


def true_result(batch):
    rng = np.random.default_rng(1000 + batch)
    return rng.integers(0, 1 << 63, size=WIDTH, dtype=np.uint64)


def wrong_result(batch, rank):
    r = true_result(batch).copy()
    r[1 + rank % (WIDTH - 1)] ^= np.uint64(1 << (rank % 60))  # e.g. one gradient bit
    return r


def scenario_table(sc, n, offset):
    kinds = {f["rank"]: f["kind"] for f in sc["faults"]}
    table = np.zeros((n, 2, WIDTH), dtype=np.uint64)
    for r in range(n):
        k = kinds.get(r)
        table[r, 0] = wrong_result(r, r) if k in ("persistent", "transient_own") else true_result(r)
        t = (r + offset) % n
        table[r, 1] = wrong_result(t, r) if k in ("persistent", "transient_replay") else true_result(t)
    return table, kinds


def confirmation_inputs(pair, table, kinds, n, offset):
    target, replayer = pair
    third = (target + offset) % n
    third_r = wrong_result(target, third) if kinds.get(third) == "persistent" else true_result(target)
    # a persistent fault reproduces its own wrong answer; a transient one does not recur
    self_r = table[target, 0] if kinds.get(target) == "persistent" else true_result(target)
    return third, third_r, self_r, table[target, 0], table[replayer, 1]


@pytest.mark.parametrize("sc", FIX["scenarios"], ids=[s["name"][:40] for s in FIX["scenarios"]])
def test_oracle_reproduces_the_pages_scenarios(sc):
    n, off = FIX["n"], FIX["offset"]
    table, kinds = scenario_table(sc, n, off)
    mism = O.ring_pairs(table, n, off)
    pairs = sorted([[(r + off) % n, r] for r in range(n) if mism[r]])
    assert pairs == sorted(sc["pairs"])
    cul, amb = O.ring_localize(mism, n, off)
    assert [q for q in range(n) if cul[q]] == sc["culprits"]
    ambiguous = sorted([[(r + off) % n, r] for r in range(n) if amb[r]])
    assert ambiguous == sorted(v["pair"] for v in sc["verdicts"])
    for v in sc["verdicts"]:
        third, third_r, self_r, orig, peer = confirmation_inputs(v["pair"], table, kinds, n, off)
        assert third == v["third"]
        kind = O.VERDICTS[O.confirm_verdict(third_r, self_r, orig, peer)]
        assert kind == v["kind"]
        suspect = v["pair"][1] if kind == "replayer computed wrong" else v["pair"][0]
        assert suspect == v["suspect"]


def test_three_instances_same_alarms_only_peers_change():
    # "On 3 instances, every scenario raised the same alarm ... naming the same
    # ranks.  Only the peer ranks changed." (24 ranks, offset 8)
    n, off = 24, 8
    for sc in FIX["scenarios"]:
        table, kinds = scenario_table(sc, n, off)
        mism = O.ring_pairs(table, n, off)
        cul, amb = O.ring_localize(mism, n, off)
        assert [q for q in range(n) if cul[q]] == sc["culprits"]
        faulty = {f["rank"] for f in sc["faults"]}
        for r in range(n):
            if mism[r]:
                assert {(r + off) % n, r} & faulty


def counter_localize(pairs):
    hits = Counter(x for p in pairs for x in p)
    culprits = sorted(x for x, c in hits.items() if c >= 2)
    ambiguous = [p for p in pairs if not set(p) & set(culprits)]
    return culprits, ambiguous


def test_localize_brute_force():
    rng = np.random.default_rng(4)
    for n in range(1, 11):
        for off in range(0, n + 2):
            for _ in range(30):
                mism = (rng.random(n) < 0.3).astype(np.uint8)
                pairs = [((r + off) % n, r) for r in range(n) if mism[r]]
                culprits, ambiguous = counter_localize(pairs)
                cul, amb = O.ring_localize(mism, n, off)
                assert [q for q in range(n) if cul[q]] == culprits
                assert [((r + off) % n, r) for r in range(n) if amb[r]] == ambiguous


def test_verdict_table_exhaustive():
    # Each verdict row of "Decide what the alarm means" as a statement about
    # the four results, checked over every assignment of three values.
    vals = [np.full(3, v, dtype=np.uint64) for v in (1, 2, 3)]
    for witness, retry, original, replay in itertools.product(range(3), repeat=4):
        got = O.VERDICTS[O.confirm_verdict(vals[witness], vals[retry], vals[original], vals[replay])]
        sided_with_replayer = witness == replay and witness != original
        if witness == original:  # "the replaying GPU, not the target, was wrong"
            want = "replayer computed wrong"
        elif sided_with_replayer and retry == original:  # "reproduced its own wrong answer"
            want = "persistent"
        elif sided_with_replayer and retry == witness:  # "retry came out right and agreed"
            want = "transient"
        elif sided_with_replayer:  # the three do not line up
            want = "unclear"
        else:
            want = "unattributable"
        assert got == want, (witness, retry, original, replay)


def test_library_localize_matches_oracle_host_only():
    import silent_corruption_detection_amd as sdc
    rng = np.random.default_rng(5)
    for n in (1, 2, 3, 8, 32, 100):
        for off in (0, 1, 8, n - 1 if n > 1 else 0, 3 * n + 2):
            mism = (rng.random(n) < 0.2).astype(np.uint8)
            a = sdc.sdc_ring_localize(mism, n, off)
            b = O.ring_localize(mism, n, off)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------------------
# GPU
# ---------------------------------------------------------------------------
@pytest.mark.gpu
def test_gpu_ring_compare_matches_oracle():
    import torch
    import silent_corruption_detection_amd as sdc
    rng = np.random.default_rng(6)
    for n in (1, 2, 5, 32, 64):
        for width in (1, 7, 300, 5000):
            for off in (0, 1, 8, n + 3):
                table = rng.integers(0, 1 << 63, size=(n, 2, width), dtype=np.uint64)
                for r in range(n):  # make most pairs agree
                    if rng.random() < 0.8:
                        table[r, 1] = table[(r + off) % n, 0]
                        if rng.random() < 0.3:
                            table[r, 1, int(rng.integers(0, width))] ^= np.uint64(1)
                d = torch.from_numpy(table.view(np.int64).copy()).cuda()
                got = sdc.sdc_ring_compare(d, n, off)
                assert np.array_equal(got, O.ring_pairs(table, n, off)), (n, width, off)


@pytest.mark.gpu
def test_gpu_scenarios_and_verdicts():
    import torch
    import silent_corruption_detection_amd as sdc
    n, off = FIX["n"], FIX["offset"]
    for sc in FIX["scenarios"]:
        table, kinds = scenario_table(sc, n, off)
        d = torch.from_numpy(table.view(np.int64).copy()).cuda()
        mism = sdc.sdc_ring_compare(d, n, off)
        assert sorted([[(r + off) % n, r] for r in range(n) if mism[r]]) == sorted(sc["pairs"])
        for v in sc["verdicts"]:
            _, third_r, self_r, orig, peer = confirmation_inputs(v["pair"], table, kinds, n, off)
            dv = [torch.from_numpy(np.ascontiguousarray(x).view(np.int64).copy()).cuda()
                  for x in (third_r, self_r, orig, peer)]
            assert sdc.VERDICTS[sdc.sdc_confirm_verdict(*dv)] == v["kind"]
    vals = [torch.full((4000,), v, dtype=torch.int64, device="cuda") for v in (1, 2, 3)]
    hv = [np.full(4000, v, dtype=np.uint64) for v in (1, 2, 3)]
    for combo in itertools.product(range(3), repeat=4):
        assert sdc.sdc_confirm_verdict(*[vals[i] for i in combo]) == \
            O.confirm_verdict(*[hv[i] for i in combo])
