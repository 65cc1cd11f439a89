"""GPU parity on the five full-size workloads, in the launch configuration the
benchmark times (automatic item size).

Expected outcomes come from the generators' own records of what they wrote
(which replica / tensor / element / bit was flipped, where NaN/Inf went) and
from the oracle, never from the HIP path:
  c1, c2  every row equals the oracle's; the majority compare names exactly
          the corrupted replica.
  c3      rows, NaN/Inf counts and squared norms equal the oracle's (norms
          within the summation bound); the norm check flags the list and
          clears it without the tensors that hold NaN/Inf; the replay differs
          from the original in exactly the flipped tensor, and the flip hint
          gives the flipped element and bit.
  c4      rows equal the oracle's for all 300,000 tensors; the named replicas
          are those the corruptions went to.
  c5      (141 GB) all 723 rows equal the oracle's (the oracle's table is
          the stored table: a second scan diffed against it is empty); the
          NaN/Inf counts equal the oracle's (all zero) and the norm check is
          clear; squared norms of a sample of tensors equal the oracle's
          (within the summation bound); one seeded flip gives exactly one
          differing tensor with the exact localisation.
"""
import gc

import numpy as np
import pytest
import torch

import oracle as O
import silent_corruption_detection_amd as sdc
import workloads as W
from _util import (THREADS, assert_rows_equal, assert_sq_close, oracle_nonfinite, oracle_rows,
                   oracle_sqnorms, say)
from oracle.device_lists import rows_of_device_tensors
from silent_corruption_detection_amd.table import load_table, save_table

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def free_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def scan(w):
    plan = sdc.sdc_plan_build(w.tensors)
    out = sdc.sdc_fingerprint_plan(plan)
    torch.cuda.synchronize()
    return plan, out


def expected_suspects(w):
    return sorted({inj["replica"] for inj in w.injections})


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_replicas_with_one_flip(name):
    say(f"case {name}: generate")
    w = W.BUILDERS[name](DEV)
    plan, out = scan(w)
    say(f"case {name}: oracle over {w.R * w.T} tensors")
    assert_rows_equal(sdc.rows_numpy(out), oracle_rows(w.tensors), w.names * w.R)
    status = torch.zeros(w.T, dtype=torch.uint8, device=DEV)
    res = sdc.sdc_majority_compare(out, w.R, w.T, tensor_status=status)
    inj = w.injections[0]
    assert res["diverged"] and res["has_majority"]
    assert res["suspects"] == [inj["replica"]]
    assert res["n_diff"] == 1 and res["first_diff"] == inj["tensor"]
    st = status.cpu().numpy()
    assert st[inj["tensor"]] == 1 and int(st.sum()) == 1
    assert int(sdc.rows_numpy(out)[:, 3].sum()) == 0  # N(0, 0.02) data: no NaN/Inf
    # the same comparison restricted to the pages' two sums
    assert sdc.sdc_majority_compare(out, w.R, w.T, col_mask=sdc.COL_SUM | sdc.COL_WSUM)[
        "suspects"] == [inj["replica"]]


def test_c3_gradients_nonfinite_and_replay():
    say("case c3: generate")
    w = W.c3(DEV)
    plan, out = scan(w)
    rows = sdc.rows_numpy(out)
    say("case c3: oracle")
    assert_rows_equal(rows, oracle_rows(w.tensors), w.names * 2)
    counts, total = sdc.sdc_nonfinite(plan)
    torch.cuda.synchronize()
    ref_nf = oracle_nonfinite(w.tensors)
    assert counts.cpu().numpy().astype(np.uint64).tolist() == ref_nf.tolist()
    assert int(total.item()) == int(ref_nf.sum())
    # every written NaN/Inf is counted in the original
    assert int(ref_nf[:w.T].sum()) == w.meta["n_nonfinite"] == len(w.nonfinite)
    say("case c3: squared norms")
    sq, sq_total, flag = sdc.sdc_sqnorm(plan)
    torch.cuda.synchronize()
    ref_sq = oracle_sqnorms(w.tensors)
    assert_sq_close(sq.cpu().tolist(), ref_sq, [t.numel() for t in w.tensors])
    assert int(flag.item()) == int(len(w.nonfinite) > 0) == 1
    # the same gradients without their NaN/Inf: a finite norm, flag clear
    clean_idx = sorted({tk for tk, _, _ in w.nonfinite} ^ set(range(w.T)))
    clean = sdc.sdc_plan_build([w.tensors[k] for k in clean_idx])
    sq_c, tot_c, flag_c = sdc.sdc_sqnorm(clean)
    torch.cuda.synchronize()
    assert int(flag_c.item()) == 0
    ref_c = sum(ref_sq[k] for k in clean_idx)
    n_c = sum(w.tensors[k].numel() for k in clean_idx) + len(clean_idx)
    assert abs(float(tot_c.item()) - ref_c) <= (2 * n_c + 2) * 2.0 ** -53 * ref_c
    inj = w.injections[0]
    T = w.T
    d = sdc.sdc_fingerprint_diff(out[:T].contiguous(), out[T:].contiguous())
    assert d["n_diff"] == 1 and d["indices"] == [inj["tensor"]]
    assert d["hints"] == [(inj["index"], inj["bit"], -1 if inj["was"] else 1)]


def test_c4_small_mixed_tensors():
    say("case c4: generate")
    w = W.c4(DEV)
    plan, out = scan(w)
    rows = sdc.rows_numpy(out)
    say(f"case c4: oracle over {w.R * w.T} tensors")
    # host copies of the three flat buffers, then per-tensor views by offset
    _, numel, dtypes, offs, _ = W.c4_layout(w.seed)
    ref = np.zeros((w.R * w.T, 4), dtype=np.uint64)
    for r, flat in enumerate(w.buffers):
        h = flat.cpu().numpy()
        for k in range(w.T):
            es = W.ESIZE[int(dtypes[k])]
            o = int(offs[k])
            ref[r * w.T + k] = O.fingerprint(h[o:o + int(numel[k]) * es], int(dtypes[k]))
    assert_rows_equal(rows, ref)
    res = sdc.sdc_majority_compare(out, w.R, w.T)
    assert res["has_majority"] and res["suspects"] == expected_suspects(w)
    assert res["n_diff"] == len(w.injections)
    assert res["first_diff"] == min(i["tensor"] for i in w.injections)


def test_c5_llama70b_bf16(tmp_path):
    say("case c5: generate 141 GB")
    w = W.c5(DEV)
    assert w.elems_per_replica == 70_553_706_496
    plan, out = scan(w)
    first = out.clone()
    # every one of the 723 rows against the oracle (streamed to the host
    # through pinned buffers, 16 oracle calls at a time): the table stored
    # after a checkpoint, computed by the oracle
    say("case c5: oracle over all 723 tensors")
    ref, st = rows_of_device_tensors(w.tensors, threads=THREADS)
    say(f"case c5: oracle done: {st['bytes'] / 1e9:.1f} GB in {st['wall_s']:.1f} s "
        f"(copies {st['d2h_s']:.1f} s)")
    assert st["bytes"] == plan.total_bytes
    assert_rows_equal(sdc.rows_numpy(out), ref, w.names)
    # saved beside the checkpoint, loaded back after the restore (checked
    # against the live list's types and sizes)
    save_table(str(tmp_path / "c5"), torch.from_numpy(ref.view(np.int64)), w.tensors, names=w.names)
    stored, _ = load_table(str(tmp_path / "c5"), tensors=w.tensors, device=DEV)
    assert np.array_equal(sdc.rows_numpy(stored), ref)
    # the NaN/Inf-count and squared-norm scans on the same list (wide launch shape)
    say("case c5: NaN/Inf counts and squared norms")
    counts, total = sdc.sdc_nonfinite(plan)
    sq, sq_total, flag = sdc.sdc_sqnorm(plan)
    torch.cuda.synchronize()
    assert counts.cpu().numpy().astype(np.uint64).tolist() == ref[:, 3].tolist()
    assert int(total.item()) == 0 == int(ref[:, 3].sum())
    assert int(flag.item()) == 0
    sample = [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 365, 366, 367, 368, 369, 370, 371, 721, 722]
    picked = [w.tensors[k] for k in sample]
    assert_sq_close(sq.cpu().numpy()[sample].tolist(), oracle_sqnorms(picked),
                    [t.numel() for t in picked])
    # the check after a restore: a second scan diffed against the oracle's table
    sdc.sdc_fingerprint_plan(plan, out)
    d = sdc.sdc_fingerprint_diff(stored, out)
    assert d["n_diff"] == 0
    assert torch.equal(out, first)
    inj = W.c5_flip(w)
    say(f"case c5: flip {inj}")
    sdc.sdc_fingerprint_plan(plan, out)
    d = sdc.sdc_fingerprint_diff(stored, out)
    assert d["n_diff"] == 1 and d["indices"] == [inj["tensor"]]
    assert d["hints"] == [(inj["index"], inj["bit"], -1 if inj["was"] else 1)]
    k = inj["tensor"]
    assert_rows_equal(sdc.rows_numpy(out)[[k]], oracle_rows([w.tensors[k]]), [w.names[k]])
    del w, plan, out, first, stored
