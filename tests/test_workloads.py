"""The seeded generators (CPU, small sizes): shapes and parameter counts of the
full workloads, the small-tensor layout, determinism, and that every recorded
corruption is exactly one bit.  The oracle then confirms, on CPU, that the
recorded corruption is what the majority rule and the diff report."""
import numpy as np
import torch

import oracle as O
import workloads as W
from _util import oracle_rows


def test_gpt_shapes_match_the_stated_size():
    shapes = W.gpt_shapes()
    assert len(shapes) == 207
    assert sum(int(np.prod(s)) for _, s, _ in shapes) == 959_117_312


def test_llama70b_shapes_match_the_stated_size():
    shapes = W.llama70b_shapes()
    assert len(shapes) == 723
    n = sum(int(np.prod(s)) for _, s in shapes)
    assert n == 70_553_706_496 and 2 * n == 141_107_412_992


def test_c4_layout_properties():
    _, numel, dtypes, offs, nbytes = W.c4_layout(4)
    assert numel.size == 100_000 and numel.min() >= 1 and numel.max() <= 65536
    assert set(np.unique(dtypes).tolist()) == {0, 1, 2}
    es = np.array([W.ESIZE[int(d)] for d in dtypes])
    assert np.all(offs % es == 0)
    assert np.all(offs[1:] >= offs[:-1] + numel[:-1] * es[:-1])
    # log-uniform sizes: median near sqrt(65537) ~ 256
    assert 150 < np.median(numel) < 450
    assert 4.0e9 < 3 * nbytes < 5.5e9
    misaligned = np.count_nonzero(offs % 16)
    assert misaligned > 50_000  # most starts are not 16-byte aligned


def test_generators_are_deterministic_and_flip_one_bit():
    a = W.c1("cpu", numel=10_000)
    b = W.c1("cpu", numel=10_000)
    assert all(torch.equal(x, y) for x, y in zip(a.tensors, b.tensors))
    inj = a.injections[0]
    d = (a.tensors[0].view(torch.int32) ^ a.tensors[inj["replica"]].view(torch.int32))
    nz = torch.nonzero(d).flatten().tolist()
    assert nz == [inj["index"]]
    assert int(d[inj["index"]].item()) & 0xFFFFFFFF == 1 << inj["bit"]


def test_c1_small_oracle_names_replica_1():
    w = W.c1("cpu", numel=50_000)
    rows = oracle_rows(w.tensors)
    res = O.majority_compare(rows, w.R, w.T)
    assert res["suspects"] == [1]


def test_c2_small_shapes():
    shapes = W.gpt_shapes(d=32, layers=2, vocab=100)
    w = W.c2("cpu", shapes=shapes)
    rows = oracle_rows(w.tensors)
    res = O.majority_compare(rows, w.R, w.T)
    assert res["suspects"] == [w.injections[0]["replica"]]
    assert res["first_diff"] == w.injections[0]["tensor"] and res["n_diff"] == 1


def test_c3_small_shapes_nonfinite_and_replay():
    shapes = W.gpt_shapes(d=64, layers=2, vocab=512)
    w = W.c3("cpu", shapes=shapes, rate=1e-3)
    assert w.meta["n_nonfinite"] == len(w.nonfinite) > 0
    rows = oracle_rows(w.tensors)
    assert int(rows[:w.T, 3].sum()) == len(w.nonfinite)
    d = O.fingerprint_diff(rows[:w.T], rows[w.T:])
    inj = w.injections[0]
    assert d["indices"] == [inj["tensor"]]
    assert d["hints"] == [(inj["index"], inj["bit"], -1 if inj["was"] else 1)]


def test_c4_small():
    w = W.c4("cpu", n_tensors=500, max_numel=4096)
    rows = oracle_rows(w.tensors)
    res = O.majority_compare(rows, w.R, w.T)
    assert res["suspects"] == sorted({i["replica"] for i in w.injections})
    assert res["n_diff"] == 5
