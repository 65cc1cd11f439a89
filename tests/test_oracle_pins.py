"""Pins for the oracle (CPU only).

Each test ties the oracle to something other than its own formula: the pages'
worked example and fault table (tests/golden/), closed forms, exact invariants
(single bit flips, swaps, compensating changes, concatenation), big-integer
brute force written differently (W as a sum of suffix sums, no products),
numpy/torch library routines (uint64 wrap-around sums, isfinite over every
16-bit pattern) and brute force over every small majority table.

Pages cited: AWS Machine Learning Blog, "Detecting and recovering from silent
data corruption on Amazon SageMaker HyperPod" -- sections "Compare by
fingerprint", "Step 1: Detect with three checks in your training loop",
"Check 3: Weight fingerprints, after the optimizer step", "Fault scenarios".
"""
import functools
import itertools
import json
import os
from collections import Counter

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle as O

M64 = (1 << 64) - 1
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NP_INT = {O.F32: np.uint32, O.BF16: np.uint16, O.F16: np.uint16}


# ---------------------------------------------------------------------------
# independent references
# ---------------------------------------------------------------------------
def brute_row(raw: bytes, dtype: int):
    """Big-integer brute force from raw little-endian bytes.  W is formed as
    the sum of the n suffix sums (sum_{k} sum_{i>=k} x_i = sum_i (i+1) x_i),
    so it shares no multiply with the oracle.  NF uses library float
    classification, not an exponent mask."""
    es = O.ESIZE[dtype]
    xs = [int.from_bytes(raw[i:i + es], "little", signed=False) for i in range(0, len(raw), es)]
    s = sum(xs) & M64
    suffix, w = 0, 0
    for v in reversed(xs):
        suffix += v
        w += suffix
    x = functools.reduce(lambda a, b: a ^ b, xs, 0)
    nf = int(np.count_nonzero(~library_isfinite(np.frombuffer(raw, dtype=NP_INT[dtype]), dtype)))
    return (s, w & M64, x, nf)


def library_isfinite(bits: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == O.F32:
        return np.isfinite(bits.astype(np.uint32).view(np.float32))
    if dtype == O.F16:
        return np.isfinite(bits.astype(np.uint16).view(np.float16))
    t = torch.from_numpy(bits.astype(np.uint16).view(np.int16).copy()).view(torch.bfloat16)
    return torch.isfinite(t).numpy()


def numpy_row(bits: np.ndarray, dtype: int):
    """numpy uint64 arithmetic wraps modulo 2^64: an independent library form."""
    x = bits.astype(np.uint64)
    n = x.size
    with np.errstate(over="ignore"):
        s = int(x.sum(dtype=np.uint64))
        w = int((np.arange(1, n + 1, dtype=np.uint64) * x).sum(dtype=np.uint64))
    xr = int(np.bitwise_xor.reduce(x)) if n else 0
    nf = int(np.count_nonzero(~library_isfinite(bits, dtype)))
    return (s, w, xr, nf)


EDGE16 = [0x0000, 0xFFFF, 0x8000, 0x7FFF, 0x7F80, 0xFF80, 0x7FC0, 0x7C00, 0xFC00, 0x7E00,
          0x0001, 0x7F81, 0x7C01, 0x3C00, 0x3F80]
EDGE32 = [0x00000000, 0xFFFFFFFF, 0x80000000, 0x7FFFFFFF, 0x7F800000, 0xFF800000, 0x7FC00000,
          0x7F800001, 0xFFC00001, 0x00000001, 0x3F800000, 0x3EF0A3D7]


def rand_bits(rng, n, dtype, edge_frac=0.3):
    hi = 1 << (8 * O.ESIZE[dtype])
    b = rng.integers(0, hi, size=n, dtype=np.uint64)
    edges = EDGE32 if dtype == O.F32 else EDGE16
    m = rng.random(n) < edge_frac
    b[m] = rng.choice(np.array(edges, dtype=np.uint64), size=int(m.sum()))
    return b.astype(NP_INT[dtype])


# ---------------------------------------------------------------------------
# fingerprint definition: brute force, library routine, closed forms
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [O.F32, O.BF16, O.F16])
def test_brute_force_small(dtype):
    rng = np.random.default_rng(100 + dtype)
    for n in range(0, 17):
        for _ in range(40):
            bits = rand_bits(rng, n, dtype)
            assert O.fingerprint(bits, dtype) == brute_row(bits.tobytes(), dtype), (n, bits)


@pytest.mark.parametrize("dtype", [O.F32, O.BF16, O.F16])
def test_numpy_uint64_reference(dtype):
    rng = np.random.default_rng(7 + dtype)
    for n in (1, 1000, 65537, 1_000_003):
        bits = rand_bits(rng, n, dtype, edge_frac=0.01)
        assert O.fingerprint(bits, dtype) == numpy_row(bits, dtype)


def test_wsum_wraps_modulo_2_64():
    # All-ones fp32 patterns at large positions overflow 64 bits quickly.
    n = 300_000
    bits = np.full(n, 0xFFFFFFFF, dtype=np.uint32)
    c = 0xFFFFFFFF
    assert O.fingerprint(bits, O.F32)[:3] == ((n * c) & M64, (c * n * (n + 1) // 2) & M64, c * (n % 2))


@pytest.mark.parametrize("dtype", [O.F32, O.BF16, O.F16])
@pytest.mark.parametrize("c", [0, 1, 0x7FFF, 0x8000, 0xFFFF])
@pytest.mark.parametrize("n", [1, 2, 3, 17, 4096, 100_001])
def test_closed_form_constant(dtype, c, n):
    bits = np.full(n, c, dtype=NP_INT[dtype])
    s, w, x, _ = O.fingerprint(bits, dtype)
    assert s == (n * c) & M64
    assert w == (c * n * (n + 1) // 2) & M64
    assert x == (c if n % 2 else 0)


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
@pytest.mark.parametrize("n", [1, 2, 5, 1000, 65536])
def test_closed_form_ramp(dtype, n):
    # x_i = i: S = n(n-1)/2 and W = sum (i+1) i = (n-1) n (n+1) / 3.
    bits = np.arange(n, dtype=np.uint64).astype(NP_INT[dtype])
    s, w, _, _ = O.fingerprint(bits, dtype)
    assert s == n * (n - 1) // 2
    assert w == (n - 1) * n * (n + 1) // 3


def test_positions_are_one_based_and_ordered():
    # A single nonzero element at index i contributes (i+1)*x to W.
    for i in range(8):
        bits = np.zeros(8, dtype=np.uint16)
        bits[i] = 5
        assert O.fingerprint(bits, O.BF16)[1] == 5 * (i + 1)
    a = np.array([1, 2, 3], dtype=np.uint16)
    assert O.fingerprint(a, O.BF16)[1] == 1 + 4 + 9
    assert O.fingerprint(a[::-1].copy(), O.BF16)[1] == 3 + 4 + 3


def test_zero_extension_not_sign_extension():
    # 0x8000 (bf16 -0.0) and 0x80000000 (fp32 -0.0) count as large unsigned values.
    assert O.fingerprint(np.array([0x8000], dtype=np.uint16), O.BF16)[0] == 0x8000
    assert O.fingerprint(np.array([0x80000000], dtype=np.uint32), O.F32)[0] == 0x80000000
    assert O.fingerprint(np.array([0xFFFF, 0xFFFF], dtype=np.uint16), O.F16)[:3] == (
        0x1FFFE, 0xFFFF * 3, 0)


def test_little_endian_bytes():
    raw = bytes([0x01, 0x02, 0x03, 0x04])
    arr = np.frombuffer(raw, dtype=np.uint8)
    assert O.fingerprint(arr, O.F32)[0] == 0x04030201
    assert O.fingerprint(arr, O.BF16)[:2] == (0x0201 + 0x0403, 0x0201 + 2 * 0x0403)


def test_none_and_empty_rows_are_zero():
    # "Compare by fingerprint": a missing tensor leaves its row at zero.
    assert O.fingerprint(None, O.F32) == (0, 0, 0, 0)
    assert O.fingerprint(np.zeros(0, dtype=np.uint16), O.BF16) == (0, 0, 0, 0)
    rows = O.fingerprint_list([None, np.array([1], dtype=np.uint32), None], [O.F32, O.F32, O.BF16])
    assert [tuple(int(v) for v in r) for r in rows] == [(0, 0, 0, 0), (1, 1, 1, 0), (0, 0, 0, 0)]


def test_same_bits_fp16_bf16_differ_only_in_nonfinite():
    bits = np.array([0x7C00, 0x7F80, 0x3C00, 0x7E00], dtype=np.uint16)
    a, b = O.fingerprint(bits, O.F16), O.fingerprint(bits, O.BF16)
    assert a[:3] == b[:3]
    assert a[3] == np.count_nonzero(~library_isfinite(bits, O.F16)) == 3
    assert b[3] == np.count_nonzero(~library_isfinite(bits, O.BF16)) == 1


def test_bad_dtype_rejected():
    import ctypes
    r = O.Row()
    assert O.lib().oracle_fingerprint(None, 0, 99, ctypes.byref(r)) == -2
    assert O.lib().oracle_element_size(99) == 0


# ---------------------------------------------------------------------------
# nonfinite classification: exhaustive over 16-bit patterns, sampled fp32
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [O.BF16, O.F16])
def test_nonfinite_exhaustive_16bit(dtype):
    bits = np.arange(1 << 16, dtype=np.uint64).astype(np.uint16)
    lib_bad = ~library_isfinite(bits, dtype)
    ours = np.array([O.lib().oracle_is_nonfinite(int(b), dtype) for b in bits], dtype=bool)
    assert np.array_equal(ours, lib_bad)
    counts, total = O.nonfinite_list([bits], [dtype])
    assert int(counts[0]) == total == int(lib_bad.sum())
    assert O.fingerprint(bits, dtype)[3] == int(lib_bad.sum())


def test_nonfinite_fp32_sampled():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    bits[:len(EDGE32)] = EDGE32
    # force many exponent-all-ones patterns with random payloads and signs
    bits[1000:200000] |= np.uint32(0x7F800000)
    expect = int(np.count_nonzero(~np.isfinite(bits.view(np.float32))))
    assert O.fingerprint(bits, O.F32)[3] == expect
    counts, total = O.nonfinite_list([bits, None, bits[:10]], [O.F32, O.F32, O.F32])
    assert total == expect + int(np.count_nonzero(~np.isfinite(bits[:10].view(np.float32))))
    assert int(counts[1]) == 0


# ---------------------------------------------------------------------------
# exact invariants of the definition
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [O.F32, O.BF16, O.F16])
def test_single_bit_flip_deltas(dtype):
    rng = np.random.default_rng(11 + dtype)
    nbits = 8 * O.ESIZE[dtype]
    for _ in range(200):
        n = int(rng.integers(1, 5000))
        bits = rand_bits(rng, n, dtype)
        i, b = int(rng.integers(0, n)), int(rng.integers(0, nbits))
        s0, w0, x0, _ = O.fingerprint(bits, dtype)
        was_set = (int(bits[i]) >> b) & 1
        bits[i] ^= NP_INT[dtype](1 << b)
        s1, w1, x1, _ = O.fingerprint(bits, dtype)
        sign = -1 if was_set else 1
        assert (s1 - s0) & M64 == (sign * (1 << b)) & M64
        assert (w1 - w0) & M64 == (sign * (i + 1) * (1 << b)) & M64
        assert x0 ^ x1 == 1 << b
        # the flip hint inverts these deltas exactly
        h = O.flip_hint((s0, w0, x0, 0), (s1, w1, x1, 0))
        assert h == (i, b, 1 if not was_set else -1)


def test_swap_changes_only_wsum():
    # "Fault scenarios": a swap of two values leaves the plain sum unchanged.
    rng = np.random.default_rng(5)
    for _ in range(200):
        n = int(rng.integers(2, 3000))
        bits = rand_bits(rng, n, O.F32)
        i, j = sorted(rng.choice(n, size=2, replace=False).tolist())
        if bits[i] == bits[j]:
            continue
        s0, w0, x0, nf0 = O.fingerprint(bits, O.F32)
        xi, xj = int(bits[i]), int(bits[j])
        bits[i], bits[j] = bits[j], bits[i]
        s1, w1, x1, nf1 = O.fingerprint(bits, O.F32)
        assert (s1, x1, nf1) == (s0, x0, nf0)
        assert (w1 - w0) & M64 == ((j - i) * (xi - xj)) & M64 != 0


def test_compensating_pair_changes_only_wsum():
    # "Fault scenarios": +4096 and -4096 on two bit patterns; S unchanged.
    rng = np.random.default_rng(6)
    for _ in range(200):
        n = int(rng.integers(2, 3000))
        bits = rng.integers(4096, (1 << 32) - 4096, size=n, dtype=np.uint64).astype(np.uint32)
        i, j = rng.choice(n, size=2, replace=False).tolist()
        s0, w0, _, _ = O.fingerprint(bits, O.F32)
        bits[i] += np.uint32(4096)
        bits[j] -= np.uint32(4096)
        s1, w1, _, _ = O.fingerprint(bits, O.F32)
        assert s1 == s0
        assert (w1 - w0) & M64 == (4096 * (i - j)) & M64 != 0


def test_fault_kinds_from_pages():
    cases = json.load(open(os.path.join(GOLDEN, "fault_kinds.json")))["cases"]
    rng = np.random.default_rng(8)
    for c in cases:
        dt = {"f32": O.F32, "bf16": O.BF16}[c["dtype"]]
        vals = rng.normal(0, 0.02, size=4096).astype(np.float32)
        bits = vals.view(np.uint32).copy() if dt == O.F32 else (vals.view(np.uint32) >> 16).astype(np.uint16)
        before = O.fingerprint(bits, dt)
        i, j = 100, 2900
        if c["kind"] == "bit_flip":
            bits[i] ^= NP_INT[dt](1 << c["bit"])
        elif c["kind"] == "swap":
            bits[i], bits[j] = bits[j], bits[i]
        elif c["kind"] == "add_pair":
            bits[i] += NP_INT[dt](c["delta"])
            bits[j] -= NP_INT[dt](c["delta"])
        after = O.fingerprint(bits, dt)
        assert (before[0] != after[0]) == c["plain_sum_changes"], c["name"]
        assert (before[1] != after[1]) == c["weighted_sum_changes"], c["name"]


@settings(max_examples=300, deadline=None)
@given(st.data())
def test_one_or_two_element_changes_always_detected(data):
    # "Compare by fingerprint": any change to one or two elements of a tensor
    # with fewer than 2^32 elements of at most 4 bytes changes (S, W).
    dtype = data.draw(st.sampled_from([O.F32, O.BF16, O.F16]))
    hi = (1 << (8 * O.ESIZE[dtype])) - 1
    n = data.draw(st.integers(1, 64))
    xs = data.draw(st.lists(st.integers(0, hi), min_size=n, max_size=n))
    bits = np.array(xs, dtype=NP_INT[dtype])
    k = data.draw(st.integers(1, min(2, n)))
    idx = data.draw(st.lists(st.integers(0, n - 1), min_size=k, max_size=k, unique=True))
    new = bits.copy()
    for i in idx:
        new[i] = data.draw(st.integers(0, hi).filter(lambda v, i=i: v != int(bits[i])))
    a, b = O.fingerprint(bits, dtype), O.fingerprint(new, dtype)
    assert a[:2] != b[:2]


def test_three_element_collision_is_not_detected_by_s_and_w():
    # Equal fingerprints are evidence, not proof: +1, -2, +1 at i, i+1, i+2
    # leaves S and W unchanged.
    rng = np.random.default_rng(9)
    bits = rng.integers(10, 1000, size=64, dtype=np.uint64).astype(np.uint32)
    a = O.fingerprint(bits, O.F32)
    bits[20] += np.uint32(1)
    bits[21] -= np.uint32(2)
    bits[22] += np.uint32(1)
    b = O.fingerprint(bits, O.F32)
    assert a[:2] == b[:2]


def test_concatenation_identity():
    # W(A||B) = W(A) + W(B) + |A| S(B); S, X, NF combine by +, ^, +.
    rng = np.random.default_rng(10)
    for dtype in (O.F32, O.BF16, O.F16):
        for _ in range(50):
            n = int(rng.integers(0, 20000))
            bits = rand_bits(rng, n, dtype, edge_frac=0.05)
            cut = int(rng.integers(0, n + 1))
            A, B = bits[:cut], bits[cut:]
            ra, rb, rab = O.fingerprint(A, dtype), O.fingerprint(B, dtype), O.fingerprint(bits, dtype)
            assert rab[0] == (ra[0] + rb[0]) & M64
            assert rab[1] == (ra[1] + rb[1] + cut * rb[0]) & M64
            assert rab[2] == ra[2] ^ rb[2]
            assert rab[3] == ra[3] + rb[3]


def test_chunking_does_not_change_the_result():
    # The pages' chunked loop offsets positions per chunk; any chunk size gives
    # the same row.  Chunks are merged here with the identity above.
    rng = np.random.default_rng(12)
    bits = rand_bits(rng, 100_000, O.BF16, edge_frac=0.01)
    whole = O.fingerprint(bits, O.BF16)
    for chunk in (1, 7, 4096, 1 << 14, 99_999, 1 << 20):
        s = w = x = nf = 0
        for start in range(0, bits.size, chunk):
            r = O.fingerprint(bits[start:start + chunk], O.BF16)
            s, w, x, nf = (s + r[0]) & M64, (w + r[1] + start * r[0]) & M64, x ^ r[2], nf + r[3]
        assert (s, w, x, nf) == whole


# ---------------------------------------------------------------------------
# strict-majority compare
# ---------------------------------------------------------------------------
def naive_majority(copies_per_tensor, R):
    """The rule of "Check 3", written with collections.Counter: for every
    tensor whose copies are not all equal, a replica is named only if some
    value is held by more than half of the copies and the replica's differs."""
    diverged, no_major, suspects, status = False, [], set(), []
    for k, copies in enumerate(copies_per_tensor):
        if len(set(copies)) == 1:
            status.append(0)
            continue
        diverged = True
        value, count = Counter(copies).most_common(1)[0]
        if 2 * count <= R:
            no_major.append(k)
            status.append(2)
            continue
        status.append(1)
        suspects |= {r for r, c in enumerate(copies) if c != value}
    return diverged, no_major, suspects, status


def table_from_values(vals, R, T, palette):
    t = np.zeros((R * T, 4), dtype=np.uint64)
    for r in range(R):
        for k in range(T):
            t[r * T + k] = palette[vals[r * T + k]]
    return t


def test_majority_brute_force_all_small_tables():
    palette = {0: (1, 2, 3, 0), 1: (1, 2, 4, 0), 2: (9, 2, 3, 1)}
    for R in range(1, 6):
        for T in (1, 2):
            for vals in itertools.product(range(3), repeat=R * T):
                table = table_from_values(vals, R, T, palette)
                res = O.majority_compare(table, R, T)
                copies = [[vals[r * T + k] for r in range(R)] for k in range(T)]
                diverged, no_major, suspects, status = naive_majority(copies, R)
                diffs = [k for k in range(T) if status[k] != 0]
                assert res["diverged"] == diverged
                assert res["has_majority"] == (not no_major)
                assert res["n_diff"] == len(diffs)
                assert res["first_diff"] == (diffs[0] if diffs else O.U64MAX)
                assert res["first_no_majority"] == (no_major[0] if no_major else O.U64MAX)
                assert list(res["tensor_status"]) == status
                if no_major:
                    assert res["suspects"] is None and not res["suspect_flags"].any()
                else:
                    assert res["suspects"] == sorted(suspects)


def test_majority_special_cases_from_pages():
    # With two copies a disagreement names no one; one copy never diverges.
    a, b = (1, 1, 1, 0), (2, 1, 1, 0)
    r2 = O.majority_compare(np.array([a, b], dtype=np.uint64), 2, 1)
    assert r2["diverged"] and r2["suspects"] is None
    r1 = O.majority_compare(np.array([a], dtype=np.uint64), 1, 1)
    assert not r1["diverged"] and r1["suspects"] == []
    # 2-2 split among four copies: no strict majority.
    r4 = O.majority_compare(np.array([a, a, b, b], dtype=np.uint64), 4, 1)
    assert r4["diverged"] and not r4["has_majority"]
    # 3 of 5 agree: the other two are named.
    c = (3, 3, 3, 0)
    r5 = O.majority_compare(np.array([a, b, a, c, a], dtype=np.uint64), 5, 1)
    assert r5["suspects"] == [1, 3]


def test_majority_column_mask():
    a, b = (1, 2, 3, 0), (1, 2, 7, 0)   # differ only in the xorsum column
    t = np.array([a, a, b], dtype=np.uint64)
    assert O.majority_compare(t, 3, 1, O.COL_ALL)["suspects"] == [2]
    assert not O.majority_compare(t, 3, 1, O.COL_SUM | O.COL_WSUM)["diverged"]


def test_majority_rejects_bad_arguments():
    t = np.zeros((3, 4), dtype=np.uint64)
    with pytest.raises(ValueError):
        O.majority_compare(t, 3, 1, 0)
    with pytest.raises(ValueError):
        O.majority_compare(t, 3, 1, 16)


def test_worked_example_from_pages():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    f32 = np.float32
    R, lr = g["replicas"], f32(g["learning_rate"])

    def dp_step(w0, grads):
        # the all-reduce averages once, in rank order, and every replica
        # applies the same average
        acc = f32(0)
        for x in grads:
            acc = f32(acc + f32(x))
        avg = f32(acc / f32(R))
        return avg, [f32(f32(w) - f32(lr * avg)) for w in w0]

    avg, w1 = dp_step(g["weight_at_start"], g["local_gradient"])
    assert avg == f32(g["averaged_gradient"])
    assert [float(w) for w in w1] == [float(f32(v)) for v in g["weight_after_step"]]
    assert np.array(w1, dtype=np.float32).view(np.uint32).tolist() == [0x3EF0A3D7] * 3

    def table(ws):
        return np.array([O.fingerprint(np.array([w], dtype=np.float32).view(np.uint32), O.F32)
                         for w in ws], dtype=np.uint64)

    assert not O.majority_compare(table(w1), R, 1)["diverged"]

    # a wrong local gradient spreads identically: the weights still match
    bad = list(g["local_gradient"])
    bad[g["faulty_local_gradient"]["replica"]] = g["faulty_local_gradient"]["value"]
    _, w_bad = dp_step(g["weight_at_start"], bad)
    assert len({float(w) for w in w_bad}) == 1 and float(w_bad[0]) != float(w1[0])
    assert not O.majority_compare(table(w_bad), R, 1)["diverged"]

    # a weight corrupted on replica 1 after the step is named
    w_flip = np.array(w1, dtype=np.float32).view(np.uint32).copy()
    w_flip[1] ^= np.uint32(1 << 22)
    res = O.majority_compare(table(w_flip.view(np.float32)), R, 1)
    assert res["diverged"] and res["suspects"] == [1]


# ---------------------------------------------------------------------------
# diff of two tables and the flip hint
# ---------------------------------------------------------------------------
def test_diff_finds_injected_flips_in_order():
    rng = np.random.default_rng(13)
    T = 300
    arrays = [rand_bits(rng, int(rng.integers(1, 3000)), O.BF16) for _ in range(T)]
    a = O.fingerprint_list(arrays, [O.BF16] * T)
    hit = sorted(rng.choice(T, size=17, replace=False).tolist())
    expect = {}
    for k in hit:
        i = int(rng.integers(0, arrays[k].size))
        b = int(rng.integers(0, 16))
        was = (int(arrays[k][i]) >> b) & 1
        arrays[k][i] ^= np.uint16(1 << b)
        expect[k] = (i, b, -1 if was else 1)
    bt = O.fingerprint_list(arrays, [O.BF16] * T)
    d = O.fingerprint_diff(a, bt)
    assert d["n_diff"] == len(hit) and d["indices"] == hit
    assert d["hints"] == [expect[k] for k in hit]
    d5 = O.fingerprint_diff(a, bt, cap=5)
    assert d5["n_diff"] == len(hit) and d5["indices"] == hit[:5]
    assert O.fingerprint_diff(a, a)["n_diff"] == 0


def test_flip_hint_rejects_other_changes():
    a = (100, 1000, 7, 0)
    assert O.flip_hint(a, a) == (O.U64MAX, -1, 0)
    assert O.flip_hint(a, (100, 1000, 7 ^ 3, 0)) == (O.U64MAX, -1, 0)       # two bits
    assert O.flip_hint(a, (100 + 4, 1000 + 12, 7 ^ 4, 0)) == (2, 2, 1)       # i=2, b=2
    assert O.flip_hint(a, (100 + 4, 1000 + 13, 7 ^ 4, 0)) == (O.U64MAX, -1, 0)
    assert O.flip_hint(a, (100 - 4, 1000 - 12, 7 ^ 4, 0)) == (2, 2, -1)
    assert O.flip_hint(a, (100 + 4, 1000 - 12, 7 ^ 4, 0)) == (O.U64MAX, -1, 0)  # sign mismatch


def test_diff_column_mask_and_empty():
    a = np.array([[1, 2, 3, 0]], dtype=np.uint64)
    b = np.array([[1, 2, 3, 1]], dtype=np.uint64)
    assert O.fingerprint_diff(a, b)["n_diff"] == 1
    assert O.fingerprint_diff(a, b, O.COL_SUM | O.COL_WSUM | O.COL_XOR)["n_diff"] == 0
    e = np.zeros((0, 4), dtype=np.uint64)
    assert O.fingerprint_diff(e, e)["n_diff"] == 0
