"""GPU parity: the HIP path against the oracle, bit for bit, through the C ABI.

Cases: sizes that span several work items and leave ragged heads and tails,
misaligned starts (tensors carved from a byte buffer at every element-aligned
offset), item sizes from 16 bytes to 4 MiB (the rows must not depend on how a
tensor is split), random bit patterns with many NaN/Inf values and every 16-bit pattern
(the exact count of flagged rounds), large finite bf16 values that trip the packed fp16 pre-check,
None and empty tensors, and the majority / diff kernels on random tables.
"""
import numpy as np
import pytest
import torch

import oracle as O
import silent_corruption_detection_amd as sdc
from _util import assert_rows_equal, oracle_nonfinite, oracle_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
ES = {torch.float32: 4, torch.bfloat16: 2, torch.float16: 2}
SIZES = [1, 2, 3, 5, 7, 8, 9, 15, 16, 17, 31, 33, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025,
         4095, 4096, 4097, 8191, 8193, 65535, 65537, 262143, 262145, 1_000_003]


def gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def random_bits(nbytes, seed):
    return torch.randint(0, 256, (max(nbytes, 1),), dtype=torch.uint8, device=DEV,
                         generator=gen(seed))[:nbytes]


def carve(buf, offset, n, dtype):
    es = torch.empty(0, dtype=dtype).element_size()
    return buf[offset:offset + n * es].view(dtype)


def scan(tensors, item_bytes=0):
    plan = sdc.sdc_plan_build(tensors, item_bytes=item_bytes)
    out = sdc.sdc_fingerprint_plan(plan)
    torch.cuda.synchronize()
    return sdc.rows_numpy(out), plan


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_sizes_and_offsets_random_bits(dtype):
    es = ES[dtype]
    for n in SIZES:
        buf = random_bits(n * es + 16, seed=n)
        tensors = [carve(buf, off, n, dtype) for off in range(0, 16, es)]
        say(f"case sizes dtype={dtype} n={n}")
        rows, _ = scan(tensors)
        assert_rows_equal(rows, oracle_rows(tensors))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_normal_values_all_item_sizes(dtype):
    g = gen(11)
    es = ES[dtype]
    tensors = []
    for off, n in ((0, 3_000_017), (es, 1_234_567), (6 * es, 77_777), (2 * es, 5)):
        buf = torch.zeros(n * es + 16, dtype=torch.uint8, device=DEV)
        t = carve(buf, off, n, dtype)
        t.normal_(0, 0.02, generator=g)
        tensors.append(t)
    ref = oracle_rows(tensors)
    for ib in (0, 16, 48, 4096, 65536, 1 << 20, 4 << 20):
        say(f"case items dtype={dtype} item_bytes={ib}")
        rows, plan = scan(tensors, item_bytes=ib)
        assert_rows_equal(rows, ref)


def test_misaligned_clone_views_and_nonfinite_patterns():
    # every NaN/Inf class, in every dtype, at head, body and tail positions
    specials = {torch.float32: [0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001, 0xFFFFFFFF],
                torch.bfloat16: [0x7F80, 0xFF80, 0x7FC0, 0x7F81, 0xFFFF],
                torch.float16: [0x7C00, 0xFC00, 0x7E00, 0x7C01, 0xFFFF]}
    rng = np.random.default_rng(21)
    tensors = []
    for dtype, pats in specials.items():
        es = ES[dtype]
        for n in (3, 17, 4099, 300_001):
            buf = torch.zeros(n * es + 16, dtype=torch.uint8, device=DEV)
            t = carve(buf, es, n, dtype)
            t.normal_(0, 0.02, generator=gen(n))
            iv = t.view(torch.int32 if es == 4 else torch.int16)
            pos = sorted(set([0, n - 1, n // 2] + rng.integers(0, n, size=min(n, 9)).tolist()))
            for j, p in enumerate(pos):
                v = pats[j % len(pats)]
                iv[p] = v - (1 << (8 * es)) if v >= 1 << (8 * es - 1) else v
            tensors.append(t)
    say("case nonfinite patterns")
    rows, plan = scan(tensors)
    assert_rows_equal(rows, oracle_rows(tensors))
    counts, total = sdc.sdc_nonfinite(plan)
    torch.cuda.synchronize()
    ref = oracle_nonfinite(tensors)
    assert counts.cpu().numpy().astype(np.uint64).tolist() == ref.tolist()
    assert int(total.item()) == int(ref.sum())


def test_launch_shapes_rows_counts_and_norms():
    # A plan's workgroup items run in one of three launch shapes chosen by the
    # average item size: short (< 96 KiB), deep (96-512 KiB) and wide (>= 512 KiB:
    # one workgroup per CU, non-pipelined rounds of 12 vectors per lane).  Rows,
    # NaN/Inf counts and squared norms equal the oracle's in every shape, with
    # sparse NaN/Inf (every class, misaligned heads, ragged tails) and with random
    # bits (one element in 256 is NaN/Inf, and one in 32 trips the packed fp16
    # pre-check, so most lanes' rounds are counted exactly).
    from _util import assert_sq_close, oracle_sqnorms
    specials = {4: [0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001, 0xFFFFFFFF],
                2: [0x7F80, 0xFF80, 0x7FC0, 0x7F81, 0xFFFF]}
    rng = np.random.default_rng(31)
    tensors = []
    for dtype, off, n in ((torch.float32, 0, 6_000_000), (torch.bfloat16, 2, 5_000_003),
                          (torch.float16, 6, 3_000_001)):
        es = ES[dtype]
        buf = torch.zeros(n * es + 16, dtype=torch.uint8, device=DEV)
        t = carve(buf, off, n, dtype)
        t.normal_(0, 0.02, generator=gen(n))
        iv = t.view(torch.int32 if es == 4 else torch.int16)
        pos = sorted(set([0, n - 1] + rng.integers(0, n, size=40).tolist()))
        pats = specials[es] if dtype != torch.float16 else [0x7C00, 0xFC00, 0x7E00, 0x7C01, 0xFFFF]
        for j, p in enumerate(pos):
            v = pats[j % len(pats)]
            iv[p] = v - (1 << (8 * es)) if v >= 1 << (8 * es - 1) else v
        tensors.append(t)
    tensors.append(random_bits(2 * 2_000_005, seed=77).view(torch.bfloat16))
    # small tensors (wave items), a missing and an empty one in the same launches
    tiny = random_bits(4 * 3000 + 16, seed=78)
    tensors += [carve(tiny, 4, 1, torch.float32), None, carve(tiny, 2, 7, torch.bfloat16),
                tiny[:0].view(torch.float16), carve(tiny, 6, 2000, torch.float16),
                carve(tiny, 8, 100, torch.float32)]
    ref_rows = oracle_rows(tensors)
    ref_nf = oracle_nonfinite(tensors)
    ref_sq = oracle_sqnorms(tensors)
    numels = [0 if t is None else t.numel() for t in tensors]
    assert int(ref_nf[3]) > 5_000  # the random-bits tensor: about 2M / 256 NaN/Inf
    for ib, want in ((65536, "short"), (256 << 10, "deep"), (1 << 20, "wide"), (4 << 20, "wide")):
        plan = sdc.sdc_plan_build(tensors, item_bytes=ib)
        avg = plan.total_bytes // plan.n_items
        shape = "wide" if avg >= 512 << 10 else ("deep" if avg >= 96 << 10 else "short")
        assert shape == want, (ib, avg)
        say(f"case launch shape {shape} item_bytes={ib}")
        out = sdc.sdc_fingerprint_plan(plan)
        counts, total = sdc.sdc_nonfinite(plan)
        sq, sq_total, flag = sdc.sdc_sqnorm(plan)
        torch.cuda.synchronize()
        assert_rows_equal(sdc.rows_numpy(out), ref_rows)
        assert counts.cpu().numpy().astype(np.uint64).tolist() == ref_nf.tolist()
        assert int(total.item()) == int(ref_nf.sum())
        assert_sq_close(sq.cpu().tolist(), ref_sq, numels)
        assert int(flag.item()) == 1


def test_large_finite_bf16_are_not_counted():
    # bf16 values with exponent 0xF8..0xFE look like fp16 NaN/Inf to the packed
    # pre-check; the exact count must not count them.
    g = gen(5)
    t = torch.empty(1 << 20, dtype=torch.bfloat16, device=DEV).normal_(0, 0.02, generator=g)
    iv = t.view(torch.int16)
    iv[::97] = 0x7C00 + 0x55   # exponent 0xF8, finite
    iv[::1013] = 0x7F00        # exponent 0xFE, finite
    iv[5] = 0x7F80             # +Inf
    say("case large finite bf16")
    rows, plan = scan([t])
    assert_rows_equal(rows, oracle_rows([t]))
    assert int(rows[0, 3]) == 1


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_every_16bit_pattern_nan_dense(dtype):
    # all 2^16 patterns (shuffled) in a tensor of several rounds per lane and in
    # wave-item-sized slices: NaN/Inf in almost every lane's every round, so the
    # exact count of flagged rounds runs everywhere
    rng = np.random.default_rng(33)
    pats = rng.permutation(1 << 16).astype(np.int64)
    pats = np.where(pats >= 1 << 15, pats - (1 << 16), pats).astype(np.int16)
    big = torch.from_numpy(np.tile(pats, 5)[:5 * 65536 - 3].copy()).to(DEV).view(dtype)
    tensors = [big, big[1:]] + [big[k * 4096 + (k % 8):(k + 1) * 4096] for k in range(16)]
    say(f"case every 16-bit pattern {dtype}")
    rows, plan = scan(tensors)
    assert_rows_equal(rows, oracle_rows(tensors))
    counts, total = sdc.sdc_nonfinite(plan)
    one = sdc.sdc_fingerprint_tensor(big)
    torch.cuda.synchronize()
    ref = oracle_nonfinite(tensors)
    assert counts.cpu().numpy().astype(np.uint64).tolist() == ref.tolist()
    assert int(total.item()) == int(ref.sum())
    assert_rows_equal(sdc.rows_numpy(one), oracle_rows([big]))
    # each copy of the 2^16 patterns holds 2^(16-E) with the E exponent bits all ones
    mask = 0x7F80 if dtype == torch.bfloat16 else 0x7C00
    dropped = sum(1 for p in pats[-3:] if int(p) & mask == mask)
    assert int(rows[0, 3]) == 5 * (1 << (16 - bin(mask).count("1"))) - dropped


def test_none_empty_and_many_tiny_tensors():
    g = gen(9)
    rng = np.random.default_rng(9)
    tensors = []
    for k in range(5000):
        kind = k % 7
        if kind == 0:
            tensors.append(None)
        elif kind == 1:
            tensors.append(torch.empty(0, dtype=torch.float32, device=DEV))
        else:
            dt = [torch.float32, torch.bfloat16, torch.float16][int(rng.integers(0, 3))]
            n = int(rng.integers(1, 40))
            tensors.append(torch.empty(n, dtype=dt, device=DEV).normal_(0, 1, generator=g))
    say("case none/empty/tiny")
    rows, _ = scan(tensors)
    assert_rows_equal(rows, oracle_rows(tensors))
    out = sdc.sdc_fingerprint(tensors)  # one-shot form
    torch.cuda.synchronize()
    assert_rows_equal(sdc.rows_numpy(out), rows)


def test_repeated_scans_and_stale_output_are_overwritten():
    g = gen(3)
    ts = [torch.empty(n, dtype=torch.bfloat16, device=DEV).normal_(0, 0.02, generator=g)
          for n in (5_000_000, 123, 2_000_001)]
    plan = sdc.sdc_plan_build(ts, item_bytes=65536)
    out = torch.full((3, 4), -1, dtype=torch.int64, device=DEV)  # garbage must be cleared
    ref = oracle_rows(ts)
    for i in range(5):
        say(f"case repeat {i}")
        sdc.sdc_fingerprint_plan(plan, out)
        torch.cuda.synchronize()
        assert_rows_equal(sdc.rows_numpy(out), ref)


def test_plan_errors_are_reported():
    t = torch.zeros(4, dtype=torch.float32, device=DEV)
    with pytest.raises(sdc.SdcError):
        sdc.sdc_plan_build([t], item_bytes=24)  # not a multiple of 16
    with pytest.raises(ValueError):
        sdc.sdc_plan_build([t[::2]])  # plans read tensors in place: must be contiguous


# ---------------------------------------------------------------------------
# majority and diff kernels
# ---------------------------------------------------------------------------
def random_table(R, T, rng, p_diff=0.3, palette=3):
    base = rng.integers(0, 1 << 63, size=(T, 4), dtype=np.uint64)
    alt = rng.integers(0, 1 << 63, size=(palette, T, 4), dtype=np.uint64)
    table = np.repeat(base[None], R, axis=0)
    for r in range(R):
        for k in range(T):
            if rng.random() < p_diff:
                c = int(rng.integers(0, palette))
                col = int(rng.integers(0, 4))
                table[r, k] = base[k]
                table[r, k, col] = alt[c, k, col]
    return table.reshape(R * T, 4)


def to_dev(table):
    return torch.from_numpy(np.ascontiguousarray(table).view(np.int64)).to(DEV)


@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 7, 16])
def test_majority_matches_oracle(R):
    rng = np.random.default_rng(R)
    for T in (1, 2, 7, 300, 5000):
        for p in (0.0, 0.01, 0.3):
            for mask in (O.COL_ALL, O.COL_SUM | O.COL_WSUM, O.COL_XOR):
                table = random_table(R, T, rng, p)
                say(f"case majority R={R} T={T} p={p} mask={mask}")
                status = torch.zeros(T, dtype=torch.uint8, device=DEV)
                got = sdc.sdc_majority_compare(to_dev(table), R, T, col_mask=mask,
                                               tensor_status=status)
                ref = O.majority_compare(table, R, T, mask)
                for key in ("diverged", "has_majority", "n_diff", "first_diff",
                            "first_no_majority", "suspects"):
                    assert got[key] == ref[key], (key, got[key], ref[key])
                assert np.array_equal(got["suspect_flags"], ref["suspect_flags"])
                assert np.array_equal(status.cpu().numpy(), ref["tensor_status"])


@pytest.mark.parametrize("R,T", [(1024, 3), (1025, 3), (3, 1024), (3, 1025), (1100, 40)])
def test_majority_one_workgroup_and_grid_paths(R, T):
    # tables of at most 1024 replicas and 1024 tensors take the one-workgroup
    # path; the boundary cases on either side must agree with the oracle
    rng = np.random.default_rng(R * 7 + T)
    for p in (0.0, 0.002, 0.05):
        table = random_table(R, T, rng, p, palette=2)
        say(f"case majority paths R={R} T={T} p={p}")
        got = sdc.sdc_majority_compare(to_dev(table), R, T)
        ref = O.majority_compare(table, R, T, O.COL_ALL)
        for key in ("diverged", "has_majority", "n_diff", "first_diff", "first_no_majority",
                    "suspects"):
            assert got[key] == ref[key], (key, got[key], ref[key])
        assert np.array_equal(got["suspect_flags"], ref["suspect_flags"])


def test_majority_rejects_bad_arguments():
    t = to_dev(np.zeros((3, 4), dtype=np.uint64))
    with pytest.raises(sdc.SdcError):
        sdc.sdc_majority_compare(t, 3, 1, col_mask=0)
    with pytest.raises(sdc.SdcError):
        sdc.sdc_majority_compare(t, 3, 1, col_mask=16)


def test_diff_matches_oracle():
    rng = np.random.default_rng(77)
    for T in (1, 5, 1023, 1024, 1025, 4097, 300_000):
        a = rng.integers(0, 1 << 63, size=(T, 4), dtype=np.uint64)
        b = a.copy()
        nd = int(rng.integers(0, min(T, 50) + 1))
        hit = rng.choice(T, size=nd, replace=False)
        for j, k in enumerate(hit):
            if j % 2 == 0:  # the exact signature of one bit flip
                i, bit = int(rng.integers(0, 1 << 20)), int(rng.integers(0, 32))
                d = 1 << bit
                a[k, 2] &= ~np.uint64(d)
                b[k, 2] = a[k, 2] | np.uint64(d)
                b[k, 0] = a[k, 0] + np.uint64(d)
                b[k, 1] = a[k, 1] + np.uint64((i + 1) * d)
            else:
                b[k, int(rng.integers(0, 4))] ^= np.uint64(int(rng.integers(1, 1 << 30)))
        for mask in (O.COL_ALL, O.COL_SUM | O.COL_WSUM):
            for cap in (None, 0, 3):
                say(f"case diff T={T} nd={nd} mask={mask} cap={cap}")
                got = sdc.sdc_fingerprint_diff(to_dev(a), to_dev(b), col_mask=mask, idx_cap=cap)
                ref = O.fingerprint_diff(a, b, mask, cap=T if cap is None else cap)
                assert got["n_diff"] == ref["n_diff"]
                assert got["indices"] == ref["indices"]
                assert got["hints"] == ref["hints"]
        got = sdc.sdc_fingerprint_diff(to_dev(a), to_dev(b), hints=False)
        assert got["indices"] == O.fingerprint_diff(a, b, O.COL_ALL, cap=T)["indices"]
        if T <= 1025:  # an index cap far above T, through the C ABI: it counts as T
            say(f"case diff T={T} huge cap")
            got = diff_raw(to_dev(a), to_dev(b), T, (1 << 58) - 1)
            ref = O.fingerprint_diff(a, b, O.COL_ALL, cap=T)
            assert got == (0, ref["n_diff"], ref["indices"])


def diff_raw(da, db, T, cap):
    """sdc_fingerprint_diff through ctypes with an index array of T entries
    (what the call may write: min(n_diff, cap) <= T)."""
    import ctypes
    lib = ctypes.CDLL(sdc.LIB_PATH)
    ws_b = ctypes.c_uint64(0)
    assert lib.sdc_diff_ws_bytes(ctypes.c_uint64(T), ctypes.c_uint64(cap), ctypes.byref(ws_b)) == 0
    ws = torch.empty(ws_b.value, dtype=torch.uint8, device=DEV)
    n = ctypes.c_uint64(0)
    idx = (ctypes.c_uint64 * T)()
    st = lib.sdc_fingerprint_diff(
        ctypes.c_void_p(da.data_ptr()), ctypes.c_void_p(db.data_ptr()), ctypes.c_uint64(T),
        ctypes.c_uint32(O.COL_ALL), ctypes.c_void_p(ws.data_ptr()), ctypes.c_uint64(ws.numel()),
        ctypes.byref(n), idx, ctypes.c_uint64(cap), None,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, n.value, [int(idx[i]) for i in range(min(n.value, T))]


# ---------------------------------------------------------------------------
# every element type, zero- and sign-extended
# ---------------------------------------------------------------------------
ALL_TYPES = [torch.float32, torch.bfloat16, torch.float16, torch.float64, torch.uint8, torch.int8,
             torch.float8_e4m3fn, torch.float8_e5m2, torch.float8_e4m3fnuz, torch.float8_e5m2fnuz,
             torch.int16, torch.int32, torch.int64]
TYPE_SIZES = [1, 2, 3, 7, 15, 16, 17, 33, 255, 511, 513, 4095, 4097, 8191, 8193, 65537, 1_000_003]


@pytest.mark.parametrize("dtype", ALL_TYPES, ids=[str(t).split(".")[1] for t in ALL_TYPES])
@pytest.mark.parametrize("signed", [False, True])
def test_all_types_sizes_offsets(dtype, signed):
    es = torch.empty(0, dtype=dtype).element_size()
    flags = O.SIGNED if signed else 0
    for n in TYPE_SIZES:
        buf = random_bits(n * es + 16, seed=1000 + n)
        tensors = [carve(buf, off, n, dtype) for off in range(0, 16, es)]
        say(f"case types dtype={dtype} signed={signed} n={n}")
        plan = sdc.sdc_plan_build(tensors, signed=signed)
        out = sdc.sdc_fingerprint_plan(plan)
        counts, total = sdc.sdc_nonfinite(plan)
        torch.cuda.synchronize()
        ref = oracle_rows(tensors, flags=flags)
        assert_rows_equal(sdc.rows_numpy(out), ref)
        assert counts.cpu().numpy().astype(np.uint64).tolist() == ref[:, 3].tolist()
        assert int(total.item()) == int(ref[:, 3].sum())


@pytest.mark.parametrize("dtype", ALL_TYPES, ids=[str(t).split(".")[1] for t in ALL_TYPES])
@pytest.mark.parametrize("signed", [False, True])
def test_all_types_deep_and_wide_shapes(dtype, signed):
    # the deep (96-512 KiB items) and wide (>= 512 KiB) launch shapes for every
    # element type and widening mode: rows, NaN/Inf counts and squared norms
    from _util import assert_sq_close, oracle_sqnorms
    es = torch.empty(0, dtype=dtype).element_size()
    n = 3_000_007
    buf = random_bits(n * es + 16, seed=2000 + es)
    tensors = [carve(buf, off, n, dtype) for off in range(0, 16, max(es, 4))]
    ref = oracle_rows(tensors, flags=O.SIGNED if signed else 0)
    ref_sq = oracle_sqnorms(tensors)
    for ib, want in ((256 << 10, "deep"), (1 << 20, "wide"), (4 << 20, "wide")):
        plan = sdc.sdc_plan_build(tensors, item_bytes=ib, signed=signed)
        avg = plan.total_bytes // plan.n_items
        assert ("wide" if avg >= 512 << 10 else "deep" if avg >= 96 << 10 else "short") == want
        say(f"case types shape={want} dtype={dtype} signed={signed} item_bytes={ib}")
        out = sdc.sdc_fingerprint_plan(plan)
        counts, total = sdc.sdc_nonfinite(plan)
        sq, _, _ = sdc.sdc_sqnorm(plan)
        torch.cuda.synchronize()
        assert_rows_equal(sdc.rows_numpy(out), ref)
        assert counts.cpu().numpy().astype(np.uint64).tolist() == ref[:, 3].tolist()
        assert int(total.item()) == int(ref[:, 3].sum())
        assert_sq_close(sq.cpu().tolist(), ref_sq, [t.numel() for t in tensors])


def test_all_types_item_sizes_and_mixed_lists():
    rng = np.random.default_rng(99)
    tensors = []
    for k in range(3000):
        dt = ALL_TYPES[int(rng.integers(0, len(ALL_TYPES)))]
        es = torch.empty(0, dtype=dt).element_size()
        n = int(np.exp(rng.uniform(0, np.log(300_000))))
        off = es * int(rng.integers(0, 16 // es))
        tensors.append(carve(random_bits(n * es + 16, seed=5000 + k), off, n, dt))
    for signed in (False, True):
        ref = oracle_rows(tensors, flags=O.SIGNED if signed else 0)
        for ib in (0, 768, 4096, 1 << 20):
            say(f"case mixed types signed={signed} item_bytes={ib}")
            plan = sdc.sdc_plan_build(tensors, item_bytes=ib, signed=signed)
            out = sdc.sdc_fingerprint_plan(plan)
            torch.cuda.synchronize()
            assert_rows_equal(sdc.rows_numpy(out), ref)


def test_fp8_and_fp64_special_patterns():
    # every fp8 pattern repeated, and fp64 NaN/Inf at head, body and tail
    b = torch.arange(256, dtype=torch.int16, device=DEV).to(torch.uint8).repeat(1000)
    tensors = [b.view(t) for t in (torch.float8_e4m3fn, torch.float8_e5m2,
                                   torch.float8_e4m3fnuz, torch.float8_e5m2fnuz, torch.uint8)]
    d = torch.empty(100_001, dtype=torch.float64, device=DEV).normal_(generator=gen(8))
    iv = d.view(torch.int64)
    iv[0] = 0x7FF0000000000000
    iv[50_000] = -0x0008000000000000  # 0xFFF8..., a negative quiet NaN
    iv[-1] = 0x7FF0000000000001
    tensors.append(d)
    say("case fp8/fp64 specials")
    rows, plan = scan(tensors)
    ref = oracle_rows(tensors)
    assert_rows_equal(rows, ref)
    assert rows[:, 3].tolist() == [2000, 8000, 1000, 1000, 0, 3]


@pytest.mark.parametrize("dtype,signed", [(torch.uint8, False), (torch.bfloat16, True),
                                          (torch.float16, False)])
def test_tensor_with_more_than_2_32_elements(dtype, signed):
    # positions i + 1 beyond 2^32 (the weighted sum's 64-bit position products),
    # through the list scan (automatic and 4 MiB items) and the single-tensor scan
    es = torch.empty(0, dtype=dtype).element_size()
    n = (1 << 32) + 12_345
    raw = torch.empty(n * es + 16, dtype=torch.uint8, device=DEV)
    g = gen(32)
    for lo in range(0, raw.numel(), 1 << 30):  # random bytes, 1 GiB at a time
        hi = min(raw.numel(), lo + (1 << 30))
        raw[lo:hi].random_(0, 256, generator=g)
    t = carve(raw, 2 * es if es > 1 else 3, n, dtype)
    say(f"case >2^32 elements dtype={dtype} signed={signed}: oracle")
    ref = oracle_rows([t], threads=1, flags=O.SIGNED if signed else 0)
    for ib in (0, 4 << 20):
        say(f"case >2^32 elements item_bytes={ib}")
        plan = sdc.sdc_plan_build([t], item_bytes=ib, signed=signed)
        out = sdc.sdc_fingerprint_plan(plan)
        torch.cuda.synchronize()
        assert_rows_equal(sdc.rows_numpy(out), ref)
        del plan
    r = sdc.sdc_fingerprint_tensor(t, signed=signed)
    torch.cuda.synchronize()
    assert_rows_equal(sdc.rows_numpy(r), ref)
    del raw, t
    torch.cuda.empty_cache()


def test_non_contiguous_inputs_use_logical_order():
    # the pages' fingerprint reads a tensor's contiguous (row-major) form; the
    # one-shot and single-tensor scans copy a strided view first, a plan refuses it
    g = gen(41)
    a = torch.empty((300, 517), dtype=torch.float32, device=DEV).normal_(0, 1, generator=g)
    b = torch.empty((64, 33, 7), dtype=torch.float32, device=DEV).normal_(0, 1,
                                                                          generator=g).bfloat16()
    views = [a.t(), a[:, ::3], b.permute(2, 0, 1), b[::2, 1:]]
    assert not any(v.is_contiguous() for v in views)
    ref = oracle_rows([v.contiguous() for v in views])
    out = sdc.sdc_fingerprint(views)
    torch.cuda.synchronize()
    assert_rows_equal(sdc.rows_numpy(out), ref)
    for k, v in enumerate(views):
        r = sdc.sdc_fingerprint_tensor(v)
        torch.cuda.synchronize()
        assert_rows_equal(sdc.rows_numpy(r), ref[k:k + 1])
    with pytest.raises(ValueError):
        sdc.sdc_plan_build(views)
