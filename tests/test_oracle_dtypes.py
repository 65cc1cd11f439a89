"""Pins for the oracle's 1-, 2-, 4- and 8-byte element types and its signed
mode (CPU only).

- Big-integer brute force from raw bytes (int.from_bytes, signed for 2-/4-byte
  elements in signed mode; W as a sum of suffix sums).
- The pages' definition ("Compare by fingerprint": view 1/2/4/8-byte elements
  as uint8/int16/int32/int64, widen to int64, plain sum and sum weighted by
  1-based position) evaluated with torch int64 ops: signed mode must equal it.
- Closed forms tying signed and unsigned rows through the count and the
  positions of elements with the top bit set.
- NaN/Inf over all 256 patterns of every fp8 encoding against torch, fp64
  against numpy, and never for the raw integer types.
"""
import functools

import numpy as np
import pytest
import torch

import oracle as O

M64 = (1 << 64) - 1
ALL = [O.F32, O.BF16, O.F16, O.F64, O.U8, O.FP8_E4M3, O.FP8_E5M2, O.FP8_E4M3FNUZ,
       O.FP8_E5M2FNUZ, O.U16, O.U32, O.U64]
NP_UINT = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}
TORCH_VIEW = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}
FP8 = {O.FP8_E4M3: torch.float8_e4m3fn, O.FP8_E5M2: torch.float8_e5m2,
       O.FP8_E4M3FNUZ: torch.float8_e4m3fnuz, O.FP8_E5M2FNUZ: torch.float8_e5m2fnuz}


def rand_raw(rng, n, es):
    raw = rng.integers(0, 256, size=n * es, dtype=np.uint64).astype(np.uint8)
    # sprinkle all-ones / top-bit / zero elements
    for i in rng.choice(n, size=min(n, 3), replace=False) if n else []:
        raw[i * es:(i + 1) * es] = [0xFF, 0x80, 0x00][int(rng.integers(0, 3))]
    return raw


def brute(raw, es, signed):
    xs = [int.from_bytes(bytes(raw[i:i + es]), "little", signed=signed and es in (2, 4))
          for i in range(0, len(raw), es)]
    s = sum(xs) & M64
    suffix = w = 0
    for v in reversed(xs):
        suffix += v
        w += suffix
    x = functools.reduce(lambda a, b: a ^ b, [v & M64 for v in xs], 0)
    return s, w & M64, x


@pytest.mark.parametrize("dtype", ALL)
@pytest.mark.parametrize("flags", [0, O.SIGNED])
def test_brute_force_all_types(dtype, flags):
    es = O.ESIZE[dtype]
    rng = np.random.default_rng(dtype * 7 + flags)
    for n in range(0, 17):
        for _ in range(25):
            raw = rand_raw(rng, n, es)
            assert O.fingerprint(raw, dtype, flags)[:3] == brute(raw, es, bool(flags))


def pages_definition(raw, es):
    """(S, W) of the pages' fingerprint: the integer view by element size,
    widened to int64, plain and 1-based-position-weighted sums (torch int64
    arithmetic wraps modulo 2^64)."""
    t = torch.from_numpy(raw.copy()).view(TORCH_VIEW[es]).to(torch.int64)
    pos = torch.arange(1, t.numel() + 1, dtype=torch.int64)
    return int(t.sum()) & M64, int((t * pos).sum()) & M64


@pytest.mark.parametrize("es,dtype", [(1, O.U8), (2, O.BF16), (2, O.F16), (4, O.F32), (8, O.F64)])
def test_signed_mode_equals_the_pages_definition(es, dtype):
    rng = np.random.default_rng(es)
    for n in (1, 2, 3, 100, 4097, 300_001):
        raw = rng.integers(0, 256, size=n * es, dtype=np.uint64).astype(np.uint8)
        assert O.fingerprint(raw, dtype, O.SIGNED)[:2] == pages_definition(raw, es)
    # normal-distributed weights, as a training run has them
    if dtype in (O.F32, O.BF16, O.F16):
        v = torch.randn(200_003, generator=torch.Generator().manual_seed(1)) * 0.02
        v = v.to({O.F32: torch.float32, O.BF16: torch.bfloat16, O.F16: torch.float16}[dtype])
        raw = v.view(torch.uint8).numpy().copy()
        assert O.fingerprint(raw, dtype, O.SIGNED)[:2] == pages_definition(raw, es)


@pytest.mark.parametrize("es,dtype", [(2, O.BF16), (4, O.F32), (2, O.U16), (4, O.U32)])
def test_signed_unsigned_closed_form(es, dtype):
    # S_signed = S - 2^(8w) N_msb and W_signed = W - 2^(8w) sum_{msb set} (i+1);
    # X_signed is X sign-extended from the element width.
    rng = np.random.default_rng(30 + es)
    for n in (1, 5, 1000, 65537):
        x = rng.integers(0, 1 << (8 * es), size=n, dtype=np.uint64).astype(NP_UINT[es])
        su, wu, xu, _ = O.fingerprint(x, dtype)
        ss, ws, xs, _ = O.fingerprint(x, dtype, O.SIGNED)
        msb = (x.astype(np.uint64) >> np.uint64(8 * es - 1)) & np.uint64(1)
        nmsb = int(msb.sum())
        pos = int((np.nonzero(msb)[0] + 1).sum())
        big = 1 << (8 * es)
        assert ss == (su - big * nmsb) & M64
        assert ws == (wu - big * pos) & M64
        sext = xu - big if xu >> (8 * es - 1) else xu
        assert xs == sext & M64


@pytest.mark.parametrize("dtype", [O.U8, O.F64, O.U64])
def test_signed_flag_does_not_change_1_and_8_byte_elements(dtype):
    rng = np.random.default_rng(40 + dtype)
    raw = rng.integers(0, 256, size=8 * 1001, dtype=np.uint64).astype(np.uint8)
    assert O.fingerprint(raw, dtype) == O.fingerprint(raw, dtype, O.SIGNED)


def test_eight_byte_closed_forms_wrap():
    n = 100_003
    for c in (1, 0x8000000000000001, M64, 0x0123456789ABCDEF):
        x = np.full(n, c, dtype=np.uint64)
        s, w, xr, _ = O.fingerprint(x, O.U64)
        assert s == (n * c) & M64 and w == (c * n * (n + 1) // 2) & M64
        assert xr == (c if n % 2 else 0)


@pytest.mark.parametrize("dtype", list(FP8))
def test_fp8_nonfinite_exhaustive(dtype):
    b = np.arange(256, dtype=np.uint16).astype(np.uint8)
    lib_bad = (~torch.isfinite(torch.from_numpy(b.copy()).view(FP8[dtype]).float())).numpy()
    ours = np.array([O.lib().oracle_is_nonfinite(int(v), dtype) for v in b], dtype=bool)
    assert np.array_equal(ours, lib_bad)
    assert O.fingerprint(b, dtype)[3] == int(lib_bad.sum())


def test_fp64_nonfinite_sampled():
    rng = np.random.default_rng(50)
    x = rng.integers(0, 1 << 64, size=1 << 18, dtype=np.uint64)
    x[::7] |= np.uint64(0x7FF0000000000000)
    x[::11] &= ~np.uint64(1 << 52)
    want = int(np.count_nonzero(~np.isfinite(x.view(np.float64))))
    assert O.fingerprint(x, O.F64)[3] == want


@pytest.mark.parametrize("dtype", [O.U8, O.U16, O.U32, O.U64])
def test_raw_integer_types_are_never_nonfinite(dtype):
    es = O.ESIZE[dtype]
    raw = np.random.default_rng(dtype).integers(0, 256, size=es * 70000, dtype=np.uint64)
    raw = raw.astype(np.uint8)
    raw[:es * 4] = 0xFF
    assert O.fingerprint(raw, dtype)[3] == 0


def test_bad_flags_rejected():
    import ctypes
    r = O.Row()
    assert O.lib().oracle_fingerprint_ex(None, 0, O.F32, 2, ctypes.byref(r)) == -1
