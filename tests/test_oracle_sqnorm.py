"""Pins for the oracle's squared norm (CPU only) -- the norm-based non-finite
check of "Check 1: NaN/Inf gradients, before and after the all-reduce" (AWS
blog post): a rank is flagged when its local gradient norm is NaN or Inf in
fp32, which also happens for a finite norm above about 1.8e19.

- Element values decoded by the oracle equal torch's (bf16, fp16, all four fp8
  encodings: every bit pattern) and numpy's (fp32, fp64: samples).
- Squared sums equal numpy's float64 sums within the summation error bound,
  and exactly for small integers.
- The flag equals the pages' computation in torch fp32 (square, sum, sqrt,
  isfinite) away from the overflow threshold, and marks the threshold itself.
"""
import numpy as np
import pytest
import torch

import oracle as O

T16 = {O.BF16: torch.bfloat16, O.F16: torch.float16}
T8 = {O.FP8_E4M3: torch.float8_e4m3fn, O.FP8_E5M2: torch.float8_e5m2,
      O.FP8_E4M3FNUZ: torch.float8_e4m3fnuz, O.FP8_E5M2FNUZ: torch.float8_e5m2fnuz}


def same(a, b):
    return (np.isnan(a) and np.isnan(b)) or a == b


@pytest.mark.parametrize("dtype", list(T16) + list(T8))
def test_values_every_pattern(dtype):
    es = O.ESIZE[dtype]
    n = 1 << (8 * es)
    raw = np.arange(n, dtype=np.uint64).astype(np.uint16 if es == 2 else np.uint8)
    tt = T16.get(dtype) or T8[dtype]
    ref = torch.from_numpy(raw.view(np.int16 if es == 2 else np.uint8).copy()).view(tt).double().numpy()
    for x, r in zip(raw, ref):
        assert same(O.value(int(x), dtype), float(r)), (dtype, hex(int(x)))


def test_values_fp32_fp64_samples():
    rng = np.random.default_rng(1)
    x32 = rng.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    x32[:6] = [0, 0x80000000, 0x7F800000, 0xFF800000, 0x00000001, 0x7F7FFFFF]
    for x, r in zip(x32, x32.view(np.float32).astype(np.float64)):
        assert same(O.value(int(x), O.F32), float(r))
    x64 = rng.integers(0, 1 << 64, size=20000, dtype=np.uint64)
    x64[:3] = [0x7FF0000000000000, 0x0000000000000001, 0x7FEFFFFFFFFFFFFF]
    for x, r in zip(x64, x64.view(np.float64)):
        assert same(O.value(int(x), O.F64), float(r))


def test_raw_integers_have_no_value():
    for dt in (O.U8, O.U16, O.U32, O.U64):
        assert O.value(0x7F, dt) == 0.0
        assert O.sqnorm(np.full(100, 0xFF, dtype=np.uint8), dt) == 0.0


@pytest.mark.parametrize("dtype,npdt", [(O.F32, np.float32), (O.F16, np.float16), (O.F64, np.float64)])
def test_sqnorm_matches_numpy(dtype, npdt):
    rng = np.random.default_rng(2)
    for n in (1, 17, 100_000, 3_000_001):
        v = (rng.standard_normal(n) * 0.02).astype(npdt)
        got = O.sqnorm(v, dtype)
        d = v.astype(np.float64)
        want = float(np.sum(d * d))
        assert abs(got - want) <= 2 * n * 2.0 ** -53 * want


def test_sqnorm_exact_on_small_integers():
    v = np.arange(-500, 501, dtype=np.float32)
    assert O.sqnorm(v, O.F32) == float(sum(i * i for i in range(-500, 501)))


def test_flag_matches_the_pages_fp32_norm():
    # away from the threshold the fp32 computation of the pages decides the same
    rng = np.random.default_rng(3)
    cases = [rng.standard_normal(10_000).astype(np.float32) * s for s in (1e-3, 1.0, 1e10, 1e17)]
    big = np.ones(4, dtype=np.float32)
    big[2] = 2e19                           # finite weight, square overflows fp32
    cases.append(big)
    nan = np.ones(8, dtype=np.float32)
    nan[3] = np.nan
    cases.append(nan)
    inf = np.ones(8, dtype=np.float32)
    inf[7] = np.inf
    cases.append(inf)
    for v in cases:
        t = torch.from_numpy(v)
        pages = not bool(torch.isfinite(t.float().pow(2).sum().sqrt()))
        assert O.sqnorm_flag(O.sqnorm(v, O.F32)) == pages


def test_flag_threshold():
    fmax = float(np.finfo(np.float32).max)
    assert not O.sqnorm_flag(fmax * 0.999)
    assert O.sqnorm_flag(fmax * 1.001)
    assert not O.sqnorm_flag((1.8e19) ** 2)   # a norm of 1.8e19 is still finite
    assert O.sqnorm_flag((1.9e19) ** 2)
    assert O.sqnorm_flag(float("nan")) and O.sqnorm_flag(float("inf"))
