"""GPU parity of the squared norm (the norm-based form of "Check 1: NaN/Inf
gradients, before and after the all-reduce", AWS blog post) through the C ABI.

Per-tensor values are sums of non-negative doubles, so the oracle's
index-order sum and the kernel's tree sum of the same exact terms differ by at
most 2 (n + 1) 2^-53 times the sum (each side's rounding is below
(n + 1) 2^-53 relative: n additions, one product rounding for fp64).  NaN and
Inf results must match exactly, and so must the flag wherever the total is not
within that bound of the fp32 threshold.  Repeated calls on one plan are
bit-identical.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle as O
import silent_corruption_detection_amd as sdc
from _util import CODE, host_bytes, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
FLOATS = [torch.float32, torch.bfloat16, torch.float16, torch.float64, torch.float8_e4m3fn,
          torch.float8_e5m2, torch.float8_e4m3fnuz, torch.float8_e5m2fnuz]
ALL = FLOATS + [torch.uint8, torch.int16, torch.int32, torch.int64]
IDS = [str(t).split(".")[1] for t in ALL]


def gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def carve(buf, offset, n, dtype):
    es = torch.empty(0, dtype=dtype).element_size()
    return buf[offset:offset + n * es].view(dtype)


def tol(n, ref):
    return (2 * n + 2) * 2.0 ** -53 * abs(ref)


def close(got, ref, n):
    if math.isnan(ref) or math.isinf(ref):
        return (math.isnan(got) and math.isnan(ref)) or got == ref
    return abs(got - ref) <= tol(n, ref)


def oracle_sq(tensors):
    return [O.sqnorm(host_bytes(t), CODE[t.dtype]) if t is not None else 0.0 for t in tensors]


def run(tensors, item_bytes=0):
    plan = sdc.sdc_plan_build(tensors, item_bytes=item_bytes)
    sq, total, flag = sdc.sdc_sqnorm(plan)
    torch.cuda.synchronize()
    return plan, sq.cpu().numpy(), float(total.item()), int(flag.item())


def check(tensors, item_bytes=0):
    ns = [t.numel() if t is not None else 0 for t in tensors]
    ref = oracle_sq(tensors)
    _, sq, total, flag = run(tensors, item_bytes)
    for k, (g, r, n) in enumerate(zip(sq.tolist(), ref, ns)):
        assert close(g, r, n), (k, tensors[k].dtype if tensors[k] is not None else None, n, g, r)
    ref_total = math.fsum(ref) if all(map(math.isfinite, ref)) else sum(ref)
    assert close(total, ref_total, sum(ns) + len(ns))
    near = math.isfinite(ref_total) and abs(ref_total - 3.4028234663852886e38) <= tol(sum(ns) + len(ns), ref_total)
    if not near:
        assert flag == O.sqnorm_flag(ref_total)
    return sq, total, flag


def normal_values(n, dtype, seed, scale=1.0):
    g = gen(seed)
    x = torch.empty(max(n, 1), dtype=torch.float32, device=DEV).normal_(0, scale, generator=g)[:n]
    if dtype.is_floating_point:
        return x.to(dtype)
    return torch.randint(0, 100, (n,), device=DEV, generator=g).to(dtype)


@pytest.mark.parametrize("dtype", ALL, ids=IDS)
def test_sizes_offsets_normal_values(dtype):
    es = torch.empty(0, dtype=dtype).element_size()
    for n in (1, 3, 7, 8, 9, 17, 63, 64, 65, 257, 1023, 4097, 8193, 65537, 262145, 1_000_003):
        say(f"case sqnorm sizes dtype={dtype} n={n}")
        vals = normal_values(n, dtype, seed=n, scale=4.0 if es == 1 else 1.0)
        tensors = []
        for off in range(0, 16, es):
            buf = torch.zeros(n * es + 16, dtype=torch.uint8, device=DEV)
            t = carve(buf, off, n, dtype)
            t.copy_(vals)
            tensors.append(t)
        check(tensors)


@pytest.mark.parametrize("dtype", FLOATS, ids=IDS[:len(FLOATS)])
def test_random_bit_patterns(dtype):
    # every pattern class: NaN, Inf, subnormals, both zeros, the largest values
    es = torch.empty(0, dtype=dtype).element_size()
    tensors = []
    for seed, n in ((1, 5), (2, 333), (3, 4096), (4, 100_003)):
        raw = torch.randint(0, 256, (n * es + 16,), dtype=torch.uint8, device=DEV, generator=gen(seed))
        tensors.append(carve(raw, es, n, dtype))
    say(f"case sqnorm bits dtype={dtype}")
    sq, total, flag = check(tensors)
    if es == 1 and dtype in (torch.float8_e5m2, torch.float8_e4m3fn):
        assert flag == 1  # random fp8 bytes hold NaN patterns


def test_every_fp8_and_16bit_pattern_one_by_one():
    # single-element tensors of every 1- and 2-byte pattern: the decoded value
    # squared must equal the oracle's exactly
    for dtype in (torch.float8_e4m3fn, torch.float8_e5m2, torch.float8_e4m3fnuz,
                  torch.float8_e5m2fnuz, torch.bfloat16, torch.float16):
        es = torch.empty(0, dtype=dtype).element_size()
        n = 1 << (8 * es)
        raw = torch.arange(n, dtype=torch.int32, device=DEV)
        raw = raw.to(torch.uint8) if es == 1 else raw.to(torch.int16)
        buf = raw.view(dtype)
        tensors = [buf[i:i + 1] for i in range(0, n, 1 if es == 1 else 7)]
        say(f"case sqnorm patterns dtype={dtype} tensors={len(tensors)}")
        ref = oracle_sq(tensors)
        _, sq, _, _ = run(tensors)
        for k, (g, r) in enumerate(zip(sq.tolist(), ref)):
            assert (math.isnan(g) and math.isnan(r)) or g == r, (dtype, k, g, r)


def test_overflow_threshold_and_nonfinite():
    f32 = torch.ones(1000, dtype=torch.float32, device=DEV)
    ok, over, nan, inf = f32.clone(), f32.clone(), f32.clone(), f32.clone()
    ok[10] = 1.8e19           # norm just below fp32 max: finite
    over[10] = 1.9e19         # finite element, fp32 norm overflows
    nan[999] = float("nan")
    inf[0] = float("-inf")
    big64 = torch.ones(77, dtype=torch.float64, device=DEV)
    big64[5] = 1e200          # square overflows double
    for tensors, want in (([ok], 0), ([over], 1), ([nan], 1), ([inf], 1), ([big64], 1),
                          ([ok, f32], 0), ([f32, over], 1)):
        say(f"case sqnorm threshold want={want}")
        _, _, flag = check(tensors)
        assert flag == want
    # a list whose norm overflows only in total (2.0e38 per tensor, 6.1e38 in all)
    parts = [torch.full((1000,), 4.5e17, dtype=torch.float32, device=DEV) for _ in range(3)]
    _, total, flag = check(parts)
    assert flag == 1 and math.isfinite(total)
    assert not O.sqnorm_flag(O.sqnorm(host_bytes(parts[0]), O.F32))


def test_item_sizes_determinism_and_empty():
    g = gen(21)
    tensors = []
    for n, dt in ((3_000_017, torch.float32), (1_234_567, torch.bfloat16), (77_777, torch.float16),
                  (5, torch.float64), (0, torch.float32), (999_999, torch.float8_e4m3fn)):
        tensors.append(torch.empty(max(n, 1), dtype=torch.float32, device=DEV)
                       .normal_(0, 0.02, generator=g)[:n].to(dt))
    tensors.insert(2, None)
    for ib in (0, 768, 4096, 65536, 1 << 20, 4 << 20):
        say(f"case sqnorm item_bytes={ib}")
        sq, total, _ = check(tensors, item_bytes=ib)
        plan, sq2, total2, _ = run(tensors, item_bytes=ib)
        sq3, tot3, _ = sdc.sdc_sqnorm(plan)
        torch.cuda.synchronize()
        assert np.array_equal(sq.view(np.uint64), sq3.cpu().numpy().view(np.uint64))
        assert total == total2 == float(tot3.item())
        assert sq[2] == 0.0 and sq[5] == 0.0
    _, sq, total, flag = run([])
    assert sq.size == 0 and total == 0.0 and flag == 0
    _, sq, total, flag = run([None, torch.empty(0, device=DEV)])
    assert sq.tolist() == [0.0, 0.0] and flag == 0


def test_rejects_bad_arguments():
    # checked on the host before any launch
    plan = sdc.sdc_plan_build([torch.ones(10, device=DEV)])
    total = torch.empty(1, dtype=torch.float64, device=DEV)
    L = sdc._lib
    assert L.sdc_sqnorm(None, None, None, None, None, None) == -1
    assert L.sdc_sqnorm(plan.buf.data_ptr(), ctypes.byref(plan.info), None, total.data_ptr(),
                        None, None) == -1
    bad = type(plan.info).from_buffer_copy(plan.info)
    bad.magic ^= 1
    sq = torch.empty(1, dtype=torch.float64, device=DEV)
    assert L.sdc_sqnorm(plan.buf.data_ptr(), ctypes.byref(bad), sq.data_ptr(), total.data_ptr(),
                        None, None) == -6


def test_total_over_many_tensors():
    # more tensors than one chunk of the ordered total (4096): chunk sums, then
    # their sum; the total is within the bound of the oracle's and repeatable
    g = gen(31)
    sizes = torch.randint(1, 3000, (20_001,), generator=torch.Generator().manual_seed(5)).tolist()
    big = torch.empty(sum(sizes), dtype=torch.float32, device=DEV).normal_(0, 1.0, generator=g)
    tensors = list(torch.split(big, sizes))
    say(f"case sqnorm many tensors n={len(tensors)}")
    sq, total, flag = check(tensors)
    assert flag == 0
    plan = sdc.sdc_plan_build(tensors)
    _, t1, _ = sdc.sdc_sqnorm(plan)
    _, t2, _ = sdc.sdc_sqnorm(plan)
    torch.cuda.synchronize()
    assert float(t1.item()) == float(t2.item())
