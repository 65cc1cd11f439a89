"""The streaming-read reference kernel (sdc_read_sum) through the C ABI: the
sum of a buffer's 32-bit words equals the sum column of the oracle's
fingerprint of the same bytes read as fp32, for sizes around every edge of
its traversal (no whole vector, a ragged last round, a partial last 1 MiB
chunk, 0..3 trailing words), with a reused workspace and at a size of several
GiB.  Argument errors are checked on the CPU in tests/test_abi.py."""
import numpy as np
import pytest
import torch

import oracle as O
import silent_corruption_detection_amd as sdc
from _util import host_bytes, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
MIB = 1 << 20


def random_words(nbytes, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    t = torch.empty(max(nbytes // 4, 1), dtype=torch.int64, device=DEV)
    t.random_(0, 1 << 32, generator=g)
    return t.to(torch.int32)[:nbytes // 4]   # every 32-bit pattern, top bit included


def expected(buf):
    return O.fingerprint(host_bytes(buf), O.F32)[0] if buf.numel() else 0


def read_sum(buf, ws=None):
    out = torch.full((1,), -1, dtype=torch.int64, device=DEV)   # stale value
    sdc.sdc_read_sum(buf, out=out, ws=ws)
    torch.cuda.synchronize()
    return int(out.cpu().numpy().view(np.uint64)[0])


SIZES = [0, 4, 12, 16, 20, 60, 4096, 4100, 32 * 1024 - 4, 32 * 1024, 64 * 1024 + 12,
         MIB - 16, MIB, MIB + 4, MIB + 16, 3 * MIB + 36, 7_000_004]


@pytest.mark.parametrize("nbytes", SIZES)
def test_read_sum_matches_oracle(nbytes):
    say(f"case read_sum {nbytes} bytes")
    buf = random_words(nbytes, seed=nbytes + 1)
    assert read_sum(buf) == expected(buf)


def test_read_sum_reused_workspace():
    # one workspace sized for the largest buffer, reused for smaller ones
    bufs = [random_words(n, seed=n) for n in (3 * MIB + 8, 20, MIB, 0, 5 * 4096 + 4)]
    ws = torch.empty(sdc.sdc_read_sum_ws_bytes(3 * MIB + 8), dtype=torch.uint8, device=DEV)
    ws.fill_(0xAB)
    for b in bufs:
        assert read_sum(b, ws) == expected(b)
    with pytest.raises(sdc.SdcError):          # too small for 3 MiB + 8 bytes (3 chunks: 24 bytes)
        sdc.sdc_read_sum(bufs[0], ws=ws[:16])


def test_read_sum_views_and_other_types():
    base = random_words(2 * MIB, seed=4)
    # a 16-byte aligned view into the buffer, and the same bytes as bf16
    v = base[4:4 + 300_001]
    assert read_sum(v) == expected(v)
    b = base.view(torch.bfloat16)[8:8 + 2 * 100_002]
    assert read_sum(b) == expected(b.view(torch.int32))
    with pytest.raises(sdc.SdcError):          # 4-byte but not 16-byte aligned
        sdc.sdc_read_sum(base[1:])
    with pytest.raises(sdc.SdcError):          # not a whole number of words
        sdc.sdc_read_sum(base.view(torch.uint8)[:6])


def test_read_sum_at_benchmark_size():
    # several GiB (the benchmark reads 32 GiB); 4 GiB + 12 bytes keeps the oracle to seconds
    nbytes = (4 << 30) + 12
    say(f"case read_sum {nbytes} bytes")
    buf = random_words(nbytes, seed=5)
    got = read_sum(buf)
    h = host_bytes(buf)
    assert got == O.fingerprint(h, O.F32)[0]
    del buf
    torch.cuda.empty_cache()
