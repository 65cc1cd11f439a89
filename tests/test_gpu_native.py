"""A native C++ program that uses only include/sdc.h and the HIP runtime
(tests/native/abi_demo.cpp, built by __graft_entry__.build()) scans three
replicas of a seeded tensor list with one flipped bit; its rows, majority
result and diff equal the oracle's on the same bit patterns."""
import os
import subprocess

import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "native", "abi_demo")
SPECS = [(1, O.F32), (1000, O.BF16), (1048577, O.F32), (33333, O.BF16)]
FLIP = (2, 2, 12345, 7)  # replica, tensor, element, bit


def pattern(n, k):
    """The program's seeded pattern of elements 0..n-1 of tensor k (uint32)."""
    m = np.uint64(0xFFFFFFFF)
    i = np.arange(n, dtype=np.uint64)
    h = (((i + np.uint64(1)) * np.uint64(0x9E3779B1)) & m)
    h = (h + np.uint64((k * 0x85EBCA77) & 0xFFFFFFFF)) & m
    h ^= h >> np.uint64(15)
    h = (h * np.uint64(0x2C1B3C6D)) & m
    h ^= h >> np.uint64(12)
    return h.astype(np.uint32)


def test_native_consumer_matches_the_oracle():
    assert os.path.exists(EXE), "run __graft_entry__.build() first"
    out = subprocess.run([EXE], check=True, capture_output=True, text=True, timeout=120).stdout
    lines = [l.split() for l in out.splitlines()]
    rows = np.array([[int(x) for x in l[2:]] for l in lines if l[0] == "ROW"], dtype=np.uint64)
    ref = []
    for r in range(3):
        for k, (n, dt) in enumerate(SPECS):
            p = pattern(n, k)
            if (r, k) == FLIP[:2]:
                p[FLIP[2]] ^= np.uint32(1 << FLIP[3])
            data = p if dt == O.F32 else p.astype(np.uint16)
            ref.append(O.fingerprint(data, dt))
    ref = np.array(ref, dtype=np.uint64)
    assert np.array_equal(rows, ref)
    maj = next(l for l in lines if l[0] == "MAJ")
    oref = O.majority_compare(ref, 3, 4)
    assert [int(x) for x in maj[1:5]] == [1, 1, oref["n_diff"], oref["first_diff"]]
    assert [int(x) for x in maj[5:]] == [0, 0, 1] and oref["suspects"] == [2]
    diff = next(l for l in lines if l[0] == "DIFF")
    was = (int(pattern(SPECS[FLIP[1]][0], FLIP[1])[FLIP[2]]) >> FLIP[3]) & 1
    assert [int(x) for x in diff[1:]] == [1, FLIP[1], FLIP[2], FLIP[3], -1 if was else 1]
