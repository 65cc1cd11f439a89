"""Build ``libsdc.so`` (the gfx950 HIP library behind include/sdc.h) in-tree.

hipcc cross-compiles for gfx950 without a GPU.  Packed-FP32 instruction
selection is switched off for device code (``-packed-fp32-ops``); the host
pass warns that it does not know the feature, which is expected.
"""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsdc.so")
SOURCES = ["scan.hip", "tensor.hip", "nonfinite.hip", "norm.hip", "compare.hip", "readsum.hip",
           "plan.cpp", "misc.cpp"]
ARCH = os.environ.get("SDC_OFFLOAD_ARCH", "gfx950")


def hipcc_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = (["hipcc", "-shared"] + hipcc_flags() + [os.path.join(CSRC, s) for s in SOURCES]
           + ["-o", tmp])
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if err.strip() and verbose:
        print(err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
