"""Build ``libsdc.so`` (the gfx950 HIP library behind include/sdc.h) in-tree.

hipcc cross-compiles for gfx950 without a GPU.  Packed-FP32 instruction
selection is switched off for device code (``-packed-fp32-ops``); the host
pass warns that it does not know the feature, which is expected.  Each source
is compiled to its own object (in parallel, under ``_build/``), then linked.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsdc.so")
OBJ_DIR = os.path.join(ROOT, "_build", "libsdc")
SOURCES = ["scan.hip", "tensor.hip", "nonfinite.hip", "norm.hip", "compare.hip", "readsum.hip",
           "noalloc.hip", "plan.cpp", "device.cpp", "misc.cpp"]
ARCH = os.environ.get("SDC_OFFLOAD_ARCH", "gfx950")
NOISE = "is not a recognized feature for this target"


def hipcc_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)} failed:\n{err}")
    return err


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = []
    for s in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o")
        lang = ["-x", "hip"] if s.endswith(".hip") else []
        jobs.append((["hipcc", "-c"] + hipcc_flags() + lang + [os.path.join(CSRC, s), "-o", obj], obj))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    if verbose:
        print(f"hipcc -c {' '.join(hipcc_flags())} <{len(jobs)} sources, {workers} at a time>",
              flush=True)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        errs = list(ex.map(lambda j: _run(j[0]), jobs))
    tmp = LIB + ".tmp"
    errs.append(_run(["hipcc", "-shared", "--offload-arch=" + ARCH, "-fPIC"]
                     + [o for _, o in jobs] + ["-o", tmp]))
    if verbose:
        for e in errs:
            if e.strip():
                print(e)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
