"""Build ``libsdc.so`` (the gfx950 HIP library behind include/sdc.h) in-tree.

hipcc cross-compiles for gfx950 without a GPU.  Packed-FP32 instruction
selection is switched off for device code (``-packed-fp32-ops``); the host
pass warns that it does not know the feature, which is expected.  Each source
is compiled to its own object (in parallel, under ``_build/``), then linked.

``python silent_corruption_detection_amd/_build.py --sanitize`` builds a
variant whose host code (the plan builder, argument checks, host decisions)
carries AddressSanitizer and UndefinedBehaviorSanitizer, into
``_build/sanitize/libsdc.so``, for CPU test runs (the binding loads it when
SDC_LIB_PATH names it; the sanitizer runtime must be preloaded, see
``SANITIZE_PRELOAD``).  Device code is built as usual.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsdc.so")
OBJ_DIR = os.path.join(ROOT, "_build", "libsdc")
SANITIZE_DIR = os.path.join(ROOT, "_build", "sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, "libsdc.so")
# host-only sanitizer flags: each -fsanitize= applies to the host pass only
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g"]
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


def sanitize_preload():
    """The shared sanitizer runtime a process that loads the sanitizer build
    must preload (LD_PRELOAD)."""
    res = subprocess.run(["hipcc", "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True)
    return res.stdout.strip()


def build(verbose: bool = False, sanitize: bool = False) -> str:
    obj_dir = SANITIZE_DIR if sanitize else OBJ_DIR
    lib = SANITIZE_LIB if sanitize else LIB
    extra = SANITIZE_FLAGS if sanitize else []
    os.makedirs(obj_dir, exist_ok=True)
    jobs = []
    for s in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(s)[0] + ".o")
        lang = ["-x", "hip"] if s.endswith(".hip") else []
        jobs.append((["hipcc", "-c"] + hipcc_flags() + extra + lang + [os.path.join(CSRC, s), "-o", obj],
                     obj))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    if verbose:
        print(f"hipcc -c {' '.join(hipcc_flags())} <{len(jobs)} sources, {workers} at a time>",
              flush=True)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        errs = list(ex.map(lambda j: _run(j[0]), jobs))
    tmp = lib + ".tmp"
    link_extra = ["-fsanitize=address,undefined", "-shared-libsan"] if sanitize else []
    errs.append(_run(["hipcc", "-shared", "--offload-arch=" + ARCH, "-fPIC"] + link_extra
                     + [o for _, o in jobs] + ["-o", tmp]))
    if verbose:
        for e in errs:
            if e.strip():
                print(e)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
