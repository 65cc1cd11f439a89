"""Compile tests/native/abi_demo.cpp, a C++ consumer of include/sdc.h that
links libsdc.so (host code only; run by tests/test_gpu_native.py)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "abi_demo.cpp")
    exe = os.path.join(HERE, "abi_demo")
    libdir = os.path.join(ROOT, "silent_corruption_detection_amd")
    cmd = ["hipcc", "-O2", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include"), src,
           "-o", exe + ".tmp", "-L", libdir, "-l:libsdc.so",
           "-Wl,-rpath,$ORIGIN/../../silent_corruption_detection_amd"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stderr)
    os.replace(exe + ".tmp", exe)
    return exe


if __name__ == "__main__":
    print(build(verbose=True))
