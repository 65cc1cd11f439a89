"""Compile the oracle's C sources into ``oracle/libsdc_oracle.so`` with gcc.

Test infrastructure: the library it builds is loaded only by the tests, the
smoke check and the benchmark's CPU baseline.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libsdc_oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "sdc_oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-Wall", "-Wextra", "-Werror", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
