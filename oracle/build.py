"""Compile the oracle's C sources into ``oracle/libsdc_oracle.so`` with gcc.

Test infrastructure: the library it builds is loaded only by the tests, the
smoke check and the benchmark's CPU baseline.

``python oracle/build.py --sanitize`` builds the same source with clang,
AddressSanitizer and UndefinedBehaviorSanitizer into
``_build/sanitize/libsdc_oracle.so`` (loaded when SDC_ORACLE_LIB names it,
with the clang sanitizer runtime preloaded -- the runtime the HIP library's
sanitizer build uses, so both can live in one process).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libsdc_oracle.so")
SANITIZE_LIB = os.path.join(ROOT, "_build", "sanitize", "libsdc_oracle.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    src = os.path.join(HERE, "sdc_oracle.c")
    lib = SANITIZE_LIB if sanitize else LIB
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    tmp = lib + ".tmp"
    if sanitize:
        cmd = ["/opt/rocm/llvm/bin/clang", "-std=c11", "-O1", "-g", "-fPIC", "-shared",
               "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-fno-omit-frame-pointer", "-shared-libsan", "-Wall", "-Wextra", "-Werror",
               "-o", tmp, src, "-lm"]
    else:
        cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
               "-Wall", "-Wextra", "-Werror", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
