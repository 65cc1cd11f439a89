"""include/sdc.h is a plain C header: a C99 program that includes it compiles
with warnings as errors, links against libsdc.so and calls the host-only entry
points (no GPU: sizing, validation, status strings), with results equal to the
Python binding's."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "sdc.h"

int main(void) {
  sdc_tensor t[3];
  memset(t, 0, sizeof t);
  t[0].ptr = (const void*)0x10000; t[0].numel = 1000; t[0].dtype = SDC_F32;
  t[1].ptr = (const void*)0x20002; t[1].numel = 5000000; t[1].dtype = SDC_BF16;
  t[1].flags = SDC_FLAG_SIGNED;
  t[2].ptr = NULL; t[2].numel = 0; t[2].dtype = SDC_F16;
  uint64_t bytes = 0, ws = 0;
  if (sdc_plan_bytes(t, 3, 0, &bytes) != SDC_OK) return 1;
  if (sdc_tensor_ws_bytes(&t[1], 0, &ws) != SDC_OK) return 2;
  sdc_tensor bad = t[0];
  bad.dtype = 99;
  if (sdc_plan_bytes(&bad, 1, 0, &bytes) != SDC_ERR_DTYPE) return 3;
  uint8_t mis[4] = {1, 0, 0, 0}, cul[4], amb[4];
  if (sdc_ring_localize(mis, 4, 1, cul, amb) != SDC_OK) return 4;
  printf("%llu %llu %u %s|%s\n", (unsigned long long)bytes, (unsigned long long)ws,
         sdc_abi_version(), sdc_status_string(SDC_ERR_ALIGN), sdc_status_string(SDC_OK));
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_compiles_as_c99_and_links(tmp_path):
    import silent_corruption_detection_amd as sdc
    src = tmp_path / "prog.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "prog"
    libdir = os.path.dirname(sdc.LIB_PATH)
    # a sanitizer build of the library resolves its runtime from the preloaded
    # one at run time (the program inherits LD_PRELOAD)
    lax = ["-Wl,--allow-shlib-undefined"] if os.environ.get("SDC_LIB_PATH") else []
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    "-L", libdir, "-l:libsdc.so", f"-Wl,-rpath,{libdir}"] + lax, check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    nbytes, ws, version = int(out[0]), int(out[1]), int(out[2])
    assert version == sdc.sdc_abi_version()
    assert " ".join(out[3:]).split("|") == [sdc.sdc_status_string(-3), "ok"]
    assert nbytes > 64 and ws >= 32
