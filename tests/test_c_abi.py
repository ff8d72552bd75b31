"""The C ABI from C: a C99 program includes include/xstage.h, links libxstage.so and calls the
host-only entry points (workspace sizes, the Burst-Gap formula and pacing chooser, status
names, an argument reject).  Nothing here launches a kernel, so it runs without a GPU; it
checks that the header is valid C and that the library is usable without Python."""

import os
import shutil
import subprocess

import pytest

from attention_ulysses_a2a_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include "xstage.h"
int main(void) {
  unsigned long long b = 0;
  double t = 0.0;
  int st = xstage_attn_split_ws_size(1, 4608, 3, 128, &b);
  printf("split_ws_size %d %llu\n", st, b);
  st = xstage_attn_nsplit_ws_size(1, 4608, 3, 128, 4, &b);
  printf("nsplit_ws_size %d %llu\n", st, b);
  printf("t_iss %.17g\n", xstage_bg_t_iss(1e-6, 2e-6, 64.0 * 1048576.0, 5.64e12));
  int c = xstage_bg_pacing_chunks(8388608.0, 600e-6, 86e-9, 256 * 131e9, 5.64e12, 6.5 * 1048576.0, 8, &t);
  printf("pacing %d %.17g\n", c, t);
  printf("status %s %s\n", xstage_status_str(0), xstage_status_str(1));
  printf("reject %d\n", xstage_attn_a2a_fwd(0, 0, 0, 0, 1, 256, 2, 64, 2, 0.125f, 0, 0, 0));
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_calls_the_library(tmp_path):
    if not os.path.exists(_lib.LIB_PATH):
        from attention_ulysses_a2a_amd.build import build

        build()
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(_lib.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-L", libdir, "-lxstage", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    out = dict(line.split(" ", 1) for line in subprocess.run([str(exe)], check=True, capture_output=True,
                                                              text=True).stdout.strip().splitlines())
    # FLUX-1024 share: 108 tiles x 4 key splits, records of 4 waves x 9 chunks x 64 lanes x 16 B
    assert out["split_ws_size"] == f"0 {16384 + 108 * 4 * 4 * 9 * 64 * 16}"
    assert out["nsplit_ws_size"] == f"0 {16384 + 108 * 4 * 4 * 9 * 64 * 16}"
    # max(T0, V/R - G) with V = 64 MiB, R = 5.64 TB/s, G = 1 us, T0 = 2 us
    assert abs(float(out["t_iss"]) - (64 * 2 ** 20 / 5.64e12 - 1e-6)) < 1e-15
    c, tv = out["pacing"].split()
    assert c == "1" and abs(float(tv) - (86e-9 + 8388608.0 / (256 * 131e9))) < 1e-15
    assert out["status"] == "XSTAGE_OK XSTAGE_ERR_INVALID"
    assert out["reject"] == str(_lib.XSTAGE_ERR_INVALID)
