"""The fused call from a C program on MI355X, with no Python or torch in the process.

A C99 program (built with gcc against include/xstage.h, the HIP runtime and libxstage.so)
reads seeded inputs from files, allocates every buffer with the HIP runtime (q, k, v, the P
slabs carved from one allocation, the split workspace sized by xstage_attn_split_ws_size and
zeroed), calls xstage_attn_a2a_fwd on a stream of its own twice (the second call reuses the
workspace) and writes the slabs back.  They must equal the Python binding's result on the
same inputs bit for bit (same library, same plan).  Workload: the FLUX-1024 share (key
splits merged through the workspace)."""

import os
import shutil
import subprocess
import sys

import numpy as np
import pytest
import torch

import attention_ulysses_a2a_amd as xs
from attention_ulysses_a2a_amd import _lib
from synth import make_inputs, workload
from tests.gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

PROGRAM = r"""
#include <stdio.h>
#include <stdlib.h>
#include <hip/hip_runtime_api.h>
#include "xstage.h"

#define CHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
  fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__); return 2; } } while (0)

static int read_file(const char* path, void* dst, size_t n) {
  FILE* f = fopen(path, "rb");
  if (!f) return -1;
  size_t got = fread(dst, 1, n, f);
  fclose(f);
  return got == n ? 0 : -1;
}

int main(int argc, char** argv) {
  if (argc != 11) return 3;
  const int B = atoi(argv[5]), S = atoi(argv[6]), H = atoi(argv[7]), D = atoi(argv[8]), P = atoi(argv[9]);
  const float scale = strtof(argv[10], NULL); /* 9 significant digits: the exact float */
  const size_t n = (size_t)B * S * H * D * 2, slab = n / P;
  void* host = malloc(n);
  void *q, *k, *v, *out, *ws = NULL;
  const char* in[3] = {argv[1], argv[2], argv[3]};
  void** dev[3] = {&q, &k, &v};
  for (int i = 0; i < 3; ++i) {
    if (read_file(in[i], host, n)) return 4;
    CHECK(hipMalloc(dev[i], n));
    CHECK(hipMemcpy(*dev[i], host, n, hipMemcpyHostToDevice));
  }
  CHECK(hipMalloc(&out, n));
  void* slabs[64];
  for (int p = 0; p < P; ++p) slabs[p] = (char*)out + (size_t)p * slab;
  unsigned long long ws_bytes = 0;
  int st = xstage_attn_split_ws_size(B, S, H, D, &ws_bytes);
  if (st != XSTAGE_OK) { fprintf(stderr, "ws size: %s\n", xstage_status_str(st)); return 5; }
  if (ws_bytes) {
    CHECK(hipMalloc(&ws, ws_bytes));
    CHECK(hipMemset(ws, 0, ws_bytes));
  }
  hipStream_t stream;
  CHECK(hipStreamCreate(&stream));
  for (int rep = 0; rep < 2; ++rep) {
    st = xstage_attn_a2a_fwd(q, k, v, slabs, B, S, H, D, P, scale, ws, ws_bytes, (void*)stream);
    if (st != XSTAGE_OK) { fprintf(stderr, "fwd: %s\n", xstage_status_str(st)); return 6; }
  }
  CHECK(hipStreamSynchronize(stream));
  CHECK(hipMemcpy(host, out, n, hipMemcpyDeviceToHost));
  FILE* f = fopen(argv[4], "wb");
  if (!f || fwrite(host, 1, n, f) != n) return 7;
  fclose(f);
  printf("ws_bytes %llu status %s\n", ws_bytes, xstage_status_str(st));
  CHECK(hipStreamDestroy(stream));
  return 0;
}
"""


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="gcc or the HIP headers are not available")
def test_c_program_matches_binding(tmp_path):
    w = workload("flux1024")
    qb, kb, vb = make_inputs(w)
    paths = []
    for name, bits in (("q", qb), ("k", kb), ("v", vb)):
        p = tmp_path / f"{name}.bin"
        np.ascontiguousarray(bits).view(np.uint16).tofile(p)
        paths.append(str(p))
    out_path = tmp_path / "slabs.bin"
    src = tmp_path / "fwd.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "fwd"
    libdir = os.path.dirname(_lib.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
                    "-I", os.path.join(ROOT, "include"), str(src), "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-L", libdir, "-lxstage", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", f"-Wl,-rpath,{libdir}",
                    "-o", str(exe)], check=True)
    log(f"C program: FLUX-1024 share B={w.B} S={w.S} H={w.H} D={w.D} P={w.P}")
    scale = f"{float(np.float32(w.scale)):.9g}"
    assert np.float32(float(scale)) == np.float32(w.scale)
    res = subprocess.run([str(exe), *paths, str(out_path), str(w.B), str(w.S), str(w.H), str(w.D), str(w.P), scale],
                         capture_output=True, text=True, timeout=120)
    log(f"  rc={res.returncode} out={res.stdout.strip()} err={res.stderr.strip()}")
    assert res.returncode == 0
    got = np.fromfile(out_path, dtype=np.uint16).reshape(w.P, w.B, w.S // w.P, w.H, w.D)
    # the binding on the same inputs, with a workspace of the same size
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    slabs = torch.empty((w.P, w.B, w.S // w.P, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    xs.xstage_attn_a2a_fwd(q, k, v, slabs, w.scale, split_ws=xs.split_workspace(w.B, w.S, w.H, w.D, "cuda"))
    torch.cuda.synchronize()
    want = to_host(slabs).reshape(got.shape)
    log(f"  equal to the binding's slabs: {np.array_equal(got, want)}")
    assert np.array_equal(got, want)
