"""The public header is a C header: a C11 program compiles against it, links
the library and calls its host-only entry points (no GPU needed).

gcc, not hipcc, builds the program; the HIP runtime header it includes for
hipStream_t needs the platform macro (-D__HIP_PLATFORM_AMD__) like any plain
C user of HIP's runtime API.  The expected values are counted by hand for the
shapes used: a 1000 x 777 matrix is 16 x 13 = 208 chunks of 64 x 64 and a
300-element vector 5 chunks of 64, k = 8 entries each.
"""
import os
import shutil
import subprocess

import pytest

from communication_compressed_optimizer_demo_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

C_PROGRAM = r"""
#include "demo_codec.h"

#include <stdio.h>

int main(void) {
  demo_shape sh[2];
  sh[0].ndim = 2; sh[0].dims[0] = 1000; sh[0].dims[1] = 777;
  sh[1].ndim = 1; sh[1].dims[0] = 300; sh[1].dims[1] = 0;
  int64_t chunks = 0, entries = 0, begin[3] = {-1, -1, -1};
  if (demo_plan(sh, 2, DEMO_CHUNK, 8, &chunks, &entries, begin) != DEMO_OK) return 1;
  printf("plan %lld %lld %lld %lld %lld\n", (long long)chunks, (long long)entries, (long long)begin[0],
         (long long)begin[1], (long long)begin[2]);
  int64_t vb = 0, ib = 0;
  if (demo_wire_size(DEMO_CHUNK, entries, &vb, &ib) != DEMO_OK) return 2;
  printf("wire %lld %lld\n", (long long)vb, (long long)ib);
  sh[0].ndim = 3;
  demo_status s = demo_plan(sh, 2, DEMO_CHUNK, 8, &chunks, &entries, NULL);
  printf("status %d %s\n", (int)s, demo_last_error());
  demo_codec_cfg cfg = {DEMO_CHUNK, 8, 0.999f, 0.2f, DEMO_MOMENTUM_DAMPED, DEMO_BASIS_DCT, NULL, NULL,
                        DEMO_SUBTRACT_LOCAL};
  s = demo_encode(NULL, 0, sh, NULL, DEMO_F32, NULL, &cfg, NULL, NULL, 0, NULL);
  printf("null-ctx %d\n", (int)s);
  return 0;
}
"""


@pytest.fixture(scope="module")
def program(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(B.LIB_PATH):
        from communication_compressed_optimizer_demo_amd import build
        build.build()
    d = tmp_path_factory.mktemp("c_abi")
    src = d / "main.c"
    src.write_text(C_PROGRAM)
    exe = d / "main"
    libdir = os.path.dirname(B.LIB_PATH)
    cmd = [cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include",
           f"-I{ROCM}/include", str(src), f"-L{libdir}", "-ldemo_codec", f"-Wl,-rpath,{libdir}",
           f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"C program did not build:\n{' '.join(cmd)}\n{r.stderr}"
    return exe


def test_header_compiles_as_c_and_links(program):
    r = subprocess.run([str(program)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = dict(l.split(" ", 1) for l in r.stdout.strip().splitlines())
    # 208 + 5 chunks; 8 entries each; the vector's entries start after the matrix's 1664
    assert lines["plan"] == "213 1704 0 1664 1704"
    # values 2 B per entry; indices 12 bytes per group of 8 entries (213 groups)
    assert lines["wire"] == "3408 2556"
    status, msg = lines["status"].split(" ", 1)
    assert int(status) == 2 and "ndim" in msg  # DEMO_ERR_SHAPE, with a message
    assert lines["null-ctx"] != "0"  # an encode without a context is refused before any device work
