"""Build the codec's shared library in-tree with hipcc for gfx950.

    python -m communication_compressed_optimizer_demo_amd.build

Produces ``communication_compressed_optimizer_demo_amd/libdemo_codec.so``.
Objects go to ``communication_compressed_optimizer_demo_amd/_build/``, and so
does ``valu_issue_probe``, a standalone program that measures the issue cost
of single VALU instruction forms (the basis of the kernels' VALU rooflines).
Packed fp32 VALU instructions are switched off for all device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdemo_codec.so")
ARCH = "gfx950"

SOURCES = ["kernels.hip", "kernels128.hip", "kernels_muon.hip", "codec.cpp"]
PROBE_SRC = "valu_issue_probe.hip"
PROBE = os.path.join(BUILD, "valu_issue_probe")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    path = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the codec is built with ROCm's hipcc for gfx950")
    return path


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every source and link the library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        jobs.append((obj, [cc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]))
    probe = (PROBE, [cc, *COMMON, os.path.join(CSRC, PROBE_SRC), "-o", PROBE])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs) + 1) as ex:
        logs = list(ex.map(lambda j: _run(j[1]), jobs + [probe]))
    tmp = LIB + ".tmp"
    logs.append(_run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[j[0] for j in jobs], "-o", tmp]))
    os.replace(tmp, LIB)
    if verbose:
        for l in logs:
            if l.strip():
                print(l, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
