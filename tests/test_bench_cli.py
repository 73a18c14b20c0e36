"""bench.py's argument checks, on the CPU: combinations that are not built, and
more than one GPU, are refused with exit status 2 and a message before any
device is touched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


@pytest.mark.parametrize("args,text", [
    (["--gpus", "2"], "one GPU only"),
    (["--gpus", "8", "--steps", "3"], "one GPU only"),
    (["--chunk", "128", "--basis", "identity"], "chunk 128"),
    (["--chunk", "128", "--download", "signs"], "chunk 128"),
    (["--basis", "random", "--chunk", "128"], "basis random"),
    (["--basis", "random", "--subtraction", "aggregated"], "basis random"),
    (["--phi", "muon", "--download", "signs"], "phi muon"),
    (["--download", "wire", "--subtraction", "aggregated"], "download wire"),
    (["--download", "signs", "--subtraction", "aggregated"], "download signs"),
])
def test_refused_combinations(args, text):
    r = run_bench(*args)
    assert r.returncode == 2, (r.returncode, r.stdout, r.stderr)
    assert text in r.stderr
    assert r.stdout == ""  # no bench line


def test_unknown_workload_is_an_argument_error():
    r = run_bench("--workload", "no_such_set")
    assert r.returncode == 2 and "invalid choice" in r.stderr
