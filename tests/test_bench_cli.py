"""bench.py's host logic, on the CPU: combinations that are not built, and
more than one GPU, are refused with exit status 2 and a message before any
device is touched; counter summaries are calibrated, keyed and invalidated
as the roofline's traffic figure assumes."""
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
    (["--chunk", "128", "--phi", "muon"], "phi muon"),
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


# --------------------------------------------------------------------------- counter summaries (host logic)

def _write_pmc_csv(path, counter, rows):
    import csv
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_pmc_summary_calibrates_and_keys_records_by_source(tmp_path, monkeypatch):
    """Synthetic counter files: the copy probe fixes the scale, the last dispatch of each codec kernel is
    the timed one, chunk-64 and chunk-128 records carry the hashes of their own sources, and a record
    stops counting once its hash no longer matches."""
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    gib_kib = (1 << 30) // 1024
    fetch = [("__amd_rocclr_copyBuffer", 524308),  # FETCH_SIZE reads about half the copied bytes
             ("void demo::encode_kernel<false>(...)", 100.0), ("void demo::encode_kernel<false>(...)", 50.0),
             ("void demo::(anonymous namespace)::encode128_kernel<false>(...)", 30.0),
             ("void demo::(anonymous namespace)::decode128_kernel<1>(...)", 20.0),
             ("void demo::gemm_tile_kernel<...>(...)", 999.0)]
    write = [("__amd_rocclr_copyBuffer", gib_kib), ("void demo::encode_kernel<false>(...)", 7.0),
             ("void demo::encode_kernel<false>(...)", 8.0),
             ("void demo::(anonymous namespace)::encode128_kernel<false>(...)", 9.0),
             ("void demo::(anonymous namespace)::decode128_kernel<1>(...)", 10.0)]
    _write_pmc_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _write_pmc_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    recs = bench.pmc_summary(bench.DI.WORKLOADS["olmo_1b"], str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    assert set(recs) == {"encode_kernel", "encode128_kernel", "decode128_kernel"}
    enc = recs["encode_kernel"]
    assert enc["dispatches"] == 2
    f_cal = 524308 / gib_kib
    assert enc["calibration"]["fetch_factor"] == pytest.approx(f_cal)
    assert enc["fetch_bytes_per_launch"] == pytest.approx(50.0 * 1024 / f_cal)  # the last dispatch, scaled
    assert enc["write_bytes_per_launch"] == pytest.approx(8.0 * 1024)
    assert enc["kernel_sources_sha256"] == bench.kernel_source_hash(64)
    assert recs["decode128_kernel"]["kernel_sources_sha256"] == bench.kernel_source_hash(128)
    assert bench.kernel_source_hash(64) != bench.kernel_source_hash(128)
    for name in recs:
        assert (tmp_path / f"traffic_{name}_olmo_1b.json").exists()
    assert bench._traffic("decode128_kernel", "olmo_1b") == pytest.approx(20.0 * 1024 / f_cal + 10.0 * 1024)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda chunk=64: "changed")
    assert bench._traffic("decode128_kernel", "olmo_1b") is None
