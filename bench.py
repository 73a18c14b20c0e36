#!/usr/bin/env python3
"""Throughput of the DeMo momentum codec on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload olmo_1b]

One step is the whole per-step hot path for one worker: encode (momentum
update, 64x64 chunking, DCT, per-chunk top-k, payload, momentum subtraction)
of every tensor, then decode/apply of all W workers' payloads (sparse
average, inverse DCT, phi, weight-decayed update) of every tensor.  The
whole tensor list goes into one call per half (one launch each for up to 96
tensors).  The step is captured once into a HIP graph and replayed, as a
training loop would replay its optimizer step; the host clock around the
replays gives the step time.  Per-kernel times come from HIP events on the
launch stream between eager calls of the same step (--no-graph: the step
time from those eager calls too).

Inputs are synthetic and resident in HBM before timing: gradients drawn once
with a seeded device generator, momentum starting at zero, parameters
N(0, 0.02^2); the W-1 other workers' payloads are encoded once, untimed,
from their own seeded gradients.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import demo_inputs as DI  # noqa: E402

METRIC = "params/s for encode+decode/apply per step; achieved HBM GB/s vs MI355X peak"
HBM_PEAK_GBPS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3
BF16_MFMA_PEAK_TFLOPS = 2500.0
# The whole-tile Muon products run every float32-accurate product as six
# bfloat16 part products on the matrix cores.
MUON_PARTS = 6
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "communication_compressed_optimizer_demo_amd", "csrc")
COPY_PROBE_BYTES = 1 << 30


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="olmo_1b", choices=sorted(DI.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--basis", default="dct", choices=("dct", "identity", "random"),
                    help="projection (identity: the ablation that ranks in the parameter domain)")
    ap.add_argument("--subtraction", default="local", choices=("local", "aggregated"),
                    help="momentum subtraction of the worker's own coefficients, or of the averaged ones")
    ap.add_argument("--chunk", type=int, default=64, choices=(64, 128),
                    help="chunk edge s (128: DCT basis)")
    ap.add_argument("--phi", default=None, choices=("muon",),
                    help="override the workload's phi: muon runs decode + Newton-Schulz phi on every whole tensor")
    ap.add_argument("--muon-iters", type=int, default=24, help="Newton-Schulz iterations of the Muon phi")
    ap.add_argument("--download", default="apply", choices=("apply", "signs", "wire"),
                    help="apply: decode/apply in one kernel; signs: the Signum variant's one-bit download, "
                         "decode to packed sign bits then apply them (phi = sign); wire: this worker's payload "
                         "packed into the compact wire format (bfloat16 values, 12- or 14-bit positions), the decode "
                         "reading all W payloads in that format")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every call eagerly instead of replaying a captured HIP graph of the step")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one untimed 1 GiB device-to-device copy (calibrates HBM byte counters)")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="print the HBM rates plain torch streaming kernels reach on this device and exit")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) of a "
                         "--copy-probe run into profiles/traffic_<kernel>_<workload>.json and exit")
    return ap.parse_args()


# ----------------------------------------------------------------------------- CPU oracle leg

def _foreign_payload(args):
    name, worker, tensor = args
    from threadpoolctl import threadpool_limits
    from oracle import demo_oracle as O
    w = DI.WORKLOADS[name]
    with threadpool_limits(1):
        g = DI.gradient(w, worker, 0, tensor)
        import numpy as np
        out = O.encode(np.zeros_like(g), g, beta=w.beta, alpha=w.alpha, k=w.k)
    return out["values"], out["idx"]


CPU_SAMPLE_PARAMS = 100_000_000  # about 10 s of oracle work on a few host cores


def cpu_baseline(w: DI.Workload):
    """The oracle, as it stands, on a bounded leading sample of the workload's tensor list."""
    import concurrent.futures
    import multiprocessing as mp

    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import demo_oracle as O
    sample, n = [], 0
    for i, shp in enumerate(w.shapes):
        if n >= CPU_SAMPLE_PARAMS:
            break
        sample.append(i)
        n += int(np.prod(shp))
    ctx = mp.get_context("fork")
    nproc = max(1, min(16, len(os.sched_getaffinity(0))))
    log(f"cpu baseline: {w.workers - 1} foreign payloads of {len(sample)} tensors ({n} params) on {nproc} processes")
    jobs = [(w.name, wk, t) for t in sample for wk in range(1, w.workers)]
    with concurrent.futures.ProcessPoolExecutor(nproc, mp_context=ctx) as ex:
        res = list(ex.map(_foreign_payload, jobs))
    foreign = {(t, wk): r for (_, wk, t), r in zip(jobs, res)}
    def timed(tensors):
        """Wall and CPU seconds (all threads of the process) of the oracle over `tensors`."""
        dt = cpu = 0.0
        for t in tensors:
            g0 = DI.gradient(w, 0, 0, t)
            x0 = DI.initial_params(w, t)
            t0, c0 = time.perf_counter(), time.process_time()
            out = O.encode(np.zeros_like(g0), g0, beta=w.beta, alpha=w.alpha, k=w.k)
            vals = np.stack([out["values"]] + [foreign[(t, wk)][0] for wk in range(1, w.workers)])
            idx = np.stack([out["idx"]] + [foreign[(t, wk)][1] for wk in range(1, w.workers)])
            O.decode_apply(x0, vals, idx, phi=w.phi, eta=w.eta, lam=w.lam)
            dt += time.perf_counter() - t0
            cpu += time.process_time() - c0
        return dt, cpu

    log("cpu baseline: timing the oracle")
    dt, cpu = timed(sample)
    log(f"cpu baseline: {dt:.2f} s wall, {cpu:.2f} s CPU")
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    # the same oracle on one thread, over the first tensor only (a few seconds)
    with threadpool_limits(1):
        dt1, _ = timed(sample[:1])
    n1 = int(np.prod(w.shapes[sample[0]]))
    log(f"cpu baseline, one thread: {dt1:.2f} s")
    return {
        "value": n / dt,
        "unit": "params/s",
        # cores actually used: CPU seconds over wall seconds of the timed region
        "cores": max(1, round(cpu / dt)),
        "kind": "oracle",
        "sample": (f"the first {len(sample)} tensors of the list ({n} params, "
                   f"{sum(1 for t in sample if len(w.shapes[t]) == 2)} matrices): worker-0 encode + decode/apply "
                   f"over W={w.workers} payloads, tensor by tensor (W-1 foreign payloads precomputed, untimed); "
                   f"{dt:.2f} s wall, {cpu:.2f} s CPU with {threads} BLAS threads available"),
        "cpu": cpu_model(),
        "one_thread": {"value": n1 / dt1, "unit": "params/s",
                       "sample": f"the first tensor ({n1} params), same work, BLAS limited to 1 thread; {dt1:.2f} s"},
    }


def cpu_model() -> str:
    """The host CPU's model name, as /proc/cpuinfo gives it."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ----------------------------------------------------------------------------- GPU leg

# The files the encode and decode kernels are built and launched from, for
# chunk edge 64 and for 128 (separate translation units; the Muon kernels are
# a third).
KERNEL_SOURCES = ("codec.cpp", "common.h", "kernels.hip", "launch.h", "topk.h", "xform.h")
KERNEL_SOURCES_128 = ("codec.cpp", "common.h", "kernels128.hip", "launch.h", "xform.h")


def kernel_source_hash(chunk: int = 64) -> str:
    """sha256 over the encode/decode kernels' sources (counter figures are void once they change)."""
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES_128 if chunk == 128 else KERNEL_SOURCES):
        h.update(f.encode())
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def _traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches this source."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sources_sha256") != kernel_source_hash(128 if "128" in kernel else 64):
        return None
    return rec.get("bytes_per_launch")


def _read_pmc(path: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter of a counter_collection.csv."""
    import csv
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def pmc_summary(w: DI.Workload, fetch_csv: str, write_csv: str):
    """Per-launch HBM traffic of the codec kernels, calibrated on the 1 GiB copy probe."""
    fetch = _read_pmc(fetch_csv, "FETCH_SIZE")
    write = _read_pmc(write_csv, "WRITE_SIZE")
    copy = [k for k in fetch if "copy" in k.lower() or "elementwise_kernel" in k]

    def probe(d):
        # the copy probe is the only dispatch of its kernel that moves ~1 GiB
        vals = [v for k in copy for v in d.get(k, []) if v * 1024 > 0.5 * COPY_PROBE_BYTES]
        assert vals, "no 1 GiB copy dispatch found: run bench.py with --copy-probe"
        return max(vals) * 1024
    f_cal = probe(fetch) / COPY_PROBE_BYTES
    w_cal = probe(write) / COPY_PROBE_BYTES
    recs = {}
    for k in fetch:
        m = re.search(r"(encode|decode)(128|_dense)?_kernel", k)
        if m is None:
            continue
        short = m.group(0)
        src = kernel_source_hash(128 if m.group(2) == "128" else 64)
        fb = [v * 1024 / f_cal for v in fetch[k]]
        wb = [v * 1024 / w_cal for v in write.get(k, [])]
        # the timed launches are the last ones of a kernel (foreign-payload encodes come first)
        rec = {
            "kernel": short, "workload": w.name,
            "fetch_bytes_per_launch": fb[-1], "write_bytes_per_launch": wb[-1] if wb else None,
            "bytes_per_launch": fb[-1] + (wb[-1] if wb else 0.0),
            "calibration": {"copy_bytes": COPY_PROBE_BYTES, "fetch_factor": f_cal, "write_factor": w_cal},
            "dispatches": len(fb), "kernel_sources_sha256": src,
        }
        recs[short] = rec
        with open(os.path.join(PROFILES, f"traffic_{short}_{w.name}.json"), "w") as fo:
            json.dump(rec, fo, indent=1)
    return recs


def hbm_probe(w: DI.Workload):
    """Rates of plain streaming torch kernels over the workload's matrices (the achievable mixes)."""
    import torch
    dev = torch.device("cuda:0")
    mats = [s for s in w.shapes if len(s) == 2]
    A = [torch.ones(s, device=dev) for s in mats]
    Bm = [torch.ones(s, device=dev) for s in mats]
    n = sum(a.numel() for a in A)
    big = torch.ones(1 << 28, device=dev)
    big2 = torch.empty_like(big)

    def med(fn, reps=7):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]))
        return sorted(ts)[reps // 2]
    out = {}
    for name, fn, nbytes in (
            ("read 2, write 1 (lerp over the matrices)", lambda: [b.lerp_(a, 0.001) for a, b in zip(A, Bm)], 12 * n),
            ("read 1, write 1 (scale over the matrices)", lambda: [b.mul_(0.999) for b in Bm], 8 * n),
            ("read 1, write 1 (1 GiB device copy)", lambda: big2.copy_(big), 2 << 30),
            ("write only (1 GiB fill)", lambda: big.fill_(1.0), 1 << 30)):
        ms = med(fn)
        out[name] = {"ms": round(ms, 4), "bytes": int(nbytes), "GBps": round(nbytes / ms / 1e6, 1)}
    return out


def muon_flops(shapes, iters: int) -> int:
    """Matrix-core flops of one Muon decode: Gram, 3 n^3 products per iteration, final product."""
    total = 0
    for s in shapes:
        if len(s) != 2:
            continue
        r, c = s
        n, k = min(r, c), max(r, c)
        total += 2 * n * n * k + iters * 3 * 2 * n ** 3 + 2 * r * c * n
    return total


def muon_whole_tiles(shapes) -> bool:
    """Every matrix's products take the whole-tile (bfloat16-split) GEMM: both dims multiples of 128."""
    return all(len(s) != 2 or (s[0] % 128 == 0 and s[1] % 128 == 0) for s in shapes)


def gpu_bench(w: DI.Workload, steps: int, warmup: int, copy_probe: bool = False, basis: str = "dct",
              subtraction: str = "local", download: str = "apply", chunk: int = 64, muon_iters: int = 0,
              graph: bool = True):
    import torch

    from communication_compressed_optimizer_demo_amd import binding as B
    if not os.path.exists(B.LIB_PATH):
        from communication_compressed_optimizer_demo_amd import build
        build.build()
    B.load_library()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    W = w.workers
    # the whole list in one call per half, as a training step would pass it
    shapes = [tuple(s) for s in w.shapes]
    aggregated = subtraction == "aggregated"
    codec = B.Codec(shapes, w.k, w.beta, w.alpha, identity=basis == "identity", aggregated=aggregated, chunk=chunk)
    launches = -(-len(shapes) // B.DEMO_MAX_TENSORS_PER_LAUNCH)
    basis_kw = {}
    if basis == "random":
        # the caller's orthonormal projection: rows of the Q factor of the step's seeded N(0, 1) draws
        # (any orthonormal basis is a valid one; the same two matrices serve every worker)
        import numpy as np
        P = [np.linalg.qr(DI.gaussian_matrix(w, 0, which).T)[0].T.astype(np.float32) for which in (0, 1)]
        basis_kw = {"P0": torch.from_numpy(P[0].copy()).to(dev), "P1": torch.from_numpy(P[1].copy()).to(dev)}
    G = [DI.device_gradient(w, 0, 0, i, dev) for i in range(len(shapes))]
    M = [torch.zeros(s, device=dev) for s in shapes]
    X = [DI.device_initial_params(w, i, dev) for i in range(len(shapes))]
    vals, pidx = codec.alloc_payload(W)
    ne = codec.n_entries
    log(f"{len(shapes)} tensors ({launches} launch(es) per call): encoding {W - 1} foreign payloads")
    scratch_m = [torch.zeros(s, device=dev) for s in shapes]
    for wk in range(1, W):  # the other workers' payloads, untimed
        for t in scratch_m:
            t.zero_()
        gf = [DI.device_gradient(w, wk, 0, i, dev) for i in range(len(shapes))]
        codec.encode(gf, scratch_m, vals[wk * ne:(wk + 1) * ne], pidx[wk * ne:(wk + 1) * ne], **basis_kw)
        del gf
    del scratch_m
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if copy_probe:
        # a plain device copy of known size, for scaling the HBM byte counters
        src = torch.ones(COPY_PROBE_BYTES // 4, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
        log(f"copy probe: {COPY_PROBE_BYTES} bytes copied")

    phi = B.DEMO_PHI_SIGN if w.phi == "sign" else B.DEMO_PHI_IDENTITY
    stream = torch.cuda.current_stream()
    signs = codec.alloc_signs() if download == "signs" else None
    if download == "wire":  # the other workers' payloads arrive packed; this worker packs its own in the step
        wv, wi = codec.alloc_wire(W)
        wb = B.demo_wire_size(ne, chunk)[1]
        codec.pack_wire(W, vals, pidx, wv, wi)
        torch.cuda.synchronize()
    muon_ws = codec.alloc_muon_workspace() if muon_iters else None
    # Muon's eps does not change the work (a fixed iteration count); 1e-12 sits below the
    # Gram eigenvalues of these M*
    muon_eps = 1e-12

    # the step's calls in order, each taking the stream to launch on
    calls = [("encode", lambda st: codec.encode(G, M, vals[:ne], pidx[:ne], stream=st, **basis_kw))]
    if download == "signs":  # server: packed sign(M*); worker: apply the bits
        calls.append(("decode", lambda st: codec.decode_signs(W, vals, pidx, signs, stream=st)))
        calls.append(("apply", lambda st: codec.apply_signs(X, signs, w.eta, w.lam, stream=st)))
    elif download == "wire":
        calls.append(("pack", lambda st: codec.pack_wire(1, vals[:ne], pidx[:ne], wv[:ne], wi[:wb], stream=st)))
        calls.append(("decode", lambda st: codec.decode_apply_wire(X, W, wv, wi, phi, w.eta, w.lam, stream=st)))
    elif muon_iters:
        calls.append(("decode", lambda st: codec.decode_apply_muon(X, W, vals, pidx, muon_ws, w.eta, w.lam, muon_eps,
                                                                   muon_iters, stream=st)))
    elif aggregated:  # this worker's parameters and momentum, one pass
        calls.append(("decode", lambda st: codec.decode_apply_subtract(X, M, W, vals, pidx, phi, w.eta, w.lam,
                                                                       stream=st)))
    else:
        calls.append(("decode", lambda st: codec.decode_apply(X, W, vals, pidx, phi, w.eta, w.lam, stream=st,
                                                              **basis_kw)))

    def one_step(ev):
        for j, (_, fn) in enumerate(calls):
            if ev:
                ev[j].record(stream)
            fn(stream)
        if ev:
            ev[len(calls)].record(stream)

    log(f"warmup {warmup} steps")
    for _ in range(warmup):
        one_step(None)
    torch.cuda.synchronize()
    # per-kernel times: HIP events on the launch stream between eager calls
    log(f"timing {steps} eager steps")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        one_step(events[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per = {name: sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / steps for j, (name, _) in enumerate(calls)}
    if graph:
        # the step time: replays of the whole step captured once as a HIP graph
        g_step = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_step):
            for _, fn in calls:
                fn(torch.cuda.current_stream())
        for _ in range(2):
            g_step.replay()
        torch.cuda.synchronize()
        log(f"timing {steps} graph replays of the step")
        t0 = time.perf_counter()
        for _ in range(steps):
            g_step.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    gbytes = 2 if w.grad_bf16 else 4
    numel = w.n_params
    kern = {}
    algo = {"encode": numel * (gbytes + 8) + ne * 6}
    if download == "signs":
        algo["decode"] = W * ne * 6 + codec.n_sign_words * 8  # W payloads read, packed signs written
        algo["apply"] = numel * 8 + codec.n_sign_words * 8    # X read and written, packed signs read
    elif download == "wire":
        algo["pack"] = ne * 6 + ne * 2 + wb                   # own payload read, wire values and indices written
        algo["decode"] = numel * 8 + W * (ne * 2 + wb)        # X read and written, W wire payloads read
    else:
        algo["decode"] = numel * (16 if aggregated else 8) + W * ne * 6  # X (and M) read and written, W payloads
    for name, b in algo.items():
        ms = per[name]
        kern[name] = {"ms": round(ms, 4), "launches": launches, "algorithmic_bytes": int(b),
                      "GBps": round(b / ms / 1e6, 1), "params": numel}
    if muon_iters:
        fl = muon_flops(shapes, muon_iters)
        kern["decode"]["mfma_flops"] = fl  # float32-accurate product flops
        kern["decode"]["TFLOPs"] = round(fl / per["decode"] / 1e9, 2)
        if muon_whole_tiles(shapes):
            kern["decode"]["bf16_mfma_flops"] = MUON_PARTS * fl
            kern["decode"]["bf16_TFLOPs"] = round(MUON_PARTS * fl / per["decode"] / 1e9, 1)
    dom = max(kern, key=lambda n: kern[n]["ms"])
    dk = kern[dom]
    achieved = dk["algorithmic_bytes"] / dk["ms"] / 1e6
    total_bytes = sum(k["algorithmic_bytes"] for k in kern.values())
    ms_per_step = elapsed / steps * 1e3
    if muon_iters and "bf16_TFLOPs" in dk:  # a chain of bfloat16 part products on the matrix cores
        roof = {"bound": "mfma", "kernel": "decode", "achieved": dk["bf16_TFLOPs"], "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(dk["bf16_TFLOPs"] / BF16_MFMA_PEAK_TFLOPS, 4)}
    elif muon_iters:  # ragged shapes: float32 matrix-core products
        roof = {"bound": "mfma", "kernel": "decode", "achieved": dk["TFLOPs"], "peak": FP32_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(dk["TFLOPs"] / FP32_MFMA_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4)}
    return {
        "ms_per_step": ms_per_step,
        "value": w.n_params / (ms_per_step / 1e3),
        "step_GBps": total_bytes / (ms_per_step / 1e3) / 1e9,
        "kernels": kern,
        "roofline": {
            **roof,
            "traffic": (_traffic(f"{dom}{'128' if chunk == 128 else ''}_kernel", w.name)
                        if launches == 1 and basis == "dct" and subtraction == "local" and download == "apply"
                        and not muon_iters else None),
        },
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): it measures the codec on "
              "one GPU's share; collectives across GPUs are not part of the library.", file=sys.stderr)
        sys.exit(2)
    w = DI.WORKLOADS[args.workload]
    if args.hbm_probe:
        print(json.dumps({"device": "cuda:0", "workload": w.name, "rates": hbm_probe(w)}))
        return
    if args.pmc_summary:
        for name, rec in pmc_summary(w, *args.pmc_summary).items():
            print(json.dumps(rec))
        return
    if args.basis == "random" and (args.chunk != 64 or args.download != "apply" or args.subtraction != "local"
                                   or args.phi):
        print("--basis random runs with chunk 64, the apply download and the local subtraction", file=sys.stderr)
        sys.exit(2)
    if args.chunk == 128 and args.basis != "dct":
        print("--chunk 128 is built for the DCT basis", file=sys.stderr)
        sys.exit(2)
    if args.phi == "muon":
        if args.download != "apply" or args.subtraction != "local" or args.chunk != 64:
            print("--phi muon runs with the apply download, the local subtraction and chunk 64", file=sys.stderr)
            sys.exit(2)
        w = w.replace(phi="muon")
    if args.download == "wire" and args.subtraction != "local":
        print("--download wire runs with the local subtraction", file=sys.stderr)
        sys.exit(2)
    if args.download == "signs":
        if args.subtraction != "local":
            print("--download signs pairs with the local subtraction only", file=sys.stderr)
            sys.exit(2)
        w = w.replace(phi="sign")  # the one-bit download exists for the Signum variant only
    cpu = None if args.no_cpu_baseline or args.phi else cpu_baseline(w)
    g = gpu_bench(w, args.steps, args.warmup, args.copy_probe, args.basis, args.subtraction, args.download,
                  args.chunk, args.muon_iters if args.phi == "muon" else 0, graph=not args.no_graph)
    line = {
        "metric": METRIC,
        "value": g["value"],
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": g["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": ("synthetic: gradients N(0, {:g}) drawn once on the device (seeded), M0 = 0, X0 ~ N(0, {:g}^2), "
                 "W-1 foreign payloads encoded untimed from their own seeded gradients").format(w.grad_std,
                                                                                                w.param_std),
        "config": {
            "workload": w.name,
            "tensors": len(w.shapes),
            "params": w.n_params,
            "chunk": args.chunk,
            "k": w.k,
            "workers": w.workers,
            "alpha": w.alpha,
            "beta": w.beta,
            "phi": w.phi,
            "grad_dtype": "bf16" if w.grad_bf16 else "fp32",
            "basis": args.basis,
            "subtraction": args.subtraction,
            "download": args.download,
            "launch": "eager" if args.no_graph else "hip_graph",
            **({"muon_iters": args.muon_iters} if args.phi == "muon" else {}),
        },
        "step_GBps": round(g["step_GBps"], 1),
        "kernels": g["kernels"],
        "roofline": g["roofline"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
