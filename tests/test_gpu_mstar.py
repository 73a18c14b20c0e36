"""Parity of the decoded momentum M* itself, through the C ABI.

decode_apply with X = 0, eta = 1, lambda = 0 and phi = identity leaves
exactly -M* in X (X - 1 * (M* + 0 * X)), so M* (DeMo summary, §3.4
Server-Side Aggregation and Momentum Reconstruction; Inverse DCT and
Unchunking) is compared with the oracle's element by element under
parity.compare_mstar: |gpu - ref| <= NOISE * ||Q_bar chunk|| + 1e-5 |ref|.

Payloads are drawn directly (demo_inputs.synthetic_payload: distinct
ascending indices per chunk, N(0, 1) values, i.e. unit scale), so the
decode is exercised on its own, over the worker counts, k, chunk edges,
averaging modes and bases the codec supports, the wire format, and the
OLMo-1B-shaped list in the launch configuration bench.py times (sampled).
"""
import numpy as np
import pytest
import torch

import demo_inputs as DI
import parity as PR
from communication_compressed_optimizer_demo_amd import binding as B
from oracle import demo_oracle as O

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()
    return torch.device("cuda:0")


def chunk_table(shapes, k, s):
    """(n_chunks, keff, index range) per tensor."""
    return [(n, keff, s * s if len(sh) == 2 else s) for (n, keff, _), sh in zip(PR.layout(shapes, k, s), shapes)]


def run_case(shapes, k, W, s=64, avg="count", basis="dct", wire=False, seed=0, where=""):
    """Decode W drawn payloads on the GPU into -M* and check every tensor's M* against the oracle."""
    codec = B.Codec(shapes, k, chunk=s, identity=basis == "identity")
    ne = codec.n_entries
    vals, idx = DI.synthetic_payload(chunk_table(shapes, k, s), W, seed=seed, scale=1.0)
    assert vals.size == W * ne
    vd, idd = torch.from_numpy(vals).cuda(), torch.from_numpy(idx.view(np.int16)).cuda()
    P0 = P1 = None
    kw = {}
    if basis == "random":
        w = DI.WORKLOADS["edge_mix"]
        P0, P1 = (O.orthonormal_rows(DI.gaussian_matrix(w, seed, which)).astype(np.float32) for which in (0, 1))
        kw = {"P0": torch.from_numpy(P0).cuda(), "P1": torch.from_numpy(P1).cuda()}
    elif basis == "identity":
        P0 = P1 = np.eye(s)
    avg_c = B.DEMO_AVG_CONTRIBUTORS if avg == "count" else B.DEMO_AVG_WORKERS
    X = [torch.zeros(sh, device="cuda") for sh in shapes]
    if wire:
        wv, wi = codec.alloc_wire(W)
        codec.pack_wire(W, vd, idd, wv, wi)  # positions of 12 bits at s = 64, 14 at s = 128
        codec.decode_apply_wire(X, W, wv, wi, B.DEMO_PHI_IDENTITY, 1.0, 0.0, avg_c, **kw)
    else:
        codec.decode_apply(X, W, vd, idd, B.DEMO_PHI_IDENTITY, 1.0, 0.0, avg_c, **kw)
    torch.cuda.synchronize()
    lay = PR.layout(shapes, k, s)
    worst = 0.0
    for i, sh in enumerate(shapes):
        n, keff, e0 = lay[i]
        v = np.stack([vals[wk * ne + e0:wk * ne + e0 + n * keff].reshape(n, keff) for wk in range(W)])
        ix = np.stack([idx[wk * ne + e0:wk * ne + e0 + n * keff].reshape(n, keff) for wk in range(W)])
        if wire:  # the wire carries the values rounded to bfloat16
            v = O.unpack_wire(*O.pack_wire(v.ravel(), ix.ravel(), s), v.size, s)[0].reshape(v.shape)
        dec = O.decode_apply(np.zeros(sh, np.float32), v, ix, phi="identity", eta=1.0, lam=0.0, mode=avg,
                             P0=P0, P1=P1, s=s)
        worst = max(worst, PR.compare_mstar(dec["Qabs"], dec["Mstar"], -X[i].cpu().numpy(), sh, np.zeros(n, bool),
                                            where=f"{where} tensor {i} {sh}", s=s,
                                            noise=PR.NOISE_DENSE if basis == "random" else PR.NOISE))
    codec.close()
    say(f"  {where}: max |gpu-ref|/||chunk|| = {worst:.3e}")
    return worst


def grid_shapes(s, W, k):
    """Full, padded and vector chunks; fewer chunks where W x keff gets large."""
    if W * min(k, s * s) > 200000:
        return ((s, 2 * s), (s + 5, s - 3), (s + 1,))
    return ((2 * s, 3 * s), (s + 5, 2 * s - 3), (3 * s + 1,), (1, 1))


LOSSLESS = 1 << 20


@pytest.mark.parametrize("s", [64, 128])
@pytest.mark.parametrize("W", [1, 3, 16, 20, 255])
@pytest.mark.parametrize("k", [1, 8, 32, 100, LOSSLESS])
def test_mstar_grid(dev, s, W, k):
    """M* over worker counts (one register batch, several, the 8-bit count limit) and k (fast scatter
    path, keff > 64, lossless), averaged by contributor count."""
    run_case(grid_shapes(s, W, k), k, W, s=s, seed=100 + W + k % 1000, where=f"grid s={s} W={W} k={k}")


@pytest.mark.parametrize("s", [64, 128])
@pytest.mark.parametrize("W,k", [(1, 8), (3, 32), (16, 32), (20, 100), (255, 8)])
def test_mstar_average_by_workers(dev, s, W, k):
    run_case(grid_shapes(s, W, k), k, W, s=s, avg="workers", seed=300 + W + k, where=f"/W s={s} W={W} k={k}")


@pytest.mark.parametrize("basis", ["identity", "random"])
@pytest.mark.parametrize("avg", ["count", "workers"])
@pytest.mark.parametrize("W,k", [(1, 1), (3, 8), (16, 32), (20, 100), (4, LOSSLESS)])
def test_mstar_bases(dev, basis, avg, W, k):
    """The identity basis (M* = Q_bar in place) and a caller basis (random orthonormal P0, P1 on the
    matrix cores)."""
    run_case(grid_shapes(64, W, k), k, W, basis=basis, avg=avg, seed=500 + W + k % 1000,
             where=f"{basis} {avg} W={W} k={k}")


@pytest.mark.parametrize("s", [64, 128])
@pytest.mark.parametrize("avg", ["count", "workers"])
@pytest.mark.parametrize("W,k", [(1, 8), (3, 32), (16, 32), (20, 100), (255, 4)])
def test_mstar_wire(dev, avg, W, k, s):
    """Decoding from the wire format: the oracle decodes the same payload rounded to bfloat16."""
    run_case(grid_shapes(s, W, k), k, W, s=s, wire=True, avg=avg, seed=700 + W + k,
             where=f"wire s={s} {avg} W={W} k={k}")


def test_mstar_full_size_olmo1b(dev):
    """The OLMo-1B-shaped list (96 tensors, 805M parameters) in bench.py's launch configuration (one call,
    k = 32, W = 16), payloads drawn on the device at unit scale; the first, last and a seeded random chunk
    of every tensor are recomputed by the oracle from the same payload slices."""
    w = DI.WORKLOADS["olmo_1b"]
    shapes = [tuple(d) for d in w.shapes]
    W, k = w.workers, w.k
    codec = B.Codec(shapes, k)
    ne = codec.n_entries
    lay = PR.layout(shapes, k)
    vals = torch.empty(W * ne, dtype=torch.float32, device=dev)
    idx = torch.empty(W * ne, dtype=torch.int16, device=dev)
    say(f"[olmo_1b M*] drawing {W} x {ne} payload entries on the device")
    for wk in range(W):
        for t, (sh, (n, keff, e0)) in enumerate(zip(shapes, lay)):
            numel = 4096 if len(sh) == 2 else 64
            gen = torch.Generator(device=dev)
            gen.manual_seed(DI.device_seed(w.config_id, DI.ROLE_PAYLOAD, wk, 0, t))
            sl = slice(wk * ne + e0, wk * ne + e0 + n * keff)
            vals[sl] = torch.randn(n * keff, generator=gen, device=dev)
            for c0 in range(0, n, 16384):
                c1 = min(n, c0 + 16384)
                score = torch.rand((c1 - c0, numel), generator=gen, device=dev)
                ix = torch.topk(score, keff, dim=1).indices.sort(dim=1).values.to(torch.int16)
                idx[wk * ne + e0 + c0 * keff:wk * ne + e0 + c1 * keff] = ix.reshape(-1)
    X = [torch.zeros(sh, device=dev) for sh in shapes]
    say("[olmo_1b M*] decode")
    codec.decode_apply(X, W, vals, idx, B.DEMO_PHI_IDENTITY, 1.0, 0.0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    worst, checked = 0.0, 0
    for t, sh in enumerate(shapes):
        n, keff, e0 = lay[t]
        assert torch.isfinite(X[t]).all()
        for c in sorted({0, n - 1, int(rng.integers(n))}):
            sl = [slice(wk * ne + e0 + c * keff, wk * ne + e0 + (c + 1) * keff) for wk in range(W)]
            v = np.stack([vals[x].cpu().numpy() for x in sl])[:, None, :]
            ix = np.stack([idx[x].cpu().numpy().view(np.uint16) for x in sl])[:, None, :]
            if len(sh) == 1:
                got = X[t][c * 64:(c + 1) * 64].cpu().numpy()
            else:
                g1 = O.chunk_grid(sh)[1]
                cr, cc = divmod(c, g1)
                got = X[t][cr * 64:(cr + 1) * 64, cc * 64:(cc + 1) * 64].cpu().numpy()
            dec = O.decode_apply(np.zeros(got.shape, np.float32), v, ix, phi="identity", eta=1.0, lam=0.0)
            worst = max(worst, PR.compare_mstar(dec["Qabs"], dec["Mstar"], -got, got.shape, np.zeros(1, bool),
                                                where=f"olmo_1b tensor {t} chunk {c}"))
            checked += 1
    say(f"[olmo_1b M*] {checked} chunks checked, max |gpu-ref|/||chunk|| = {worst:.3e}")
    codec.close()
