"""phi = Muon through the C ABI against the oracle's M (M^T M + eps I)^(-1/2).

Every worker encodes its own seeded gradients on the GPU and in the oracle
(the oracle never sees GPU output); the W payloads are then decoded with the
Muon phi on both sides.  phi couples every element of a tensor, so a tensor
any of whose chunks took a legitimately different top-k set (near ties, see
parity.py) is not compared; the tests assert that this stays rare.

Tolerance: the kernel runs the coupled Newton-Schulz iteration at float32
accuracy on the matrix cores (float32 operands split exactly into three
bfloat16 parts, six part products accumulated in float32).  The scalar form of the iteration, z <- z (3 - l z^2) / 2
for an eigenvalue l of the normalised Gram, grows z by 1.5 per step until
l z^2 nears 1 and then converges quadratically: about log_1.5(l^-1/2) + 5
steps.  With eps at 1e-3 of the largest mean Gram eigenvalue in the list,
l >= about 1e-3 / (n * dynamic range) and 24 steps converge for these
shapes; the float32 products then leave phi within 1e-4 * max|phi| of the
float64 eigendecomposition (measured 1e-7 to 3e-5).  That bound is
multiplied by eta for the parameters.
"""
import numpy as np
import pytest
import torch

import demo_inputs as DI
import parity as PR
from communication_compressed_optimizer_demo_amd import binding as B
from oracle import demo_oracle as O

pytestmark = pytest.mark.gpu

PHI_TOL = 1e-4


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()
    return torch.device("cuda:0")


def run_case(name, shapes, k, W, eta, lam, iters=24, eps_rel=1e-3, avg="count"):
    w = DI.WORKLOADS["tiny_256"].replace(name=name, shapes=tuple(shapes), k=k, workers=W, eta=eta, lam=lam)
    codec = B.Codec(shapes, k, w.beta, w.alpha)
    lay = PR.layout(shapes, k)
    ne = codec.n_entries
    vals, idx = codec.alloc_payload(W)
    or_v = [[] for _ in shapes]
    or_i = [[] for _ in shapes]
    diverged = [False] * len(shapes)
    for wk in range(W):
        G = [DI.gradient(w, wk, 0, i) for i in range(len(shapes))]
        M = [torch.zeros(s, device="cuda") for s in shapes]
        codec.encode([torch.from_numpy(g).cuda() for g in G], M, vals[wk * ne:(wk + 1) * ne],
                     idx[wk * ne:(wk + 1) * ne])
        torch.cuda.synchronize()
        gi = idx[wk * ne:(wk + 1) * ne].cpu().numpy().view(np.uint16)
        for i, s in enumerate(shapes):
            n, keff, e0 = lay[i]
            out = O.encode(np.zeros(s, np.float32), G[i], beta=w.beta, alpha=w.alpha, k=k)
            or_v[i].append(out["values"])
            or_i[i].append(out["idx"])
            diverged[i] |= not np.array_equal(gi[e0:e0 + n * keff].reshape(n, keff), out["idx"])
    # eps: 1e-3 of the largest mean Gram eigenvalue over the list (from the oracle's M*); one eps
    # serves the whole list, and tensors of smaller scale are then dominated by it
    X0 = [DI.initial_params(w, i) for i in range(len(shapes))]
    mstar = [O.decode_apply(X0[i], np.stack(or_v[i]), np.stack(or_i[i]), phi="identity", eta=0.0, lam=0.0,
                            mode=avg)["Mstar"] for i in range(len(shapes))]
    eps = eps_rel * max(float(np.sum(m * m)) / (min(m.shape) if m.ndim == 2 else 1) for m in mstar)
    X = [torch.from_numpy(x.copy()).cuda() for x in X0]
    ws = codec.alloc_muon_workspace()
    say(f"  [{name}] decode with Muon phi, eps {eps:.3e}, {iters} iterations")
    codec.decode_apply_muon(X, W, vals, idx, ws, eta=eta, lam=lam, eps=eps, iters=iters,
                            avg=B.DEMO_AVG_CONTRIBUTORS if avg == "count" else B.DEMO_AVG_WORKERS)
    torch.cuda.synchronize()
    compared = 0
    for i, s in enumerate(shapes):
        if diverged[i]:
            say(f"  [{name}] tensor {i} {s}: top-k set differs at a near tie, not compared")
            continue
        phi = O.phi_muon(mstar[i], eps)
        ref = X0[i].astype(np.float64) - eta * (phi + lam * X0[i].astype(np.float64))
        got = X[i].cpu().numpy().astype(np.float64)
        tol = PR.ATOL + PR.RTOL * np.abs(ref) + eta * PHI_TOL * np.abs(phi).max()
        err = np.abs(got - ref)
        assert np.all(err <= tol), (f"{name} tensor {i} {s}: max error {err.max():.3e} "
                                    f"(phi error {err.max() / eta / np.abs(phi).max():.3e} of max|phi|)")
        say(f"  [{name}] tensor {i} {s}: phi error {err.max() / eta / np.abs(phi).max():.2e} of max|phi|")
        compared += 1
    assert compared >= len(shapes) - 1
    codec.close()


SHAPES = [(70, 90), (90, 70), (64, 64), (130, 200), (1, 7), (7, 1), (100,), (1,)]


def test_muon_lossless_phi_exposed(dev):
    """k = 4096 (M* = mean M'), eta = 1, lambda = 0: the update is X - phi, phi seen directly."""
    run_case("muon_lossless", SHAPES, 4096, 2, 1.0, 0.0)


@pytest.mark.parametrize("k,W,avg", [(64, 3, "count"), (16, 4, "workers")])
def test_muon_sparse_payloads(dev, k, W, avg):
    run_case(f"muon_k{k}", SHAPES, k, W, 1.0, 0.0, avg=avg)


def test_muon_weight_decay_and_small_eta(dev):
    run_case("muon_decay", [(256, 192), (300,)], 32, 3, 1e-2, 0.1)


def test_muon_whole_tile_products(dev):
    """Matrices large enough for 128 x 128 workgroup tiles: wide (Gram M M^T, then Z M) and tall (Gram M^T M,
    then M Z) take the whole-tile GEMM for every product; 2048 x 2100 sends the Gram and the last product
    (K or N not a multiple of the tile) through the bounds-checked GEMM while its iterations stay whole-tile."""
    run_case("muon_whole_tiles", [(2048, 2304), (2304, 2048), (2048, 2100)], 32, 2, 1.0, 0.0)


def test_muon_batched_small_tiles(dev):
    """Three matrices with n = 256 share each Newton-Schulz launch; too few 128 x 128 tiles for the GPU, so the
    batch runs the whole-tile GEMM with 64 x 64 tiles (grid z = matrix); a vector sits between them in the list."""
    run_case("muon_batch_256", [(256, 320), (300,), (320, 256), (256, 256)], 16, 3, 1.0, 0.0)
