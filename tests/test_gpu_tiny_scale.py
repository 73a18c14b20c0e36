"""Chunks of tiny magnitude through encode and decode, against the oracle,
compared relative to each chunk with no absolute term.

The other parity tests add an absolute floor of 1e-7, which says nothing
about chunks whose values are many orders of magnitude smaller (a momentum
that has decayed for a long time, a frozen parameter).  Here every value of a
128 x 192 tensor is drawn at scale 1, 1e-30 or 1e-36 (the last within a few
binades of float32's subnormal range), and the payload values, the new
momentum and M* are held to the parity floor per unit of chunk norm (NOISE
for the fast DCT, NOISE_DENSE for a caller basis on the matrix cores).
"""
import numpy as np
import pytest
import torch

import parity as PR
from communication_compressed_optimizer_demo_amd import binding as B
from oracle import demo_oracle as O

pytestmark = pytest.mark.gpu

SHAPE = (128, 192)
K = 8
W = 2


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()
    return torch.device("cuda:0")


def chunk_view(T, s):
    return O.split_chunks(np.asarray(T, dtype=np.float64), s).reshape(-1, s * s)


@pytest.mark.parametrize("basis,s", [("dct", 64), ("caller_basis", 64), ("dct", 128)],
                         ids=["dct", "caller_basis", "dct_s128"])
@pytest.mark.parametrize("scale", [1.0, 1e-30, 1e-36])
def test_tiny_magnitude_chunks(dev, basis, s, scale):
    rng = np.random.default_rng(11)
    rand = basis == "caller_basis"
    noise = PR.NOISE_DENSE if rand else PR.NOISE
    shape = SHAPE if s == 64 else (256, 384)
    P0 = P1 = P0d = P1d = None
    if rand:
        P0 = O.orthonormal_rows(rng.standard_normal((64, 64))).astype(np.float32)
        P1 = O.orthonormal_rows(rng.standard_normal((64, 64))).astype(np.float32)
        P0d, P1d = torch.from_numpy(P0).cuda(), torch.from_numpy(P1).cuda()
    codec = B.Codec([shape], K, 0.9, 0.5, chunk=s)
    ne = codec.n_entries
    vals, idx = codec.alloc_payload(W)
    or_v, or_i = [], []
    for wk in range(W):
        G = (rng.standard_normal(shape) * scale).astype(np.float32)
        Mg = torch.zeros(shape, device="cuda")
        codec.encode([torch.from_numpy(G).cuda()], [Mg], vals[wk * ne:(wk + 1) * ne], idx[wk * ne:(wk + 1) * ne],
                     P0d, P1d)
        torch.cuda.synchronize()
        out = O.encode(np.zeros(shape, np.float32), G, beta=0.9, alpha=0.5, k=K, P0=P0, P1=P1, s=s)
        norms = np.linalg.norm(out["Q"].reshape(out["Q"].shape[0], -1), axis=1)
        gi = idx[wk * ne:(wk + 1) * ne].cpu().numpy().view(np.uint16).reshape(out["idx"].shape)
        gv = vals[wk * ne:(wk + 1) * ne].cpu().numpy().reshape(out["values"].shape).astype(np.float64)
        assert np.array_equal(gi, out["idx"]), f"worker {wk}: top-k sets differ at scale {scale:g}"
        err_v = np.max(np.abs(gv - out["values"]), axis=1) / norms
        assert err_v.max() <= noise, f"payload error {err_v.max():.3e} of the chunk norm at scale {scale:g}"
        err_m = np.max(np.abs(chunk_view(Mg.cpu().numpy(), s) - chunk_view(out["M"], s)), axis=1) / norms
        assert err_m.max() <= noise, f"momentum error {err_m.max():.3e} of the chunk norm at scale {scale:g}"
        print(f"  [{basis + ('' if s == 64 else ' s128')} {scale:g}] worker {wk}: payload {err_v.max():.2e}, "
              f"momentum {err_m.max():.2e} of the chunk norm", flush=True)
        or_v.append(out["values"])
        or_i.append(out["idx"])
    # M*: decode with X = 0, phi = identity, eta = 1, lambda = 0 leaves X = -M*
    X = torch.zeros(shape, device="cuda")
    codec.decode_apply([X], W, vals, idx, B.DEMO_PHI_IDENTITY, 1.0, 0.0, B.DEMO_AVG_CONTRIBUTORS, P0d, P1d)
    torch.cuda.synchronize()
    ref = O.decode_apply(np.zeros(shape, np.float32), np.stack(or_v), np.stack(or_i), phi="identity", eta=0.0,
                         lam=0.0, mode="count", P0=P0, P1=P1, s=s)
    qnorm = np.linalg.norm(ref["Qbar"], axis=1)
    err = np.max(np.abs(chunk_view(-X.cpu().numpy(), s) - chunk_view(ref["Mstar"], s)), axis=1) / qnorm
    assert err.max() <= noise, f"M* error {err.max():.3e} of the chunk norm at scale {scale:g}"
    print(f"  [{basis + ('' if s == 64 else ' s128')} {scale:g}] M* {err.max():.2e} of the chunk norm", flush=True)
    codec.close()
