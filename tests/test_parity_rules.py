"""The parity rules themselves, on the CPU: each comparison in parity.py must accept the oracle's own
float32 results and reject a result that is off by a factor (1 + 1e-4), ten times the stated relative
tolerance.  A planted mistake lives on the CPU side only; no GPU is involved."""
import numpy as np
import pytest

import demo_inputs as DI
import parity as PR
from oracle import demo_oracle as O


def _payload(shapes, k, W, seed, s=64):
    lay = [(n, keff, s * s if len(sh) == 2 else s) for (n, keff, _), sh in zip(PR.layout(shapes, k, s), shapes)]
    vals, idx = DI.synthetic_payload(lay, W, seed=seed, scale=1.0)
    ne = sum(n * keff for n, keff, _ in lay)
    out = []
    e = 0
    for n, keff, _ in lay:
        v = np.stack([vals[w * ne + e:w * ne + e + n * keff].reshape(n, keff) for w in range(W)])
        ix = np.stack([idx[w * ne + e:w * ne + e + n * keff].reshape(n, keff) for w in range(W)])
        out.append((v, ix))
        e += n * keff
    return out


@pytest.mark.parametrize("s", [64, 128])
@pytest.mark.parametrize("mode", ["count", "workers"])
def test_compare_mstar_rejects_a_scaled_mstar(s, mode):
    shapes = [(2 * s, s + 7), (s + 3,)]
    for (v, ix), sh in zip(_payload(shapes, 16, 3, seed=5, s=s), shapes):
        dec = O.decode_apply(np.zeros(sh, np.float32), v, ix, phi="identity", eta=1.0, lam=0.0, mode=mode, s=s)
        n = dec["Qbar"].shape[0]
        ok = np.zeros(n, bool)
        PR.compare_mstar(dec["Qabs"], dec["Mstar"], dec["Mstar"].astype(np.float32), sh, ok, s=s)
        with pytest.raises(AssertionError):
            PR.compare_mstar(dec["Qabs"], dec["Mstar"], (dec["Mstar"] * (1 + 1e-4)).astype(np.float32), sh, ok, s=s)
        # one element pushed by 10x the relative tolerance, at workload scale (1e-6): also rejected
        tiny = dec["Mstar"] * 1e-6
        bad = tiny.copy()
        j = np.unravel_index(np.argmax(np.abs(bad)), bad.shape)
        bad[j] *= 1 + 1e-4
        PR.compare_mstar(dec["Qabs"] * 1e-6, tiny, tiny.astype(np.float32), sh, ok, s=s)
        with pytest.raises(AssertionError):
            PR.compare_mstar(dec["Qabs"] * 1e-6, tiny, bad.astype(np.float32), sh, ok, s=s)
        # a chunk marked diverged is not compared
        PR.compare_mstar(dec["Qabs"], dec["Mstar"], (dec["Mstar"] * 2).astype(np.float32), sh, np.ones(n, bool), s=s)


@pytest.mark.parametrize("scale", [1.0, 1e-6])
def test_compare_encode_rejects_scaled_momentum_and_values(scale):
    rng = np.random.default_rng(3)
    sh = (130, 70)
    M = (rng.standard_normal(sh) * scale).astype(np.float32)
    G = (rng.standard_normal(sh) * scale).astype(np.float32)
    out = O.encode(M, G, beta=0.9, alpha=0.3, k=8)
    n = out["Q"].shape[0]
    P = O.dct_basis()
    args = dict(shape=sh, keff=8, alpha=0.3, P0=P, P1=P, diverged=np.zeros(n, bool))
    PR.compare_encode(out, gpu_M=out["M"], gpu_vals=out["values"], gpu_idx=out["idx"], report=PR.EncodeReport(), **args)
    with pytest.raises(AssertionError):
        PR.compare_encode(out, gpu_M=(out["M"] * np.float32(1 + 1e-4)), gpu_vals=out["values"], gpu_idx=out["idx"],
                          report=PR.EncodeReport(), **args)
    with pytest.raises(AssertionError):
        PR.compare_encode(out, gpu_M=out["M"], gpu_vals=out["values"] * np.float32(1 + 1e-4), gpu_idx=out["idx"],
                          report=PR.EncodeReport(), **args)
    # the subtraction left out of one chunk (momentum = M' there): rejected
    mp = O.merge_chunks(out["Mp_chunks"], sh).astype(np.float32)
    with pytest.raises(AssertionError):
        PR.compare_encode(out, gpu_M=mp, gpu_vals=out["values"], gpu_idx=out["idx"], report=PR.EncodeReport(), **args)


def test_compare_momentum_rejects_a_scaled_result():
    rng = np.random.default_rng(4)
    sh = (100, 64)
    M = rng.standard_normal(sh).astype(np.float32)
    Ms = rng.standard_normal(sh)
    ref = O.subtract_aggregated(M, Ms, 0.5)
    PR.compare_momentum(ref, ref, sh, np.zeros(2, bool), scale=0.5 * Ms)
    with pytest.raises(AssertionError):
        PR.compare_momentum(ref, ref * np.float32(1 + 1e-4), sh, np.zeros(2, bool), scale=0.5 * Ms)


def test_compare_decode_rejects_a_flipped_sign():
    rng = np.random.default_rng(5)
    sh = (64, 64)
    X = rng.standard_normal(sh).astype(np.float32) * np.float32(0.02)
    (v, ix), = _payload([sh], 8, 2, seed=9)
    dec = O.decode_apply(X, v, ix, phi="sign", eta=1e-3, lam=0.01)
    PR.compare_decode(dec, sh, "sign", 1e-3, dec["X"], np.zeros(1, bool), None)
    j = np.unravel_index(np.argmax(np.abs(dec["Mstar"])), sh)
    bad = dec["X"].copy()
    bad[j] += np.float32(2e-3) * np.sign(dec["Mstar"][j])  # the update taken with the opposite sign
    with pytest.raises(AssertionError):
        PR.compare_decode(dec, sh, "sign", 1e-3, bad, np.zeros(1, bool), None)


def test_tie_window_uses_the_floor():
    q = np.zeros(4096)
    q[:10] = np.arange(10, 0, -1)        # 10, 9, ..., 1
    q[10] = 1.0 + 5e-6                   # within 1e-5 of the 10th largest: a near tie
    forced, window, quota = PR.topk_window(q, 10)
    assert set(window.tolist()) == {9, 10} and quota == 1 and len(forced) == 9
    q[10] = 1.0 + 1e-4                   # clearly larger: it is the 10th, and 1.0 is out of the window
    forced, window, quota = PR.topk_window(q, 10)
    assert set(window.tolist()) == {10} and quota == 1 and len(forced) == 9
