"""Comparison rules between the HIP path and the CPU oracle.

Floating point, elementwise, on the encode's outputs (payload values, new
momentum) and on the decode's M*:
    |gpu - ref| <= NOISE * ||chunk||_F + RTOL * |ref|
with RTOL = 1e-5, the stated float32 relative tolerance, and ||chunk||_F the
Frobenius norm, over the whole (padded) chunk, of the magnitudes the value
is computed from: |beta M| + |c G| (the momentum update's two terms) for
the encode, the average of the payload values' magnitudes for M*.  A
float32 evaluation rounds at the scale of its operands, and an orthonormal
transform spreads that over the chunk, so the error scales with this norm,
not with the element (nor with a result that cancelled): near-zero
elements need an absolute floor, and NOISE sets it, scale-free, at a small
multiple of what the kernels measure (see NOISE below).  The floor is far
below the stated 1e-7 absolute tolerance at the workloads' data scales
(chunk norms of 1e-4..1e-3), so this rule is stricter than that tolerance
there, and at unit scale the relative term decides.

Parameters X after decode/apply keep the stated pair:
    |gpu - ref| <= ATOL + RTOL * |ref|,  ATOL = 1e-7;
their M* is checked on its own (compare_mstar).

Top-k indices must equal the oracle's exactly, except at near ties: with K
the oracle's keff-th largest magnitude, coefficients with |Q| > K + tol are
forced, those within tol of K form the tie window, tol = RTOL * K +
NOISE * ||Q||_F.  A GPU set that holds every forced index and fills the
rest from the window is valid; its residual is then compared with the
oracle's residual for that same set, taken from the oracle-side list of all
valid sets.  The chunk is marked diverged and left out of later steps
(its state legitimately differs from then on).

Signum: elements with |M*_ref| <= RTOL * max|M*_ref| over their chunk may
flip sign (a rounding artefact); there X may differ by up to 2 eta, and the
element is marked diverged.

Every comparison records the largest |gpu - ref| / ||chunk||_F it saw, per
kind of output, in STATS (printed after each test, and appended as one JSON
line per test to the file PARITY_STATS_FILE names, if set).
"""
from __future__ import annotations

import itertools
from math import comb
from typing import List, Optional, Sequence, Tuple

import numpy as np

from oracle import demo_oracle as O

RTOL = 1e-5
ATOL = 1e-7
# Absolute floor per unit of chunk norm, set at a small multiple of the
# largest floor the GPU parity tests need (measured on MI355X, every GPU test,
# loose floors): with the fast DCT or the identity basis 9.7e-8 (2^-23.3;
# payload 3.8e-8, M* 4.9e-8), and 6.1e-8 over a 700-step free-running run
# (the momentum's own rounding drifts over its memory and levels off near
# 2^-24.4); with a caller basis, whose 64-term float32 products round more
# than the fast transform, 2.4e-7 (2^-22.0).
NOISE = 2.0 ** -22          # 2.5x the measured 2^-23.3
NOISE_DENSE = 2.0 ** -21    # 2x the measured 2^-22.0
MAX_ALTERNATIVES = 256

# per output kind, since the last reset: the largest floor a comparison needed,
# max((|gpu - ref| - RTOL |ref|) / ||chunk||_F), and (kind + "_raw") the
# largest |gpu - ref| / ||chunk||_F
STATS: dict = {}


def _ratio(x: np.ndarray, norms: np.ndarray) -> np.ndarray:
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(norms > 0, x / np.where(norms > 0, norms, 1.0), np.where(x > 0, np.inf, 0.0))


def record(kind: str, diff: np.ndarray, norms: np.ndarray, mask: Optional[np.ndarray] = None,
           ref: Optional[np.ndarray] = None) -> float:
    """Note the floor these elements need (and their raw error) per unit of chunk norm; returns the floor."""
    diff = np.asarray(diff, np.float64)
    excess = diff if ref is None else np.maximum(diff - RTOL * np.abs(ref), 0.0)
    need, raw = _ratio(excess, norms), _ratio(diff, norms)
    if mask is not None:
        need, raw = np.where(mask, need, 0.0), np.where(mask, raw, 0.0)
    m = float(np.max(need)) if need.size else 0.0
    STATS[kind] = max(STATS.get(kind, 0.0), m)
    STATS[kind + "_raw"] = max(STATS.get(kind + "_raw", 0.0), float(np.max(raw)) if raw.size else 0.0)
    return m


def layout(shapes: Sequence[Sequence[int]], k: int, s: int = 64) -> List[Tuple[int, int, int]]:
    """(n_chunks, keff, entry_begin) per tensor, counted by the oracle's rules."""
    out, e = [], 0
    for shp in shapes:
        n = int(np.prod(O.chunk_grid(shp, s)))
        keff = O.k_effective(k, s if len(shp) == 1 else s * s)
        out.append((n, keff, e))
        e += n * keff
    return out


def chunk_mask_to_elements(mask: np.ndarray, shape, s: int = 64) -> np.ndarray:
    """Expand a per-chunk boolean mask to the tensor's elements."""
    n = mask.shape[0]
    block = (n, s) if len(shape) == 1 else (n, s, s)
    full = np.broadcast_to(mask.reshape((n,) + (1,) * (len(block) - 1)), block)
    return O.merge_chunks(full, shape, s).astype(bool)


def _tol(ref: np.ndarray, atol) -> np.ndarray:
    return atol + RTOL * np.abs(ref)


def topk_window(q: np.ndarray, keff: int, noise: float = NOISE, scale: Optional[float] = None):
    """(forced, window, quota) of one chunk's valid top-k sets (oracle values, float64).

    scale: the floor's chunk norm (default ||q||)."""
    mags = np.abs(q)
    numel = mags.size
    if keff >= numel:
        return np.arange(numel), np.array([], dtype=np.int64), 0
    key = mags.astype(np.float32)
    order = np.argsort(-key, kind="stable")
    kth = mags[order[keff - 1]]
    tol = RTOL * kth + noise * (np.linalg.norm(q) if scale is None else scale)
    forced = np.nonzero(mags > kth + tol)[0]
    window = np.nonzero(np.abs(mags - kth) <= tol)[0]
    return forced, window, keff - forced.size


class EncodeReport:
    def __init__(self):
        self.chunks = 0
        self.exact = 0
        self.ties = 0
        self.skipped = 0


def compare_encode(out: dict, shape, keff: int, alpha: float, P0, P1, gpu_M: np.ndarray,
                   gpu_vals: np.ndarray, gpu_idx: np.ndarray, diverged: np.ndarray,
                   report: EncodeReport, where: str = "", s: int = 64, noise: float = NOISE) -> np.ndarray:
    """Check one tensor's encode; returns the updated diverged-chunk mask.

    out: oracle.encode(...) result (float64 Mp_chunks and Q included).
    gpu_vals / gpu_idx: [n_chunks, keff] payload of the tensor.
    noise: the floor per unit of chunk norm (NOISE, or NOISE_DENSE with a
    caller basis).
    """
    n = out["Q"].shape[0]
    Qf = out["Q"].reshape(n, -1)
    norms = np.linalg.norm(out["terms_chunks"].reshape(n, -1), axis=1)  # the floor's scale per chunk
    oidx = out["idx"].astype(np.int64)
    gidx = gpu_idx.astype(np.int64)
    assert gidx.shape == oidx.shape, where
    # payload indices are ascending inside each chunk
    if keff > 1:
        assert np.all(np.diff(gidx, axis=1) > 0), f"{where}: payload indices not ascending"
    same = np.all(gidx == oidx, axis=1)
    new_div = diverged.copy()
    expect_chunks = None
    extra_atol = np.zeros(n)
    for c in np.nonzero(~same & ~diverged)[0]:
        forced, window, quota = topk_window(Qf[c], keff, noise, norms[c])
        g = set(gidx[c].tolist())
        ok = set(forced.tolist()) <= g and g <= set(forced.tolist()) | set(window.tolist())
        assert ok, (f"{where}: chunk {c} GPU top-k set is not a valid top-{keff}: "
                    f"differs from oracle at {sorted(g ^ set(oidx[c].tolist()))[:8]}")
        report.ties += 1
        new_div[c] = True
        if expect_chunks is None:
            expect_chunks = O.split_chunks(out["M"].astype(np.float64), s)
        if comb(window.size, quota) <= MAX_ALTERNATIVES:
            alts = [np.sort(np.concatenate([forced, np.array(sub, dtype=np.int64)]))
                    for sub in itertools.combinations(window.tolist(), quota)]
            match = [a for a in alts if np.array_equal(a, gidx[c])]
            assert match, f"{where}: chunk {c} set not among the oracle's valid sets"
            S = match[0][None, :]
            expect_chunks[c] = O.subtract_selected(out["Mp_chunks"][c:c + 1], out["Q"][c:c + 1], S, alpha,
                                                   P0, P1)[0]
        else:
            # huge window: coefficients in it are near the noise floor; bound the residual difference
            kth = np.abs(Qf[c][oidx[c]]).min()
            tol = RTOL * kth + noise * norms[c]
            extra_atol[c] = 2.0 * quota * (kth + tol) * abs(alpha) * (2.0 / s) * 1.01
    report.chunks += n
    report.exact += int(np.sum(same & ~diverged))
    report.skipped += int(np.sum(diverged))

    # payload values at the GPU's indices, against the oracle's Q there
    live = ~diverged
    qg = np.take_along_axis(Qf, gidx, axis=1)
    vdiff = np.abs(gpu_vals.astype(np.float64) - qg)
    record("payload", vdiff, norms[:, None], live[:, None], qg)
    bad = vdiff > _tol(qg, (noise * norms)[:, None])
    bad &= live[:, None]
    assert not bad.any(), f"{where}: payload values differ (chunk {np.nonzero(bad.any(axis=1))[0][:5]})"

    # new momentum, per element, chunks not diverged before this step
    ref_M = out["M"].astype(np.float64) if expect_chunks is None else O.merge_chunks(expect_chunks, shape, s)
    atol_e = chunk_values_to_elements(noise * norms + extra_atol, shape, s)
    emask = chunk_mask_to_elements(live, shape, s)
    diff = np.abs(gpu_M.astype(np.float64) - ref_M)
    record("momentum", diff, chunk_values_to_elements(norms, shape, s), emask, ref_M)
    bad = (diff > _tol(ref_M, atol_e)) & emask
    if bad.any():
        i = np.argmax(np.where(bad, diff, 0))
        raise AssertionError(f"{where}: momentum differs at flat {i}: gpu {gpu_M.ravel()[i]!r} "
                             f"ref {ref_M.ravel()[i]!r} ({int(bad.sum())} elements)")
    return new_div


def chunk_values_to_elements(vals: np.ndarray, shape, s: int = 64) -> np.ndarray:
    n = vals.shape[0]
    block = (n, s) if len(shape) == 1 else (n, s, s)
    full = np.broadcast_to(vals.reshape((n,) + (1,) * (len(block) - 1)), block)
    return O.merge_chunks(full, shape, s)


def compare_decode(dec: dict, shape, phi: str, eta: float, gpu_X: np.ndarray, chunk_diverged: np.ndarray,
                   elem_diverged: Optional[np.ndarray], where: str = "", s: int = 64) -> np.ndarray:
    """Check one tensor's decode/apply; returns the updated diverged-element mask."""
    ref = dec["X"].astype(np.float64)
    Mstar = dec["Mstar"]
    emask = ~chunk_mask_to_elements(chunk_diverged, shape, s)
    if elem_diverged is not None:
        emask &= ~elem_diverged
    new_elem = np.zeros(shape, dtype=bool) if elem_diverged is None else elem_diverged.copy()
    diff = np.abs(gpu_X.astype(np.float64) - ref)
    tol = _tol(ref, ATOL)
    if phi == "sign":
        ch = O.split_chunks(np.abs(Mstar), s)
        cmax = ch.reshape(ch.shape[0], -1).max(axis=1)
        thresh = chunk_values_to_elements(RTOL * cmax, shape, s)
        near0 = np.abs(Mstar) <= thresh
        flip = near0 & (diff > tol)
        assert not np.any(flip & emask & (diff > 2 * eta + tol)), f"{where}: near-zero sign element off by > 2 eta"
        new_elem |= flip
        emask &= ~flip
    STATS["params_over_tol"] = max(STATS.get("params_over_tol", 0.0), float(np.max(np.where(emask, diff / tol, 0.0))))
    bad = (diff > tol) & emask
    if bad.any():
        i = np.argmax(np.where(bad, diff, 0))
        raise AssertionError(f"{where}: parameters differ at flat {i}: gpu {gpu_X.ravel()[i]!r} "
                             f"ref {ref.ravel()[i]!r} M* {Mstar.ravel()[i]!r} ({int(bad.sum())} elements)")
    return new_elem


def compare_momentum(ref_M: np.ndarray, gpu_M: np.ndarray, shape, chunk_diverged: np.ndarray, where: str = "",
                     s: int = 64, scale: Optional[np.ndarray] = None, noise: float = NOISE):
    """Check a momentum tensor after the aggregated subtraction M - alpha M*, chunks not diverged only.

    scale: the tensor alpha * M* (float64); the floor's chunk norm is
    ||M_new|| + ||alpha M*|| per chunk, since M - alpha M* may cancel."""
    ref = ref_M.astype(np.float64)
    n = chunk_diverged.shape[0]
    norms = np.linalg.norm(O.split_chunks(ref, s).reshape(n, -1), axis=1)
    if scale is not None:
        norms = norms + np.linalg.norm(O.split_chunks(np.asarray(scale, np.float64), s).reshape(n, -1), axis=1)
    norm_e = chunk_values_to_elements(norms, shape, s)
    live = ~chunk_mask_to_elements(chunk_diverged, shape, s)
    diff = np.abs(gpu_M.astype(np.float64) - ref)
    record("momentum_aggregated", diff, norm_e, live, ref)
    bad = (diff > _tol(ref, noise * norm_e)) & live
    if bad.any():
        i = np.argmax(np.where(bad, diff, 0))
        raise AssertionError(f"{where}: momentum differs at flat {i}: gpu {gpu_M.ravel()[i]!r} "
                             f"ref {ref.ravel()[i]!r} ({int(bad.sum())} elements)")


def compare_mstar(Qabs: np.ndarray, ref_Mstar: np.ndarray, gpu_Mstar: np.ndarray, shape, chunk_diverged: np.ndarray,
                  where: str = "", s: int = 64, noise: float = NOISE) -> float:
    """Check a decoded M* element by element: |gpu - ref| <= noise * ||Qabs chunk|| + RTOL * |ref|.

    Qabs: the oracle's average of the payload values' magnitudes [n_chunks,
    numel] (decode_apply's "Qabs"; at least the norm of the whole, uncropped
    M* chunk); ref_Mstar: its M* (cropped); gpu_Mstar: the GPU's.  Chunks in
    chunk_diverged are skipped.  Returns the largest floor needed per unit of
    chunk norm."""
    ref = np.asarray(ref_Mstar, np.float64)
    n = chunk_diverged.shape[0]
    norms = np.linalg.norm(np.asarray(Qabs, np.float64).reshape(n, -1), axis=1)
    norm_e = chunk_values_to_elements(norms, shape, s)
    live = ~chunk_mask_to_elements(chunk_diverged, shape, s)
    diff = np.abs(np.asarray(gpu_Mstar, np.float64) - ref)
    worst = record("mstar", diff, norm_e, live, ref)
    bad = (diff > _tol(ref, noise * norm_e)) & live
    if bad.any():
        i = np.argmax(np.where(bad, diff, 0))
        raise AssertionError(f"{where}: M* differs at flat {i}: gpu {np.ravel(gpu_Mstar)[i]!r} "
                             f"ref {ref.ravel()[i]!r} ({int(bad.sum())} elements; chunk norm {norm_e.ravel()[i]!r})")
    return worst


def _bits(words: np.ndarray, n_chunks: int) -> np.ndarray:
    by = np.ascontiguousarray(np.asarray(words).astype("<u8")).view(np.uint8).reshape(-1, 8)
    return np.unpackbits(by, axis=1, bitorder="little").reshape(n_chunks, -1).astype(bool)


def compare_signs(Mstar: np.ndarray, shape, gpu_words: np.ndarray, chunk_diverged: np.ndarray, where: str = "",
                  s: int = 64):
    """Check one tensor's packed sign words against the oracle's packing of its M*.

    Bit-exact on every valid element except where |M*| is within RTOL of its
    chunk's largest |M*| (float rounding may flip such a sign, as for Signum)
    and in chunks whose top-k legitimately diverged; padding bits must be 0."""
    n = chunk_diverged.shape[0]
    ref = _bits(O.pack_signs(Mstar, s), n)
    got = _bits(gpu_words, n)
    valid = O.split_chunks(np.ones(shape), s).reshape(n, -1) != 0
    pad = got & ~valid
    assert not pad.any(), f"{where}: {int(pad.sum())} padding bits set"
    a = O.split_chunks(np.abs(Mstar), s).reshape(n, -1)
    near0 = a <= RTOL * a.max(axis=1, keepdims=True)
    live = valid & ~near0 & ~chunk_diverged[:, None]
    bad = (got != ref) & live
    if bad.any():
        c, e = np.argwhere(bad)[0]
        raise AssertionError(f"{where}: sign bit differs in chunk {c} element {e} "
                             f"({int(bad.sum())} bits; M* there {O.split_chunks(Mstar, s).reshape(n, -1)[c, e]!r})")
    return int(((got != ref) & valid).sum())


def _bf16_value(codes: np.ndarray) -> np.ndarray:
    return (np.asarray(codes, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def compare_wire(values: np.ndarray, idx: np.ndarray, Q: np.ndarray, gpu_codes: np.ndarray, gpu_idx: np.ndarray,
                 diverged: np.ndarray, where: str = "", noise: float = NOISE) -> np.ndarray:
    """Check one tensor's wire entries; returns the chunks whose bfloat16 codes differ.

    values / idx: the oracle's payload [n, keff] (float32 values); Q: the
    floor's scale per chunk [n, ...] (the encode's terms_chunks); gpu_codes / gpu_idx: the
    GPU wire entries unpacked [n, keff].  Chunks already diverged are skipped.
    Indices must match exactly.  The bfloat16 code is a rounding decision
    taken on a float32 value that may itself differ from the oracle's within
    the payload tolerance, so a GPU code is valid iff it is the rounding of
    some value within that tolerance of the oracle's: between the codes of
    v - tol and v + tol (rounding is monotonic).  Chunks where it is valid
    but not the oracle's own code are returned as diverged.
    """
    n = values.shape[0]
    live = ~diverged
    gi = np.asarray(gpu_idx).astype(np.int64)
    assert np.array_equal(gi[live], np.asarray(idx).astype(np.int64)[live]), f"{where}: wire indices differ"
    norms = np.linalg.norm(np.asarray(Q, dtype=np.float64).reshape(n, -1), axis=1)
    v = np.asarray(values, dtype=np.float32)
    tol = _tol(v.astype(np.float64), (noise * norms)[:, None])
    lo = _bf16_value(O.bf16_bits((v - tol).astype(np.float32)))
    hi = _bf16_value(O.bf16_bits((v + tol).astype(np.float32)))
    g = _bf16_value(gpu_codes)
    bad = ~((lo <= g) & (g <= hi)) & live[:, None]
    assert not bad.any(), f"{where}: wire values outside the rounding of the tolerance (chunks " \
                          f"{np.nonzero(bad.any(axis=1))[0][:5]})"
    return ((np.asarray(gpu_codes) != O.bf16_bits(v)) & live[:, None]).any(axis=1)
