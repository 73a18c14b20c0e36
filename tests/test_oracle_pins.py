"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a closed form, a library routine
(SciPy's DCT, NumPy's QR), brute force over every index subset on tiny
chunks, or a number the pages print (tests/golden/pages_numbers.json).
They are chosen so that a dropped term, a flipped sign, a wrong index or a
transposed operand in the oracle fails at least one of them.
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.fft

from oracle import demo_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")


def f32(x):
    """A hyper-parameter as the codec receives it: its float32 value."""
    return float(np.float32(x))


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------- P1/P2/P3: the basis

@pytest.mark.parametrize("s", [2, 4, 8, 64, 128])
def test_dct_basis_is_scipy_orthonormal_dct2(s):
    P = O.dct_basis(s)
    assert np.abs(P @ P.T - np.eye(s)).max() < 1e-13
    assert np.abs(P.T @ P - np.eye(s)).max() < 1e-13
    ref = scipy.fft.dct(np.eye(s), type=2, norm="ortho", axis=0)
    assert np.abs(P - ref).max() < 1e-14


def test_project_matches_scipy_dctn_and_idctn():
    rng = _rng(1)
    P = O.dct_basis(64)
    B = rng.standard_normal((5, 64, 64))
    Q = O.project(B, P, P)
    assert np.abs(Q - scipy.fft.dctn(B, type=2, norm="ortho", axes=(1, 2))).max() < 1e-12
    assert np.abs(O.unproject(Q, P, P) - scipy.fft.idctn(Q, type=2, norm="ortho", axes=(1, 2))).max() < 1e-12
    b = rng.standard_normal((7, 64))
    q = O.project(b, P, P)
    assert np.abs(q - scipy.fft.dct(b, type=2, norm="ortho", axis=1)).max() < 1e-12
    assert np.abs(O.unproject(q, P, P) - b).max() < 1e-12


def test_round_trip_exact_in_fp64():
    rng = _rng(2)
    P = O.dct_basis(64)
    B = rng.standard_normal((3, 64, 64)) * 1e-3
    R = O.unproject(O.project(B, P, P), P, P)
    assert np.abs(R - B).max() <= 1e-13 * np.abs(B).max()


def test_parseval_per_chunk_including_padded_chunks():
    rng = _rng(3)
    T = rng.standard_normal((1000, 777))
    P = O.dct_basis(64)
    C = O.split_chunks(T)
    Q = O.project(C, P, P)
    nb = np.sqrt((C ** 2).sum(axis=(1, 2)))
    nq = np.sqrt((Q ** 2).sum(axis=(1, 2)))
    assert np.abs(nb - nq).max() <= 1e-12 * nb.max()
    assert abs(np.sqrt((nq ** 2).sum()) - np.linalg.norm(T)) <= 1e-10 * np.linalg.norm(T)


# --------------------------------------------------------------------------- chunking

def test_chunk_layout_row_major_with_zero_padding():
    T = np.arange(130 * 200, dtype=np.float64).reshape(130, 200)
    C = O.split_chunks(T)
    assert C.shape == (3 * 4, 64, 64)
    # chunk (1, 2) starts at row 64, column 128
    assert C[1 * 4 + 2, 0, 0] == T[64, 128]
    assert C[1 * 4 + 2, 5, 7] == T[69, 135]
    # last chunk (2, 3): rows 128..129, columns 192..199 valid, rest zero
    last = C[2 * 4 + 3]
    assert last[1, 7] == T[129, 199]
    assert np.all(last[2:, :] == 0) and np.all(last[:, 8:] == 0)
    assert np.array_equal(O.merge_chunks(C, T.shape), T)
    v = np.arange(130, dtype=np.float64)
    c1 = O.split_chunks(v)
    assert c1.shape == (3, 64) and c1[2, 1] == 129 and np.all(c1[2, 2:] == 0)
    assert np.array_equal(O.merge_chunks(c1, v.shape), v)


# --------------------------------------------------------------------------- P4: payload sizes

def test_payload_ratio_matches_printed_per_chunk_compression():
    gold = json.load(open(GOLDEN))
    for row in gold["per_chunk_compression"]:
        s, k = row["s"], row["k"]
        n = O.payload_entries([(s, s)], k, s)
        assert n == k
        assert (s * s) / n == row["ratio"]
    # sum over chunks of keff, clamped per chunk kind
    shapes = [(1000, 777), (3, 5000), (777,), (1,)]
    grids = [16 * 13, 1 * 79, 13, 1]
    assert O.payload_entries(shapes, 8) == 8 * (grids[0] + grids[1]) + 8 * (grids[2] + grids[3])
    assert O.payload_entries(shapes, 4096) == 4096 * (grids[0] + grids[1]) + 64 * (grids[2] + grids[3])


# --------------------------------------------------------------------------- momentum update

def test_momentum_half_life_printed_on_the_page():
    gold = json.load(open(GOLDEN))["momentum_half_life"]
    beta = gold["beta"]
    G = np.ones((4,))
    M = O.momentum_update(np.zeros(4), G, beta)          # impulse at step 0
    M0 = M.copy()
    for _ in range(gold["steps"]):
        M = O.momentum_update(M, np.zeros(4), beta)
    # the codec receives beta as float32: the impulse weight is 1 - float32(beta)
    assert M0[0] == pytest.approx(1.0 - float(np.float32(beta)), rel=1e-12)
    assert M0[0] == pytest.approx(1.0 - beta, rel=2e-5)
    assert M[0] / M0[0] == pytest.approx(gold["weight"], rel=2e-3)


@pytest.mark.parametrize("plain", [False, True])
def test_ddp_equivalence_closed_form_lossless_alpha0(plain):
    """k = numel, alpha = 0: M_t has the EMA's closed form and M* is the workers' mean."""
    beta, steps, W = 0.9, 5, 3
    rng = _rng(4)
    G = rng.standard_normal((64, 128)).astype(np.float32)
    Ms = [np.zeros_like(G) for _ in range(W)]
    for _ in range(steps):
        outs = [O.encode(Ms[w], G, beta=beta, alpha=0.0, k=4096, plain=plain) for w in range(W)]
        Ms = [o["M"] for o in outs]
    closed = ((1 - beta ** steps) / (1 - beta) if plain else (1 - beta ** steps)) * G.astype(np.float64)
    for w in range(W):
        assert np.abs(Ms[w] - closed).max() <= 1e-6 * np.abs(closed).max()
    vals = np.stack([o["values"] for o in outs])
    idx = np.stack([o["idx"] for o in outs])
    X = np.zeros_like(G)
    dec = O.decode_apply(X, vals, idx, phi="identity", eta=1.0, lam=0.0)
    assert np.abs(dec["Mstar"] - closed).max() <= 1e-6 * np.abs(closed).max()
    assert np.abs(dec["X"] + closed).max() <= 1e-6 * np.abs(closed).max()


def test_mean_of_local_momenta_is_momentum_of_mean_gradient():
    beta, W, steps = 0.99, 4, 6
    rng = _rng(5)
    Ms = [np.zeros(50) for _ in range(W)]
    Mg = np.zeros(50)
    for _ in range(steps):
        Gs = [rng.standard_normal(50) for _ in range(W)]
        Ms = [O.momentum_update(Ms[w], Gs[w], beta) for w in range(W)]
        Mg = O.momentum_update(Mg, np.mean(Gs, axis=0), beta)
    assert np.abs(np.mean(Ms, axis=0) - Mg).max() < 1e-14


# --------------------------------------------------------------------------- P5: lossless, subtraction

@pytest.mark.parametrize("shape", [(64, 64), (130, 70), (100,), (1, 1)])
def test_lossless_alpha1_leaves_zero_residual(shape):
    rng = _rng(6)
    M = rng.standard_normal(shape).astype(np.float32)
    G = rng.standard_normal(shape).astype(np.float32)
    out = O.encode(M, G, beta=0.9, alpha=1.0, k=4096)
    Mp = O.momentum_update(M, G, 0.9)
    assert np.abs(out["M"]).max() <= 1e-13 * np.abs(Mp).max()
    half = O.encode(M, G, beta=0.9, alpha=0.5, k=4096)
    assert np.abs(half["M"] - 0.5 * Mp).max() <= 1e-6 * np.abs(Mp).max()


def test_subtraction_decay_printed_on_the_page():
    gold = json.load(open(GOLDEN))["subtraction_decay"]
    rng = _rng(7)
    M = rng.standard_normal((64, 64)).astype(np.float32)
    beta = 0.999
    out = O.encode(M, np.zeros_like(M), beta=beta, alpha=gold["alpha"], k=4096)
    assert np.abs(out["M"] - gold["kept_fraction"] * beta * M).max() <= 1e-6 * np.abs(M).max()


def test_lossless_decode_is_mean_of_worker_momenta():
    rng = _rng(8)
    W = 3
    Mps, vals, idxs = [], [], []
    for w in range(W):
        M = rng.standard_normal((70, 64)).astype(np.float32)
        G = rng.standard_normal((70, 64)).astype(np.float32)
        o = O.encode(M, G, beta=0.5, alpha=1.0, k=4096)
        Mps.append(O.momentum_update(M, G, 0.5))
        vals.append(o["values"])
        idxs.append(o["idx"])
    X = rng.standard_normal((70, 64)).astype(np.float32)
    d = O.decode_apply(X, np.stack(vals), np.stack(idxs), phi="identity", eta=0.1, lam=0.0)
    mean = np.mean(Mps, axis=0)
    assert np.abs(d["Mstar"] - mean).max() <= 1e-6 * np.abs(mean).max()
    assert np.abs(d["X"] - (X - 0.1 * mean)).max() <= 1e-6


# --------------------------------------------------------------------------- P7: top-k error bound and optimality

def test_topk_error_bound_and_optimality():
    rng = _rng(9)
    P = O.dct_basis(64)
    B = rng.standard_normal((6, 64, 64))
    Q = O.project(B, P, P)
    for k in (1, 8, 32, 500):
        S = O.select_topk(Q.reshape(6, -1), k)
        for c in range(6):
            q = Q[c].ravel()
            qh = np.zeros_like(q)
            qh[S[c]] = q[S[c]]
            err = np.linalg.norm(q - qh)
            assert err <= np.sqrt(1 - k / 4096) * np.linalg.norm(q) + 1e-12
            # any other k-subset leaves at least as large a residual
            for _ in range(20):
                T = rng.choice(4096, size=k, replace=False)
                other = np.zeros_like(q)
                other[T] = q[T]
                assert np.linalg.norm(q - other) >= err - 1e-12


# --------------------------------------------------------------------------- P8: brute force on tiny chunks

def _brute_force_set(B, P, keff):
    """Lowest-residual keff-subset, lexicographically smallest among (near) equal residuals."""
    Q = O.project(B[None], P, P)[0]
    numel = Q.size
    best, best_sets = None, []
    for S in itertools.combinations(range(numel), keff):
        qh = np.zeros(numel)
        qh[list(S)] = Q.ravel()[list(S)]
        r = np.linalg.norm(B - O.unproject(qh.reshape(Q.shape)[None], P, P)[0])
        if best is None or r < best - 1e-12:
            best, best_sets = r, [S]
        elif abs(r - best) <= 1e-12:
            best_sets.append(S)
    return min(best_sets)


@pytest.mark.parametrize("s", [2, 4])
@pytest.mark.parametrize("ndim", [1, 2])
def test_topk_equals_brute_force_on_tiny_chunks(s, ndim):
    rng = _rng(10 + s + ndim)
    P = O.dct_basis(s)
    numel = s if ndim == 1 else s * s
    shape = (s,) if ndim == 1 else (s, s)
    cases = [rng.standard_normal(shape) for _ in range(4)]
    # exact ties: a chunk whose coefficients are +-1, +-1, 0.5, ... in a fixed pattern
    Qd = np.zeros(numel)
    Qd[::2] = 1.0
    Qd[1::3] = -1.0
    cases.append(O.unproject(Qd.reshape(shape)[None], P, P)[0])
    cases.append(np.zeros(shape))
    for B in cases:
        Q = O.project(B[None], P, P).reshape(1, numel)
        for keff in range(1, numel + 1):
            if numel == 16 and keff > 6:
                continue
            S = O.select_topk(Q, keff)[0]
            assert tuple(S) == _brute_force_set(B, P, keff)


def test_full_encode_at_s4_matches_brute_force_residual():
    rng = _rng(20)
    s, k, alpha, beta = 4, 3, 0.3, 0.9
    P = O.dct_basis(s)
    M = rng.standard_normal((6, 9)).astype(np.float32)
    G = rng.standard_normal((6, 9)).astype(np.float32)
    out = O.encode(M, G, beta=beta, alpha=alpha, k=k, P0=P, P1=P, s=s)
    Mp = O.split_chunks(beta * M.astype(np.float64) + (1 - beta) * G.astype(np.float64), s)
    expect = []
    for c in range(Mp.shape[0]):
        S = _brute_force_set(Mp[c], P, k)
        assert tuple(out["idx"][c]) == S
        Q = O.project(Mp[c][None], P, P)[0].ravel()
        qh = np.zeros(s * s)
        qh[list(S)] = Q[list(S)]
        expect.append(Mp[c] - alpha * O.unproject(qh.reshape(s, s)[None], P, P)[0])
    ref = O.merge_chunks(np.stack(expect), M.shape, s)
    assert np.abs(out["M"] - ref).max() <= 1e-6 * np.abs(ref).max()


# --------------------------------------------------------------------------- P9/P10: closed-form chunks

def test_single_basis_function_chunk():
    P = O.dct_basis(64)
    u, v, c = 5, 17, 0.75
    B = c * np.outer(P[u], P[v])
    out = O.encode(np.zeros((64, 64), np.float32), B.astype(np.float32), beta=0.0, alpha=1.0, k=1)
    assert out["idx"][0, 0] == u * 64 + v
    assert out["values"][0, 0] == pytest.approx(c, rel=1e-6)
    assert np.abs(out["M"]).max() < 1e-7


def test_nonsymmetric_basis_pair_is_not_transposed():
    """With P0 != P1, B = c * P0[u]^T P1[v] must land at (u, v), not (v, u)."""
    rng = _rng(21)
    P0 = O.orthonormal_rows(rng.standard_normal((64, 64)))
    P1 = O.orthonormal_rows(rng.standard_normal((64, 64)))
    u, v, c = 3, 40, -2.0
    B = c * np.outer(P0[u], P1[v])
    Q = O.project(B[None], P0, P1)[0]
    expect = np.zeros((64, 64))
    expect[u, v] = c
    assert np.abs(Q - expect).max() < 1e-12
    out = O.encode(np.zeros((64, 64), np.float32), B.astype(np.float32), beta=0.0, alpha=0.5, k=1, P0=P0, P1=P1)
    assert out["idx"][0, 0] == u * 64 + v
    assert np.abs(out["M"] - 0.5 * B).max() < 1e-6


def test_constant_chunk_dc_coefficient():
    P = O.dct_basis(64)
    c = 0.3
    Q = O.project(np.full((1, 64, 64), c), P, P)[0]
    assert Q[0, 0] == pytest.approx(64 * c, rel=1e-13)
    assert np.abs(Q.ravel()[1:]).max() < 1e-13
    q = O.project(np.full((1, 64), c), P, P)[0]
    assert q[0] == pytest.approx(8 * c, rel=1e-13)


def test_all_zero_chunk_payload_and_decode():
    Z = np.zeros((64, 128), np.float32)
    out = O.encode(Z, Z, beta=0.9, alpha=0.2, k=5)
    assert np.array_equal(out["idx"], np.tile(np.arange(5, dtype=np.uint16), (2, 1)))
    assert np.all(out["values"] == 0)
    X = _rng(22).standard_normal((64, 128)).astype(np.float32)
    d = O.decode_apply(X, out["values"][None], out["idx"][None], phi="sign", eta=1e-3, lam=0.01)
    assert np.all(d["Mstar"] == 0)
    assert np.array_equal(d["X"], (X.astype(np.float64) * (1 - 1e-3 * 0.01)).astype(np.float32))


# --------------------------------------------------------------------------- P11: aggregation modes

def test_aggregation_modes():
    v = np.array([[[1.0, 2.0, 3.0]]], np.float32)
    i = np.array([[[0, 5, 9]]], np.uint16)
    same_v, same_i = np.repeat(v, 3, axis=0), np.repeat(i, 3, axis=0)
    for mode in ("count", "workers"):
        Qb = O.aggregate(same_v, same_i, 16, mode)
        assert Qb[0, 0] == 1.0 and Qb[0, 5] == 2.0 and Qb[0, 9] == 3.0
    dv = np.array([[[1.0, 2.0]], [[4.0, 8.0]]], np.float32)
    di = np.array([[[0, 1]], [[2, 3]]], np.uint16)
    Qc = O.aggregate(dv, di, 4, "count")
    Qw = O.aggregate(dv, di, 4, "workers")
    assert list(Qc[0]) == [1.0, 2.0, 4.0, 8.0]
    assert list(Qw[0]) == [0.5, 1.0, 2.0, 4.0]
    # index 1 held by two of three workers, one of them with a 0.0 value (still a contributor)
    pv = np.array([[[6.0]], [[0.0]], [[9.0]]], np.float32)
    pi = np.array([[[1]], [[1]], [[2]]], np.uint16)
    Qc = O.aggregate(pv, pi, 4, "count")
    Qw = O.aggregate(pv, pi, 4, "workers")
    assert Qc[0, 1] == 3.0 and Qc[0, 2] == 9.0 and Qc[0, 0] == 0.0
    assert Qw[0, 1] == 2.0 and Qw[0, 2] == 3.0


# --------------------------------------------------------------------------- P12: random orthonormal basis

def test_random_basis_is_gram_schmidt_of_the_draw():
    g = _rng(23).standard_normal((64, 64))
    P = O.orthonormal_rows(g)
    assert np.abs(P @ P.T - np.eye(64)).max() < 1e-12
    q, r = np.linalg.qr(g.T)
    ref = (q * np.sign(np.diag(r))).T
    assert np.abs(P - ref).max() < 1e-10
    P32 = P.astype(np.float32)
    assert np.abs(P32.astype(np.float64) @ P32.T.astype(np.float64) - np.eye(64)).max() < 1e-6
    B = _rng(24).standard_normal((2, 64, 64))
    rt = O.unproject(O.project(B, P32, P32), P32, P32)
    assert np.abs(rt - B).max() < 1e-5


# --------------------------------------------------------------------------- update rule compositions

def test_signum_update_on_lossless_single_worker():
    rng = _rng(25)
    M = rng.standard_normal((64, 64)).astype(np.float32)
    G = rng.standard_normal((64, 64)).astype(np.float32)
    o = O.encode(M, G, beta=0.9, alpha=0.2, k=4096)
    X = rng.standard_normal((64, 64)).astype(np.float32)
    d = O.decode_apply(X, o["values"][None], o["idx"][None], phi="sign", eta=0.01, lam=0.1)
    # the hyper-parameters as the codec receives them (float32)
    b, eta, lam = (float(np.float32(v)) for v in (0.9, 0.01, 0.1))
    Mp = b * M.astype(np.float64) + (1 - b) * G.astype(np.float64)
    ref = X.astype(np.float64) * (1 - eta * lam) - eta * np.sign(Mp)
    # one float32 rounding of the stored result
    assert np.all(np.abs(d["X"] - ref) <= np.spacing(np.abs(ref).astype(np.float32)))


@pytest.mark.parametrize("shape", [(1, 1), (1, 64), (64, 1), (2, 3), (65, 65), (3, 5000), (777,), (1,)])
def test_tiny_and_ragged_shapes_run_and_keep_payload_sorted(shape):
    rng = _rng(26)
    M = rng.standard_normal(shape).astype(np.float32)
    G = rng.standard_normal(shape).astype(np.float32)
    for k in (1, 4, 64, 4096):
        o = O.encode(M, G, beta=0.9, alpha=0.2, k=k)
        numel = 64 if len(shape) == 1 else 4096
        assert o["idx"].shape == (int(np.prod(O.chunk_grid(shape))), min(k, numel))
        assert np.all(np.diff(o["idx"].astype(np.int64), axis=1) > 0)
        assert o["M"].shape == shape and o["M"].dtype == np.float32


def test_identity_basis_ranks_and_subtracts_in_parameter_space():
    """P0 = P1 = I (the identity choice of the projection): Q is the block itself, the payload is the
    block's own largest entries, and the residual scales exactly those entries by (1 - alpha)."""
    rng = _rng(11)
    G = rng.standard_normal((70, 130)).astype(np.float32)
    eye = np.eye(64)
    out = O.encode(np.zeros_like(G), G, beta=0.5, alpha=0.25, k=3, P0=eye, P1=eye)
    Mp = 0.5 * G.astype(np.float64)
    chunks = O.split_chunks(Mp)
    assert np.array_equal(out["Q"], chunks)
    for c in range(chunks.shape[0]):
        flat = chunks[c].ravel()
        want = np.sort(np.argsort(-np.abs(flat).astype(np.float32), kind="stable")[:3])
        assert np.array_equal(out["idx"][c], want)
        assert np.array_equal(out["values"][c], flat[want].astype(np.float32))
    expect = chunks.copy().reshape(chunks.shape[0], -1)
    rows = np.arange(chunks.shape[0])[:, None]
    expect[rows, out["idx"].astype(np.int64)] *= 0.75
    assert np.array_equal(out["M"], O.merge_chunks(expect.reshape(chunks.shape), G.shape).astype(np.float32))


@pytest.mark.parametrize("W", [1, 3])
def test_aggregated_subtraction_lossless_closed_form(W):
    """k = numel: Q_bar is the mean of the workers' full coefficients, so M* is the mean of the
    M'_w and the aggregated subtraction leaves M'_w - alpha * mean(M'); with identical workers
    and alpha = 1 that is exactly zero."""
    rng = _rng(12)
    alpha = 0.3
    Gs = [rng.standard_normal((70, 100)).astype(np.float32) for _ in range(W)]
    outs = [O.encode(np.zeros_like(g), g, beta=0.9, alpha=alpha, k=4096, subtract="aggregated") for g in Gs]
    c = 1.0 - f32(0.9)
    for g, o in zip(Gs, outs):
        assert np.array_equal(o["M"], (c * g.astype(np.float64)).astype(np.float32))  # M' kept as is
    dec = O.decode_apply(np.zeros((70, 100), np.float32), np.stack([o["values"] for o in outs]),
                         np.stack([o["idx"] for o in outs]), phi="identity", eta=1.0, lam=0.0)
    mean = np.mean([c * g.astype(np.float64) for g in Gs], axis=0)
    assert np.abs(dec["Mstar"] - mean).max() <= 1e-6 * np.abs(mean).max()
    for o in outs:
        new = O.subtract_aggregated(o["M"], dec["Mstar"], alpha)
        ref = o["M"].astype(np.float64) - f32(alpha) * mean
        assert np.abs(new - ref).max() <= 1e-6 * np.abs(ref).max()
    same = [O.encode(np.zeros_like(Gs[0]), Gs[0], beta=0.9, alpha=1.0, k=4096, subtract="aggregated")
            for _ in range(W)]
    dec = O.decode_apply(np.zeros((70, 100), np.float32), np.stack([o["values"] for o in same]),
                         np.stack([o["idx"] for o in same]), phi="identity", eta=1.0, lam=0.0)
    assert np.abs(O.subtract_aggregated(same[0]["M"], dec["Mstar"], 1.0)).max() <= 1e-7 * np.abs(same[0]["M"]).max()


# --------------------------------------------------------------------------- the one-bit sign download

def test_pack_signs_hand_built_words():
    """Words written out by hand from the layout: chunk after chunk, row-major inside a chunk,
    bit j of a word = the j-th of its 64 elements, set where M* < 0, padding 0."""
    v = np.ones(70)
    v[[0, 3, 63]] = -1.0
    v[66] = -3.0
    v[69] = 0.0  # zero reads as +1: no bit
    assert O.pack_signs(v).tolist() == [1 + 8 + (1 << 63), 4]
    m = np.ones((2, 65))
    m[0, 0] = -1.0    # chunk 0, row 0, column 0
    m[1, 5] = -1.0    # chunk 0, row 1, column 5
    m[0, 64] = -2.0   # chunk 1 (columns 64..127), row 0, column 0
    m[1, 64] = -0.5   # chunk 1, row 1, column 0
    w = O.pack_signs(m)
    assert w.shape == (128,) and O.sign_words([(2, 65)]) == 128
    want = np.zeros(128, np.uint64)
    want[0], want[1], want[64], want[65] = 1, 1 << 5, 1, 1
    assert np.array_equal(w, want)


def test_pack_signs_hand_built_words_chunk128():
    """s = 128, words written out by hand: a 128x128 chunk takes 256 words, chunk row r in words 2r
    (columns 0..63) and 2r + 1 (columns 64..127); a 128-element vector chunk two words."""
    v = np.ones(200)
    v[[1, 64, 127]] = -1.0     # chunk 0: word 0 bit 1, word 1 bits 0 and 63
    v[130] = -7.0              # chunk 1 (elements 128..255): word 2, bit 2
    w = O.pack_signs(v, 128)
    assert w.shape == (4,) and O.sign_words([(200,)], 128) == 4
    assert w.tolist() == [2, 1 + (1 << 63), 4, 0]
    m = np.ones((130, 129))
    m[0, 0] = -1.0      # chunk (0, 0), row 0, column 0: word 0, bit 0
    m[0, 100] = -1.0    # chunk (0, 0), row 0, column 100: word 1, bit 36
    m[127, 127] = -1.0  # chunk (0, 0), row 127, column 127: word 255, bit 63
    m[5, 128] = -1.0    # chunk (0, 1), row 5, column 0: word 256 + 10, bit 0
    m[129, 3] = -1.0    # chunk (1, 0), row 1, column 3: word 512 + 2, bit 3
    m[128, 128] = 0.0   # chunk (1, 1), row 0, column 0: zero reads as +1, no bit
    w = O.pack_signs(m, 128)
    assert w.shape == (1024,) and O.sign_words([(130, 129)], 128) == 1024
    want = np.zeros(1024, np.uint64)
    want[0], want[1], want[255], want[266], want[514] = 1, 1 << 36, 1 << 63, 1, 1 << 3
    assert np.array_equal(w, want)
    # padding: all-negative input sets exactly the valid elements' bits
    w = O.pack_signs(-np.ones((130, 129)), 128)
    assert bin(int(w[3 * 256 + 0])).count("1") == 1      # chunk (1, 1) row 0: one valid column
    assert w[3 * 256 + 4] == 0                           # chunk (1, 1) row 2: past the last row
    assert int(w[256 + 0]) == 1 and int(w[256 + 1]) == 0  # chunk (0, 1) row 0: column 128 only


@pytest.mark.parametrize("s", [64, 128])
@pytest.mark.parametrize("shape", [(130, 70), (64, 64), (3, 200), (777,), (1,), (257, 131)])
def test_pack_signs_bit_address_formula(shape, s):
    """Every element's bit, looked up with the address written out per element: matrix
    element (r, c) sits in chunk (r // s) * ceil(cols / s) + c // s, which starts at word
    chunk * s * s / 64; inside it the element's row-major position p = (r % s) * s + c % s gives
    word p // 64, bit p % 64; vector element e in word e // 64, bit e % 64.  Padding bits stay 0."""
    rng = _rng(40)
    M = rng.standard_normal(shape)
    w = O.pack_signs(M, s)
    assert w.shape == (O.sign_words([shape], s),)
    seen = np.zeros(w.shape[0] * 64, bool)
    for pos in np.ndindex(*shape):
        if len(shape) == 2:
            r, c = pos
            chunk = (r // s) * -(-shape[1] // s) + c // s
            p = (r % s) * s + c % s
            word = chunk * s * s // 64 + p // 64
            bit = p % 64
        else:
            word, bit = pos[0] // 64, pos[0] % 64
        assert bool((int(w[word]) >> bit) & 1) == (M[pos] < 0)
        seen[word * 64 + bit] = True
    for word in range(w.shape[0]):
        for bit in range(64):
            if not seen[word * 64 + bit]:
                assert (int(w[word]) >> bit) & 1 == 0


@pytest.mark.parametrize("s", [64, 128])
def test_apply_signs_closed_forms_and_agreement_with_signum_decode(s):
    rng = _rng(41)
    X = rng.standard_normal((70, 130)).astype(np.float32)
    X64 = X.astype(np.float64)
    n = O.sign_words([X.shape], s)
    for fill, phi in ((0, 1.0), (~np.uint64(0), -1.0)):
        got = O.apply_signs(X, np.full(n, fill, np.uint64), eta=0.01, lam=0.1, s=s)
        ref = X64 - f32(0.01) * (phi + f32(0.1) * X64)
        assert np.all(np.abs(got - ref) <= np.spacing(np.abs(ref).astype(np.float32)))
    # the bit path reproduces the Signum decode wherever M* != 0
    G = rng.standard_normal(X.shape).astype(np.float32)
    o = O.encode(np.zeros_like(G), G, beta=0.9, alpha=0.2, k=37, s=s)
    d = O.decode_apply(X, o["values"][None], o["idx"][None], phi="sign", eta=0.01, lam=0.1, s=s)
    assert np.all(d["Mstar"] != 0)
    got = O.apply_signs(X, O.pack_signs(d["Mstar"], s), eta=0.01, lam=0.1, s=s)
    assert np.array_equal(got, d["X"])
    # zero M* (no coefficient kept anywhere) reads as +1
    z = O.apply_signs(X, O.pack_signs(np.zeros(X.shape), s), eta=0.01, lam=0.0, s=s)
    assert np.all(np.abs(z - (X64 - f32(0.01))) <= np.spacing(np.abs(X64 - f32(0.01)).astype(np.float32)))


# --------------------------------------------------------------------------- chunk edge 128

def test_chunk128_projection_matches_scipy_and_round_trips():
    rng = _rng(50)
    P = O.dct_basis(128)
    B = rng.standard_normal((2, 128, 128))
    Q = O.project(B, P, P)
    assert np.abs(Q - scipy.fft.dctn(B, type=2, norm="ortho", axes=(1, 2))).max() < 1e-11
    assert np.abs(O.unproject(Q, P, P) - B).max() < 1e-12
    b = rng.standard_normal((3, 128))
    assert np.abs(O.project(b, P, P) - scipy.fft.dct(b, type=2, norm="ortho", axis=1)).max() < 1e-12


def test_chunk128_payload_sizes_printed_on_the_page():
    gold = json.load(open(GOLDEN))
    r = gold["chunk_size_payload_ratio"]
    shapes = [(2048, 6144), (2048, 2048), (8192, 2048)]
    for k in (1, 8, 32):
        small = O.payload_entries(shapes, k, r["s_small"])
        large = O.payload_entries(shapes, k, r["s_large"])
        assert small == r["ratio"] * large
    f = gold["chunk_size_fraction_kept"]
    assert O.payload_entries([(f["s"], f["s"])], f["k"], f["s"]) == f["k"]
    assert O.k_effective(10 ** 6, f["s"] * f["s"]) == f["numel"]


def test_chunk128_encode_closed_forms():
    """s = 128: lossless k with alpha = 1 leaves a zero residual; a single basis function is found
    at its index u*128 + v and removed exactly by alpha = 1."""
    rng = _rng(51)
    G = rng.standard_normal((130, 300)).astype(np.float32)
    out = O.encode(np.zeros_like(G), G, beta=0.5, alpha=1.0, k=128 * 128, s=128)
    assert np.abs(out["M"]).max() <= 1e-6 * np.abs(G).max()
    P = O.dct_basis(128)
    blk = (np.outer(P[5], P[77]) * 3.0).astype(np.float32)
    out = O.encode(np.zeros_like(blk), blk, beta=0.0, alpha=1.0, k=1, plain=True, s=128)
    assert out["idx"].tolist() == [[5 * 128 + 77]]
    assert abs(float(out["values"][0, 0]) - 3.0) < 1e-5
    assert np.abs(out["M"]).max() < 1e-5


# --------------------------------------------------------------------------- phi = Muon

@pytest.mark.parametrize("shape", [(7, 12), (12, 7), (9, 9), (1, 5), (5, 1)])
def test_muon_phi_matches_svd_form(shape):
    """M (M^T M + eps I)^(-1/2) = U diag(s / sqrt(s^2 + eps)) V^T, computed independently by SVD."""
    rng = _rng(60)
    M = rng.standard_normal(shape)
    eps = 0.3
    U, sv, Vt = np.linalg.svd(M, full_matrices=False)
    ref = (U * (sv / np.sqrt(sv ** 2 + eps))) @ Vt
    assert np.abs(O.phi_muon(M, eps) - ref).max() < 1e-12


def test_muon_phi_limits_and_scaling():
    rng = _rng(61)
    M = rng.standard_normal((6, 10))
    P = O.phi_muon(M, 0.0)                       # eps = 0: the polar factor, orthonormal rows
    assert np.abs(P @ P.T - np.eye(6)).max() < 1e-12
    c = 37.0                                     # phi(cM, c^2 eps) = phi(M, eps)
    assert np.abs(O.phi_muon(c * M, c * c * 0.5) - O.phi_muon(M, 0.5)).max() < 1e-12
    v = rng.standard_normal(11)                  # a vector is one column: m / sqrt(m.m + eps)
    assert np.abs(O.phi_muon(v, 2.0) - v / np.sqrt(v @ v + 2.0)).max() < 1e-15
    assert np.abs(O.phi_muon(v[:, None], 2.0)[:, 0] - O.phi_muon(v, 2.0)).max() < 1e-14
    # large eps: phi ~ M / sqrt(eps)
    assert np.abs(O.phi_muon(M, 1e12) * 1e6 - M).max() < 1e-6


def test_muon_decode_apply_update():
    rng = _rng(62)
    X = rng.standard_normal((70, 90)).astype(np.float32)
    G = rng.standard_normal((70, 90)).astype(np.float32)
    o = O.encode(np.zeros_like(G), G, beta=0.5, alpha=0.2, k=4096)
    d = O.decode_apply(X, o["values"][None], o["idx"][None], phi="muon", eta=0.01, lam=0.1, eps=1e-3)
    ref = X.astype(np.float64) - f32(0.01) * (O.phi_muon(d["Mstar"], 1e-3) + f32(0.1) * X.astype(np.float64))
    assert np.all(np.abs(d["X"] - ref) <= np.spacing(np.abs(ref).astype(np.float32)))
    assert np.abs(d["Mstar"] - 0.5 * G.astype(np.float64)).max() < 1e-6  # lossless k: M* = M'


# --------------------------------------------------------------------------- compact wire format

def test_wire_format_hand_built():
    one = np.float32(1.0)
    v = np.array([1.0, -2.5, one + np.float32(2.0 ** -8), one + np.float32(3 * 2.0 ** -8), 0.0], np.float32)
    # 1 + 2^-8 is a tie between 0x3F80 and 0x3F81: even wins; 1 + 3*2^-8 ties 0x3F81 / 0x3F82: even wins
    wv, wi = O.pack_wire(v, np.array([0x123, 0xABC, 0xFFF, 0, 7]))
    assert wv.tolist() == [0x3F80, 0xC020, 0x3F80, 0x3F82, 0x0000]
    # 12-bit positions, a little-endian bit string: 5 entries = 60 bits, 8 bytes
    assert wi.tolist() == [0x23, 0xC1, 0xAB, 0xFF, 0x0F, 0x00, 0x07, 0x00]
    vals, idx = O.unpack_wire(wv, wi, 5)
    assert idx.tolist() == [0x123, 0xABC, 0xFFF, 0, 7]
    assert vals.tolist() == [1.0, -2.5, 1.0, 1.0 + 2 * 2.0 ** -7, 0.0]


def test_wire_format_14_bit_positions_hand_built():
    """s = 128: a 128x128 chunk has 16384 positions, 14 bits each.  Positions 0x1234, 0x3FFF, 0, 5 at
    bits 0-13, 14-27, 28-41, 42-55: byte 0 = 0x34; byte 1 = 0x12 (bits 8-13) | 0b11 << 6 = 0xD2; byte 2 =
    0xFF; byte 3 = 0x0F (the last four ones of 0x3FFF, then four zero bits); byte 4 = 0x00; byte 5 =
    5 << 2 = 0x14; byte 6 = 0x00."""
    assert O.wire_index_bits(64) == 12 and O.wire_index_bits(128) == 14
    wv, wi = O.pack_wire(np.array([1.0, 2.0, 0.0, -1.0], np.float32), np.array([0x1234, 0x3FFF, 0, 5]), s=128)
    assert wi.tolist() == [0x34, 0xD2, 0xFF, 0x0F, 0x00, 0x14, 0x00]
    assert wv.tolist() == [0x3F80, 0x4000, 0x0000, 0xBF80]
    assert O.unpack_wire(wv, wi, 4, s=128)[1].tolist() == [0x1234, 0x3FFF, 0, 5]
    with pytest.raises(ValueError):
        O.pack_wire(np.zeros(1, np.float32), np.array([1 << 14]), s=128)
    rng = _rng(71)
    i = rng.integers(0, 1 << 14, 777)
    wv, wi = O.pack_wire(np.zeros(777, np.float32), i, s=128)
    assert wi.size == (777 * 14 + 7) // 8
    assert np.array_equal(O.unpack_wire(wv, wi, 777, s=128)[1], i.astype(np.uint16))


def test_wire_format_round_trip_and_rounding_bound():
    rng = _rng(70)
    v = (rng.standard_normal(1001) * 1e-3).astype(np.float32)
    i = rng.integers(0, 4096, 1001)
    wv, wi = O.pack_wire(v, i)
    assert wi.size == (1001 * 12 + 7) // 8
    vals, idx = O.unpack_wire(wv, wi, 1001)
    assert np.array_equal(idx, i.astype(np.uint16))
    # round to nearest: at most half a bfloat16 ulp (2^-8 relative) away
    assert np.all(np.abs(vals - v) <= np.abs(v) * 2.0 ** -8)
    with pytest.raises(ValueError):
        O.pack_wire(v[:2], np.array([1, 4096]))


# --------------------------------------------------------------------------- multi-step trajectories, lossless limits
#
# With k = numel nothing is dropped, so DeMo over T steps reduces to known
# data-parallel optimizers whose iterates have explicit sums.  These pin the
# oracle's step loop (state carried from step to step, momentum update before
# the selection, subtraction after it, X updated from the pre-update X) and
# not only single steps.  Closed forms are written as sums over the gradient
# history, never as the oracle's recursion.

def _bounded_gradients(rng, T, W, shape):
    """N(0,1) magnitudes pushed away from zero, so that sign() of float32 rounding cannot flip."""
    z = rng.standard_normal((T, W, *shape))
    return (np.sign(z) * (0.1 + np.abs(z))).astype(np.float32)


def _run_lossless(G, *, beta, alpha, phi, eta, lam, plain=False, subtract="local"):
    """Runs the oracle's encode / decode loop over G[t, w]; returns X_T and every M*_t."""
    T, W = G.shape[:2]
    shape = G.shape[2:]
    k = 64 * 64
    X = np.linspace(-1.0, 1.0, int(np.prod(shape))).reshape(shape).astype(np.float32)
    X0 = X.copy()
    Ms = [np.zeros(shape, np.float32) for _ in range(W)]
    Mstars = []
    for t in range(T):
        outs = [O.encode(Ms[w], G[t, w], beta=beta, alpha=alpha, k=k, plain=plain, subtract=subtract)
                for w in range(W)]
        d = O.decode_apply(X, np.stack([o["values"] for o in outs]), np.stack([o["idx"] for o in outs]),
                           phi=phi, eta=eta, lam=lam)
        X = d["X"]
        Mstars.append(d["Mstar"])
        if subtract == "aggregated":
            Ms = [O.subtract_aggregated(o["M"], d["Mstar"], alpha) for o in outs]
        else:
            Ms = [o["M"] for o in outs]
    return X0, X, Mstars, Ms


def _x_closed_form(X0, updates, eta, lam):
    """X_T = (1 - eta lam)^T X_0 - eta sum_t (1 - eta lam)^(T - 1 - t) u_t for X_{t+1} = X_t - eta (u_t + lam X_t)."""
    T = len(updates)
    r = 1.0 - eta * lam
    return r ** T * X0.astype(np.float64) - eta * sum(r ** (T - 1 - t) * u for t, u in enumerate(updates))


@pytest.mark.parametrize("shape,plain", [((130, 70), False), ((64, 64), True), ((100,), False)])
def test_trajectory_alpha1_is_data_parallel_sgd(shape, plain):
    """alpha = 1 and k = numel: every step sends all of M' and leaves M = 0, so M*_t is the
    workers' mean of (1 - beta) G_t (G_t with the plain form) and X follows SGD with weight decay."""
    beta, eta, lam, T, W = 0.9, 0.05, 0.1, 6, 3
    G = _bounded_gradients(_rng(40), T, W, shape)
    X0, X, Mstars, Ms = _run_lossless(G, beta=beta, alpha=1.0, phi="identity", eta=eta, lam=lam, plain=plain)
    c = 1.0 if plain else 1.0 - beta
    gbar = [c * G[t].astype(np.float64).mean(axis=0) for t in range(T)]
    for t in range(T):
        assert np.abs(Mstars[t] - gbar[t]).max() <= 1e-6 * np.abs(gbar[t]).max()
    for M in Ms:
        assert np.abs(M).max() <= 1e-6 * max(np.abs(g).max() for g in gbar)
    ref = _x_closed_form(X0, gbar, eta, lam)
    assert np.abs(X - ref).max() <= 1e-5 * np.abs(ref).max()


@pytest.mark.parametrize("shape", [(130, 70), (100,)])
def test_trajectory_alpha0_is_momentum_sgd(shape):
    """alpha = 0 and k = numel: nothing is subtracted, each worker's M_t is the EMA
    (1 - beta) sum_tau beta^(t - tau) G_tau, M*_t is its workers' mean and X is momentum SGD."""
    beta, eta, lam, T, W = 0.8, 0.05, 0.02, 7, 2
    G = _bounded_gradients(_rng(41), T, W, shape).astype(np.float64)
    X0, X, Mstars, Ms = _run_lossless(G.astype(np.float32), beta=beta, alpha=0.0, phi="identity", eta=eta, lam=lam)
    ema = [(1 - beta) * sum(beta ** (t - tau) * G[tau].mean(axis=0) for tau in range(t + 1)) for t in range(T)]
    for t in range(T):
        assert np.abs(Mstars[t] - ema[t]).max() <= 1e-5 * np.abs(ema[t]).max()
    for w in range(W):
        own = (1 - beta) * sum(beta ** (T - 1 - tau) * G[tau, w] for tau in range(T))
        assert np.abs(Ms[w] - own).max() <= 1e-5 * np.abs(own).max()
    ref = _x_closed_form(X0, ema, eta, lam)
    assert np.abs(X - ref).max() <= 1e-5 * np.abs(ref).max()


def test_trajectory_alpha1_signum_single_worker_is_signsgd():
    """One worker, alpha = 1, k = numel, phi = sign: X_T = X_0 - eta sum_t sign(G_t) exactly
    as signSGD (no weight decay); gradients are kept away from zero so no sign can flip."""
    eta, T = 0.01, 5
    G = _bounded_gradients(_rng(42), T, 1, (70, 130))
    X0, X, _, _ = _run_lossless(G, beta=0.95, alpha=1.0, phi="sign", eta=eta, lam=0.0)
    ref = _x_closed_form(X0, [np.sign(G[t, 0]).astype(np.float64) for t in range(T)], eta, 0.0)
    assert np.abs(X - ref).max() <= 1e-6


def test_trajectory_aggregated_subtraction_mean_closed_form():
    """Aggregated subtraction, k = numel: M*_t = mean of the M'_w and M_w <- M'_w - alpha M*_t,
    so the workers' mean momentum m_t obeys m_t = (1 - alpha) M*_t with
    M*_t = beta m_(t-1) + (1 - beta) gbar_t, i.e.
    M*_t = (1 - beta) sum_tau ((1 - alpha) beta)^(t - tau) gbar_tau."""
    beta, alpha, eta, lam, T, W = 0.9, 0.4, 0.05, 0.0, 6, 3
    G = _bounded_gradients(_rng(43), T, W, (64, 96)).astype(np.float64)
    X0, X, Mstars, Ms = _run_lossless(G.astype(np.float32), beta=beta, alpha=alpha, phi="identity", eta=eta,
                                      lam=lam, subtract="aggregated")
    gbar = [G[t].mean(axis=0) for t in range(T)]
    closed = [(1 - beta) * sum(((1 - alpha) * beta) ** (t - tau) * gbar[tau] for tau in range(t + 1))
              for t in range(T)]
    for t in range(T):
        assert np.abs(Mstars[t] - closed[t]).max() <= 1e-5 * np.abs(closed[t]).max()
    mean_M = np.mean([M.astype(np.float64) for M in Ms], axis=0)
    assert np.abs(mean_M - (1 - alpha) * closed[-1]).max() <= 1e-5 * np.abs(closed[-1]).max()
    ref = _x_closed_form(X0, closed, eta, lam)
    assert np.abs(X - ref).max() <= 1e-5 * np.abs(ref).max()
