"""CPU oracle for the DeMo per-step momentum codec.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
(the HIP library and its Python binding) never imports, links or calls it,
and this module imports nothing from the product.

Plain NumPy.  Every arithmetic step runs in float64; float32 appears only
where the method stores state (momentum M, parameters X, the transmitted
coefficient values), where a float decides an integer (the top-k ranks are
taken on float32 magnitudes, the precision the GPU kernels decide in), and
in the scalar hyper-parameters beta, alpha, eta and lambda, which are taken
at their float32 values (``hp``), the precision in which the codec receives
them; from those values on, every product and sum is float64.
The transforms are explicit O(s^3) matrix products against the basis built
from its definition, and top-k is a full stable sort: slow and plain on
purpose.

Pages followed (cited below by these tags):
  [S] "DeMo: Decoupled Momentum Optimization", paper-graph-ui summary of
      arXiv 2411.19870.  Section names refer to its §3.4 "Detailed,
      sentence-based technical breakdown" unless stated.
  [N] papernotes.org ICLR 2026 note "DeMo: Decoupled Momentum
      Optimization", section 方法详解 (整体框架 flowchart, 关键设计 1-3).

Readings taken where the pages are silent or disagree (the kernels take
the same ones):
  * momentum form: (1-beta)*G by default, plain G behind ``plain=True``;
  * momentum subtraction uses the worker's OWN selected coefficients
    (``subtract="aggregated"`` with ``subtract_aggregated`` gives the
    summary page's aggregated reading);
  * averaging divides by the number of workers whose payload holds the
    index (membership, even for a 0.0 value); ``mode="workers"`` divides by W;
  * dims not divisible by s are zero-padded; the full s x s block is
    transformed and ranked; residual and M* are cropped;
  * k larger than a chunk is clamped to the chunk's element count;
  * ties in float32 magnitude go to the lower chunk-local index
    idx = u*s + v (u: dimension-0 frequency, v: dimension-1 frequency);
  * sign(0) = 0; weight decay uses the pre-update X on every tensor;
  * Muon's phi acts on each whole tensor (a vector as one column) with the
    caller's eps, the formula the pages print;
  * the one-bit download (``pack_signs``) sets a bit where M* < 0, so a
    zero reads as +1 there.

Pins: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, SciPy's DCT routines, brute force over all index
subsets at s in {2, 4}, and the per-chunk compression ratio the pages print.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64
F32 = np.float32


# ---------------------------------------------------------------------------
# bases
# ---------------------------------------------------------------------------

def dct_basis(s: int = 64) -> np.ndarray:
    """Orthonormal DCT-II matrix, rows are frequencies u, columns samples n.

    P[u, n] = sqrt((2 - [u == 0]) / s) * cos(pi * (2n + 1) * u / (2 s)).
    [S] Blockwise Linear Projection (DCT): a fixed orthonormal basis, the
    standard DCT-II, with P^T = P^-1.
    """
    n = np.arange(s, dtype=F64)
    u = np.arange(s, dtype=F64)[:, None]
    P = np.cos(np.pi * (2.0 * n[None, :] + 1.0) * u / (2.0 * s))
    scale = np.full((s, 1), np.sqrt(2.0 / s))
    scale[0, 0] = np.sqrt(1.0 / s)
    return P * scale


def orthonormal_rows(gauss: np.ndarray) -> np.ndarray:
    """Gram-Schmidt on the rows of a Gaussian draw; returns the orthonormal rows.

    [S] Blockwise Linear Projection: random orthonormal matrices sampled from
    N(0, I) and orthonormalised by Gram-Schmidt, seeded by the step so every
    worker draws the same matrix.  Modified Gram-Schmidt, float64.
    """
    A = np.array(gauss, dtype=F64, copy=True)
    s = A.shape[0]
    for i in range(s):
        for j in range(i):
            A[i] -= np.dot(A[j], A[i]) * A[j]
        A[i] /= np.sqrt(np.dot(A[i], A[i]))
    return A


# ---------------------------------------------------------------------------
# encode: momentum update, chunking, projection, top-k, momentum subtraction
# ---------------------------------------------------------------------------

def hp(x: float) -> float:
    """A scalar hyper-parameter at its float32 value (returned as a Python float)."""
    return float(np.float32(x))


def momentum_update(M: np.ndarray, G: np.ndarray, beta: float, plain: bool = False) -> np.ndarray:
    """Local momentum, no gradient all-reduce.

    [S] Decoupled Local Momentum Updates: M_t = beta * M_{t-1} + (1 - beta) * G_t.
    [N] 整体框架 flowchart states the plain form M_t = beta * M_{t-1} + G_t
    (``plain=True``).  beta is taken at float32; 1 - beta is then formed in
    float64 from that value.
    """
    M64 = np.asarray(M, dtype=F64)
    G64 = np.asarray(G, dtype=F64)
    b = hp(beta)
    c = 1.0 if plain else (1.0 - b)
    return b * M64 + c * G64


def chunk_grid(shape: Sequence[int], s: int = 64) -> Tuple[int, ...]:
    """Chunks per dimension after zero-padding each dimension up to a multiple of s."""
    return tuple(-(-int(n) // s) for n in shape)


def split_chunks(T: np.ndarray, s: int = 64) -> np.ndarray:
    """Partition a 1-D or 2-D tensor into s-blocks (s x s for matrices).

    [S] Tensor Chunking: B(M) = {B_k}, block k covers rows [k0 s, (k0+1) s)
    and columns [k1 s, (k1+1) s); 64 x 64 blocks for matrices and
    64-element blocks for 1-D parameters.  Reading: trailing blocks are
    zero-padded; blocks are listed in row-major order of (k0, k1).
    Returns float64 [n_chunks, s, s] (2-D) or [n_chunks, s] (1-D).
    """
    T = np.asarray(T, dtype=F64)
    grid = chunk_grid(T.shape, s)
    if T.ndim == 1:
        pad = np.zeros(grid[0] * s, dtype=F64)
        pad[: T.shape[0]] = T
        return pad.reshape(grid[0], s)
    if T.ndim != 2:
        raise ValueError("only 1-D and 2-D tensors are chunked")
    pad = np.zeros((grid[0] * s, grid[1] * s), dtype=F64)
    pad[: T.shape[0], : T.shape[1]] = T
    return pad.reshape(grid[0], s, grid[1], s).transpose(0, 2, 1, 3).reshape(grid[0] * grid[1], s, s)


def merge_chunks(chunks: np.ndarray, shape: Sequence[int], s: int = 64) -> np.ndarray:
    """Inverse of split_chunks: reassemble the blocks and crop the padding ([S] unchunking B^-1)."""
    grid = chunk_grid(shape, s)
    if len(shape) == 1:
        return np.asarray(chunks).reshape(grid[0] * s)[: shape[0]]
    full = np.asarray(chunks).reshape(grid[0], grid[1], s, s).transpose(0, 2, 1, 3)
    full = full.reshape(grid[0] * s, grid[1] * s)
    return full[: shape[0], : shape[1]]


def project(B: np.ndarray, P0: np.ndarray, P1: np.ndarray) -> np.ndarray:
    """Forward separable transform of every chunk.

    [S] Blockwise Linear Projection: Q_k = P0 B_k P1^T for d = 2; for a
    1-D block only P0 acts (Q = P0 b).  B is [n, s, s] or [n, s].
    """
    P0 = np.asarray(P0, dtype=F64)
    P1 = np.asarray(P1, dtype=F64)
    if B.ndim == 2:
        return B @ P0.T
    return P0 @ B @ P1.T


def unproject(Q: np.ndarray, P0: np.ndarray, P1: np.ndarray) -> np.ndarray:
    """Inverse separable transform of every chunk.

    [S] Momentum Subtraction and Server-Side Aggregation: T^-1 uses
    P_i^-1 = P_i^T, so B = P0^T Q P1 (1-D: b = P0^T q).
    """
    P0 = np.asarray(P0, dtype=F64)
    P1 = np.asarray(P1, dtype=F64)
    if Q.ndim == 2:
        return Q @ P0
    return P0.T @ Q @ P1


def k_effective(k: int, chunk_numel: int) -> int:
    """Reading: a k above the chunk's element count keeps every coefficient."""
    return min(int(k), int(chunk_numel))


def select_topk(Qflat: np.ndarray, keff: int) -> np.ndarray:
    """Indices of the keff largest-magnitude coefficients of every chunk, ascending.

    [S] Top-k Sparsification: keep the k largest-magnitude coefficients, all
    others set to zero (||Q_hat||_0 = k).  The rank is taken on float32
    magnitudes; equal magnitudes go to the lower chunk-local index (a full
    stable sort on the negated key).  Qflat is [n_chunks, numel].
    """
    key = np.abs(Qflat).astype(F32)
    order = np.argsort(-key, axis=1, kind="stable")
    return np.sort(order[:, :keff], axis=1)


def subtract_selected(Mp_chunks: np.ndarray, Q: np.ndarray, S: np.ndarray, alpha: float,
                      P0: np.ndarray, P1: np.ndarray) -> np.ndarray:
    """Momentum subtraction of the coefficients at index sets S (one row per chunk).

    [S] Momentum Subtraction as Implicit Error Feedback: M <- M - alpha *
    B^-1(T^-1(Q_hat)).  [N] 关键设计 3: the worker subtracts what it itself
    decoded from its transmitted coefficients (local reading).
    """
    n = Q.shape[0]
    Qflat = Q.reshape(n, -1)
    Qhat = np.zeros_like(Qflat)
    rows = np.arange(n)[:, None]
    Qhat[rows, S] = Qflat[rows, S]
    R = unproject(Qhat.reshape(Q.shape), P0, P1)
    return Mp_chunks - hp(alpha) * R


def encode(M: np.ndarray, G: np.ndarray, *, beta: float, alpha: float, k: int,
           plain: bool = False, P0: Optional[np.ndarray] = None, P1: Optional[np.ndarray] = None,
           s: int = 64, subtract: str = "local") -> Dict[str, np.ndarray]:
    """One worker's encode of one tensor.

    Steps in the pages' order: local momentum update, chunking, projection,
    per-chunk top-k, payload (value, index), momentum subtraction.
    ``subtract="aggregated"`` leaves M' in place: [S] Momentum Subtraction
    writes the subtraction with the server's averaged coefficients, which
    only exist after the exchange (see ``subtract_aggregated``).
    Returns float32 ``M`` (new momentum), float32 ``values`` [n_chunks, keff],
    uint16 ``idx`` [n_chunks, keff] (ascending per chunk), and for the tests
    the float64 intermediates ``Mp_chunks`` and ``Q``, and ``terms_chunks``:
    per element |beta M| + |c G|, the magnitudes of the momentum update's two
    terms (the scale of a float32 evaluation's rounding error).
    """
    P0 = dct_basis(s) if P0 is None else np.asarray(P0, dtype=F64)
    P1 = dct_basis(s) if P1 is None else np.asarray(P1, dtype=F64)
    M = np.asarray(M)
    Mp = momentum_update(M, G, beta, plain)
    chunks = split_chunks(Mp, s)
    Q = project(chunks, P0, P1)
    n = Q.shape[0]
    numel = Q[0].size
    keff = k_effective(k, numel)
    S = select_topk(Q.reshape(n, numel), keff)
    vals = np.take_along_axis(Q.reshape(n, numel), S, axis=1)
    if subtract == "local":
        new_chunks = subtract_selected(chunks, Q, S, alpha, P0, P1)
    elif subtract == "aggregated":
        new_chunks = chunks
    else:
        raise ValueError(subtract)
    M_new = merge_chunks(new_chunks, M.shape, s).astype(F32)
    terms = momentum_update(np.abs(np.asarray(M, dtype=F64)), np.abs(np.asarray(G, dtype=F64)), beta, plain)
    return {
        "M": M_new,
        "values": vals.astype(F32),
        "idx": S.astype(np.uint16),
        "Mp_chunks": chunks,
        "Q": Q,
        "terms_chunks": split_chunks(terms, s),
    }


# ---------------------------------------------------------------------------
# decode / apply: sparse averaging, inverse transform, phi, update
# ---------------------------------------------------------------------------

def aggregate(values: np.ndarray, idx: np.ndarray, numel: int, mode: str = "count") -> np.ndarray:
    """Sparse top-k averaging of W workers' payloads, per chunk.

    [S] Server-Side Aggregation (AvgAllGather, the sparse top-k averaging
    procedure): per coordinate, sum the coefficients of the workers that
    selected it and divide by the count of those workers; coordinates no
    worker selected stay zero.  ``mode="workers"`` divides every sum by W
    instead (the same section's "contributing zero" wording).
    values: float32 [W, n_chunks, keff]; idx: integer [W, n_chunks, keff].
    Returns float64 [n_chunks, numel].
    """
    W, n, keff = values.shape
    total = np.zeros(n * numel, dtype=F64)
    count = np.zeros(n * numel, dtype=F64)
    base = (np.arange(n, dtype=np.int64) * numel)[:, None]
    for w in range(W):
        flat = (base + idx[w].astype(np.int64)).ravel()
        total += np.bincount(flat, weights=values[w].astype(F64).ravel(), minlength=n * numel)
        count += np.bincount(flat, minlength=n * numel)
    if mode == "count":
        out = np.zeros_like(total)
        hit = count > 0
        out[hit] = total[hit] / count[hit]
    elif mode == "workers":
        out = total / float(W)
    else:
        raise ValueError(mode)
    return out.reshape(n, numel)


def phi_muon(M: np.ndarray, eps: float) -> np.ndarray:
    """[S] Base Optimizer Update, Muon: phi(M) = M (M^T M + eps I)^(-1/2) on the whole tensor.

    Computed through the smaller Gram matrix: for a wide M (rows <= cols)
    (M M^T + eps I)^(-1/2) M, which is the same matrix (both equal
    U diag(s / sqrt(s^2 + eps)) V^T for M = U diag(s) V^T).  The inverse
    square root is taken from the symmetric eigendecomposition in float64.  A
    vector is a one-column matrix: m / sqrt(m.m + eps).
    """
    M = np.asarray(M, dtype=F64)
    if M.ndim == 1:
        return M / np.sqrt(M @ M + float(eps))
    wide = M.shape[0] <= M.shape[1]
    G = M @ M.T if wide else M.T @ M
    lam, V = np.linalg.eigh(G + float(eps) * np.eye(G.shape[0]))
    inv_sqrt = (V / np.sqrt(lam)) @ V.T
    return inv_sqrt @ M if wide else M @ inv_sqrt


def phi_map(M: np.ndarray, phi: str, eps: float = 0.0) -> np.ndarray:
    """[S] Base Optimizer Update: phi = sign (Signum), identity (SGD) or Muon; sign(0) = 0."""
    if phi == "sign":
        return np.sign(M)
    if phi == "identity":
        return M
    if phi == "muon":
        return phi_muon(M, eps)
    raise ValueError(phi)


def decode_apply(X: np.ndarray, values: np.ndarray, idx: np.ndarray, *, phi: str, eta: float,
                 lam: float, mode: str = "count", P0: Optional[np.ndarray] = None,
                 P1: Optional[np.ndarray] = None, s: int = 64, eps: float = 0.0) -> Dict[str, np.ndarray]:
    """Aggregate W payloads of one tensor, reconstruct M*, apply phi and the update.

    [S] Server-Side Aggregation and Momentum Reconstruction, Inverse DCT and
    Unchunking: M* = B^-1(T^-1(Q_bar)).  [S] Base Optimizer Update:
    X_{t+1} = X_t - eta * (phi(M*_t) + lambda * X_t), with the pre-update X.
    Returns float32 ``X``, and for the tests the float64 ``Mstar`` (cropped),
    ``Qbar`` [n_chunks, numel], the averaged coefficients, and ``Qabs``, the
    same average taken over the values' magnitudes (the scale of a float32
    evaluation's rounding error).
    """
    P0 = dct_basis(s) if P0 is None else np.asarray(P0, dtype=F64)
    P1 = dct_basis(s) if P1 is None else np.asarray(P1, dtype=F64)
    X = np.asarray(X)
    grid = chunk_grid(X.shape, s)
    numel = s if X.ndim == 1 else s * s
    n = int(np.prod(grid))
    Qbar = aggregate(values, idx, numel, mode)
    Qabs = aggregate(np.abs(np.asarray(values, dtype=F64)), idx, numel, mode)
    cshape = (n, s) if X.ndim == 1 else (n, s, s)
    Mstar = merge_chunks(unproject(Qbar.reshape(cshape), P0, P1), X.shape, s)
    X64 = X.astype(F64)
    X_new = X64 - hp(eta) * (phi_map(Mstar, phi, eps) + hp(lam) * X64)
    return {"X": X_new.astype(F32), "Mstar": Mstar, "Qbar": Qbar, "Qabs": Qabs}


def subtract_aggregated(M: np.ndarray, Mstar: np.ndarray, alpha: float) -> np.ndarray:
    """Momentum subtraction with the aggregated coefficients.

    [S] Momentum Subtraction as Implicit Error Feedback: M <- M - alpha *
    B^-1(T^-1(Q_bar)), Q_bar the server's average, i.e. M - alpha * M* with
    M* from ``decode_apply``.  Returns float32.
    """
    return (np.asarray(M, dtype=F64) - hp(alpha) * np.asarray(Mstar, dtype=F64)).astype(F32)


# ---------------------------------------------------------------------------
# Signum download path: one bit per parameter
# ---------------------------------------------------------------------------

def sign_words(shapes: Sequence[Sequence[int]], s: int = 64) -> int:
    """64-bit words of the packed sign of a tensor list: one bit per element of every (padded) chunk."""
    total = 0
    for shp in shapes:
        numel = s if len(shp) == 1 else s * s
        total += int(np.prod(chunk_grid(shp, s))) * (numel // 64)
    return total


def pack_signs(Mstar: np.ndarray, s: int = 64) -> np.ndarray:
    """The download of the Signum variant: sign(M*) as one bit per parameter.

    [S] Base Optimizer Update: with phi = sign the server broadcasts only the
    sign of the reconstructed momentum, one bit per parameter.  Layout (the
    pages fix none): chunk after chunk in chunk order; inside a chunk the
    elements in row-major order, 64 to a little-endian uint64 word (bit j of a
    word is the j-th of its 64 elements).  A bit is set where M* < 0.  One bit
    cannot carry sign(0) = 0: a zero reads as +1.  Padding positions hold 0.
    Returns uint64 words.
    """
    chunks = split_chunks(np.asarray(Mstar, dtype=F64), s)
    bits = (chunks < 0.0).reshape(-1, 64)
    return np.packbits(bits, axis=1, bitorder="little").view("<u8").reshape(-1).astype(np.uint64)


def apply_signs(X: np.ndarray, words: np.ndarray, *, eta: float, lam: float, s: int = 64) -> np.ndarray:
    """Worker side of the download: X <- X - eta * (phi + lambda * X), phi = -1 where
    the bit is set, else +1 ([S] Base Optimizer Update).  Returns float32."""
    X = np.asarray(X)
    grid = chunk_grid(X.shape, s)
    cshape = (int(np.prod(grid)), s) if X.ndim == 1 else (int(np.prod(grid)), s, s)
    by = np.ascontiguousarray(np.asarray(words, dtype="<u8")).view(np.uint8).reshape(-1, 8)
    bits = np.unpackbits(by, axis=1, bitorder="little").reshape(cshape)
    phi = merge_chunks(np.where(bits != 0, -1.0, 1.0), X.shape, s)
    X64 = X.astype(F64)
    return (X64 - hp(eta) * (phi + hp(lam) * X64)).astype(F32)


# ---------------------------------------------------------------------------
# compact wire format: bfloat16 values, 12- or 14-bit positions
# ---------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, rounding to nearest with ties to even (finite inputs)."""
    b = np.ascontiguousarray(np.asarray(x, dtype=F32)).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def wire_index_bits(s: int = 64) -> int:
    """Bits of one chunk position on the wire: enough for the s*s positions of a
    matrix chunk (12 at s = 64, 14 at s = 128)."""
    return int(s * s - 1).bit_length()


def pack_wire(values: np.ndarray, idx: np.ndarray, s: int = 64) -> Tuple[np.ndarray, np.ndarray]:
    """A worker's payload as sent: [T] ("Training over Slow Links", top-k and DeMo
    slides) counts a kept value as 2 bytes of bfloat16 plus its position.
    Values become bfloat16 (uint16 bits, entry order kept).  Positions take
    b = wire_index_bits(s) bits each (12 at s = 64: a 64x64 chunk has 4096
    positions; 14 at s = 128): entry j's position fills bits b*j .. b*j + b - 1
    of one little-endian bit string (bit t of the string is bit t mod 8 of byte
    t // 8), cut to whole bytes.  Returns (uint16 values, uint8 index bytes)."""
    b = wire_index_bits(s)
    v = bf16_bits(np.asarray(values, dtype=F32).ravel())
    i = np.asarray(idx).ravel().astype(np.uint32)
    if np.any(i >= (1 << b)):
        raise ValueError(f"{b}-bit indices")
    bits = ((i[:, None] >> np.arange(b, dtype=np.uint32)[None, :]) & 1).astype(np.uint8).ravel()
    pad = (-bits.size) % 8
    bits = np.concatenate([bits, np.zeros(pad, np.uint8)])
    return v, np.packbits(bits, bitorder="little")


def unpack_wire(wv: np.ndarray, wi: np.ndarray, n: int, s: int = 64) -> Tuple[np.ndarray, np.ndarray]:
    """Inverse of pack_wire for n entries: float32 values (bfloat16 widened) and indices."""
    b = wire_index_bits(s)
    vals = (np.asarray(wv, dtype=np.uint16)[:n].astype(np.uint32) << 16).view(F32)
    bits = np.unpackbits(np.asarray(wi, dtype=np.uint8), bitorder="little")[:n * b].reshape(n, b).astype(np.uint32)
    idx = (bits << np.arange(b, dtype=np.uint32)[None, :]).sum(axis=1).astype(np.uint16)
    return vals, idx


# ---------------------------------------------------------------------------
# payload accounting
# ---------------------------------------------------------------------------

def payload_entries(shapes: Sequence[Sequence[int]], k: int, s: int = 64) -> int:
    """(value, index) pairs one worker sends for a tensor list: sum over chunks of keff.

    [S] Top-k Sparsification: a block of prod(s_i) elements is sent as k
    coefficients, a compression of prod(s_i) / k per chunk.
    """
    total = 0
    for shp in shapes:
        numel = s if len(shp) == 1 else s * s
        total += int(np.prod(chunk_grid(shp, s))) * k_effective(k, numel)
    return total
