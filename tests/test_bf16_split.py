"""The three-way bfloat16 split behind the matrix-core products (caller basis,
Muon), checked as arithmetic on the CPU.

Both kernels round a float32 value x to bfloat16 (nearest, ties to even), take
what is left in float32, round that again, and keep the last remainder as the
third part.  The claims the kernels rest on:
  * x = h1 + h2 + h3 exactly, and h3 is itself a bfloat16 value, for every
    finite float32 x in the normal range;
  * of the nine part products of a * b, the three dropped ones (a2 b3, a3 b2,
    a3 b3) are each at most 2^-24 |a b|, so a 64-term dot product built from
    the other six, summed in float32, stays as close to the exact result as
    a plain float32 dot product.
numpy has no bfloat16, so the rounding is done on the bit pattern; the
emulation is checked against its own definition (a bfloat16 value is a
float32 whose low 16 bits are zero, and it is the nearest such value).
"""
import numpy as np
import pytest


def rne_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def split3(x: np.ndarray):
    x = np.asarray(x, dtype=np.float32)
    h1 = rne_bf16(x)
    r1 = (x - h1).astype(np.float32)
    h2 = rne_bf16(r1)
    r2 = (r1 - h2).astype(np.float32)
    h3 = rne_bf16(r2)
    return h1, h2, h3, r2


def samples(n, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * np.exp2(rng.integers(-60, 60, n))).astype(np.float32)
    edge = np.array([1.0, -1.0, 1.0 + 2.0 ** -23, 1.0 - 2.0 ** -24, 3.0, 0.1, -0.7,
                     np.float32(2.0 ** -100), np.float32(1.5 * 2.0 ** 100)], np.float32)
    # every float32 whose low 16 bits sit exactly on a bfloat16 tie
    ties = ((rng.integers(0x00800000 >> 16, 0x7F000000 >> 16, 64).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    return np.concatenate([x, edge, ties, -ties])


def test_rne_bf16_is_the_nearest_bfloat16():
    x = samples(20000, 1)
    h = rne_bf16(x)
    assert np.all(h.view(np.uint32) & 0xFFFF == 0)
    b = x.view(np.uint32)
    lo = (b & 0xFFFF0000).view(np.float32)                 # truncation toward zero
    hi = ((b & 0xFFFF0000) + 0x10000).view(np.float32)      # next bfloat16 away from zero
    d = np.abs(x.astype(np.float64) - h.astype(np.float64))
    assert np.all(d <= np.abs(x.astype(np.float64) - lo.astype(np.float64)))
    assert np.all(d <= np.abs(x.astype(np.float64) - hi.astype(np.float64)))
    # ties go to the even significand
    t = (b & 0xFFFF) == 0x8000
    assert np.all((h.view(np.uint32)[t] >> 16) & 1 == 0)


def test_split_is_exact_and_third_part_is_bfloat16():
    x = samples(50000, 2)
    h1, h2, h3, r2 = split3(x)
    assert np.array_equal(h3, r2), "the last remainder is already a bfloat16 value"
    total = h1.astype(np.float64) + h2.astype(np.float64) + h3.astype(np.float64)
    assert np.array_equal(total, x.astype(np.float64))
    ax = np.abs(x.astype(np.float64))
    assert np.all(np.abs(h2) <= ax * 2.0 ** -8)
    assert np.all(np.abs(h3) <= ax * 2.0 ** -16)


def test_dropped_part_products_are_below_float32_rounding():
    a = samples(20000, 3)
    b = samples(20000, 4)[: a.size]
    a1, a2, a3, _ = split3(a)
    b1, b2, b3, _ = split3(b)
    ab = np.abs(a.astype(np.float64) * b.astype(np.float64))
    for p, q in ((a2, b3), (a3, b2), (a3, b3)):
        assert np.all(np.abs(p.astype(np.float64) * q.astype(np.float64)) <= ab * 2.0 ** -24)


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_six_term_dot_product_matches_float32(seed):
    """64-term dot products as a 32x32x16 tile accumulates them: per 16-k step
    the six part products in the kernels' order, each bfloat16 x bfloat16
    product exact in float32, summed in float32."""
    rng = np.random.default_rng(seed)
    n = 4000
    A = rng.standard_normal((n, 64)).astype(np.float32)
    B = (rng.standard_normal((n, 64)) * 1e-3).astype(np.float32)
    exact = np.sum(A.astype(np.float64) * B.astype(np.float64), axis=1)
    a = split3(A)[:3]
    b = split3(B)[:3]
    order = [(2, 0), (1, 1), (0, 2), (1, 0), (0, 1), (0, 0)]
    acc = np.zeros(n, np.float32)
    for s in range(4):
        ks = slice(16 * s, 16 * s + 16)
        for pa, pb in order:
            prod = (a[pa][:, ks].astype(np.float64) * b[pb][:, ks].astype(np.float64)).sum(axis=1)
            acc = (acc + prod.astype(np.float32)).astype(np.float32)
    plain = np.zeros(n, np.float32)
    for k in range(64):
        plain = (plain + A[:, k] * B[:, k]).astype(np.float32)
    scale = np.sum(np.abs(A.astype(np.float64) * B.astype(np.float64)), axis=1)
    err_split = np.abs(acc - exact) / scale
    err_plain = np.abs(plain - exact) / scale
    assert err_split.max() <= 2.0 ** -20
    assert err_split.max() <= 4 * err_plain.max()
