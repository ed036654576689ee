"""Pins of the K/V projection oracle (oracle/projection.py) against exact rational
arithmetic, closed forms and hand-built rounding ties, independent of numpy's matmul."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import projection as P


def _bf16_values(rng, shape, scale=1.0):
    return F.bf16_round(rng.normal(0.0, scale, shape))


def _exact_bf16_rne(v: Fraction) -> Fraction:
    """Round an exact rational to BF16 (8 significant bits), ties to even, by integer
    arithmetic on the scaled value (normal range only)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = 0                                   # 2^e <= a < 2^(e+1)
    while a >= 2 ** (e + 1):
        e += 1
    while a < 2 ** e:
        e -= 1
    quantum = Fraction(2) ** (e - 7)
    q, rem = divmod(a, quantum)             # q integer part, rem in [0, quantum)
    q = int(q)
    if rem * 2 > quantum or (rem * 2 == quantum and q % 2 == 1):
        q += 1
    return sign * q * quantum


def _brute(x, w):
    """K/V by Python loops over exact rationals: [2][B][Hkv][d] exact and rounded."""
    two, hkv, d, hidden = w.shape
    B = x.shape[0]
    exact = np.zeros((2, B, hkv, d))
    rounded = np.zeros((2, B, hkv, d))
    for xx in range(2):
        for b in range(B):
            for h in range(hkv):
                for i in range(d):
                    s = Fraction(0)
                    for c in range(hidden):
                        s += Fraction(float(x[b, c])) * Fraction(float(w[xx, h, i, c]))
                    exact[xx, b, h, i] = float(s)
                    rounded[xx, b, h, i] = float(_exact_bf16_rne(s))
    return exact, rounded


def test_projection_matches_exact_rational_brute_force():
    rng = np.random.default_rng(11)
    x = _bf16_values(rng, (3, 24))
    w = _bf16_values(rng, (2, 2, 5, 24), 0.2)
    exact, rounded = P.kv_projection(x, w)
    want_exact, want_rounded = _brute(x, w)
    assert np.allclose(exact, want_exact, rtol=1e-14, atol=1e-300)
    assert np.array_equal(rounded, want_rounded)
    # K rows and V rows land in their own halves of the result
    assert not np.array_equal(rounded[0], rounded[1])


def test_one_hot_weights_select_channels_exactly():
    rng = np.random.default_rng(3)
    B, hkv, d, hidden = 4, 2, 8, 64
    x = _bf16_values(rng, (B, hidden), 3.0)
    sel = rng.integers(0, hidden, size=(2, hkv, d))
    w = np.zeros((2, hkv, d, hidden))
    for xx in range(2):
        for h in range(hkv):
            for i in range(d):
                w[xx, h, i, sel[xx, h, i]] = 1.0
    exact, rounded = P.kv_projection(x, w)
    for xx in range(2):
        for h in range(hkv):
            for i in range(d):
                assert np.array_equal(rounded[xx, :, h, i], x[:, sel[xx, h, i]])
                assert np.array_equal(exact[xx, :, h, i], x[:, sel[xx, h, i]])


@pytest.mark.parametrize("terms,want", [
    ((1.0, 2.0 ** -8), 1.0),                                  # midpoint, even neighbour below
    ((1.0 + 2.0 ** -7, 2.0 ** -8), 1.0 + 2.0 ** -6),          # midpoint, odd neighbour below: up
    ((-1.0, -(2.0 ** -8)), -1.0),                             # negative midpoint: to even
    ((1.0, 2.0 ** -8, 2.0 ** -30), 1.0 + 2.0 ** -7),          # just past the midpoint: up
    ((3.0, -(2.0 ** -7)), 3.0),                               # 3 - 2^-7: midpoint of 2.984375 and 3
])
def test_rounding_ties_to_even(terms, want):
    x = np.array([list(terms)])
    w = np.ones((2, 1, 1, len(terms)))
    exact, rounded = P.kv_projection(x, w)
    assert rounded[0, 0, 0, 0] == want and rounded[1, 0, 0, 0] == want
    assert float(_exact_bf16_rne(sum(Fraction(t) for t in terms))) == want


def test_magnitude_sums_bound_the_result():
    rng = np.random.default_rng(5)
    x = _bf16_values(rng, (2, 96))
    w = _bf16_values(rng, (2, 3, 4, 96), 0.1)
    exact, _ = P.kv_projection(x, w)
    mags = P.magnitude_sums(x, w)
    assert np.all(mags >= np.abs(exact) - 1e-12)
    # equality for non-negative operands
    ex2, _ = P.kv_projection(np.abs(x), np.abs(w))
    assert np.allclose(P.magnitude_sums(np.abs(x), np.abs(w)), ex2, rtol=1e-15)


def test_write_pending_touches_only_its_slot():
    rng = np.random.default_rng(9)
    B, L, hkv, d = 3, 4, 2, 8
    pending = rng.normal(size=(B, L, 2, hkv, d))
    before = pending.copy()
    kv = rng.normal(size=(2, B, hkv, d))
    P.write_pending(pending, kv, 2)
    assert np.array_equal(pending[:, 2, 0], kv[0]) and np.array_equal(pending[:, 2, 1], kv[1])
    mask = np.ones(L, bool)
    mask[2] = False
    assert np.array_equal(pending[:, mask], before[:, mask])
