"""Pins of the oracle's group quantizer: invariants, exhaustive search on tiny groups,
hand-built exact ties and the degenerate group."""
import numpy as np
import pytest

from oracle import formats as F
from oracle import residualquant as RQ


def _bf16_normal(rng, shape, outliers=0):
    x = rng.normal(0, 1, shape)
    if outliers:
        x[..., rng.choice(shape[-1], outliers, replace=False)] *= 8
    return F.bf16_round(x)


@pytest.mark.parametrize("bits,group", [(4, 32), (2, 32), (2, 16), (4, 16)])
def test_quantizer_invariants(bits, group):
    rng = np.random.default_rng(10 + bits + group)
    x = np.concatenate([_bf16_normal(rng, (300, 128), outliers=4),
                        rng.normal(0, 0.3, (300, 128))])          # bf16 keys and float residual-like rows
    q, z, s = RQ.quantize(x, bits, group)
    n = 2 ** bits - 1
    xg = x.reshape(x.shape[0], -1, group)
    qg = q.reshape(xg.shape)
    assert q.min() >= 0 and q.max() <= n
    lo, hi = xg.min(-1), xg.max(-1)
    assert np.all(z <= lo)
    # z is the largest E4M3 value <= lo: the next grid value is above lo
    nxt = F.E4M3_GRID[np.searchsorted(F.E4M3_GRID, z, side="right")]
    assert np.all(nxt > lo)
    assert np.all(z + n * s >= hi)
    # minimality of s: the previous positive grid value no longer covers the maximum
    idx = np.searchsorted(F.E4M3_POSITIVE, s)
    prev_ok = idx > 0
    prev = F.E4M3_POSITIVE[np.maximum(idx - 1, 0)]
    assert np.all(~prev_ok | (z + n * prev < hi))
    # per-element error bound s/2
    xhat = RQ.dequantize(q, z, s, group).reshape(xg.shape)
    assert np.all(np.abs(xg - xhat) <= s[..., None] / 2)
    # z and s are on the grid
    F.e4m3_encode(z)
    F.e4m3_encode(s)


def _brute_quantize_group(x, bits):
    n = 2 ** bits - 1
    lo, hi = min(x), max(x)
    z = max(v for v in F.E4M3_GRID if v <= lo)
    s = min(v for v in F.E4M3_GRID if v > 0 and z + n * v >= hi)
    codes = []
    for xi in x:
        # nearest level, ties to the even code, by scanning every code
        best = None
        for k in range(n + 1):
            err = abs(xi - (z + k * s))
            if best is None or err < best[0] or (err == best[0] and k % 2 == 0):
                best = (err, k)
        codes.append(best[1])
    return codes, z, s


def test_quantizer_matches_exhaustive_search_on_small_groups():
    rng = np.random.default_rng(11)
    for trial in range(300):
        bits = (2, 4)[trial % 2]
        scale = (0.01, 1.0, 20.0)[trial % 3]
        x = F.bf16_round(rng.normal(0, scale, 4))
        q, z, s = RQ.quantize(x[None, :], bits, 4)
        bq, bz, bs = _brute_quantize_group(list(x), bits)
        assert z[0, 0] == bz and s[0, 0] == bs
        assert list(q[0]) == bq, (x, q, bq)


def test_exact_ties_round_to_even_code():
    # group with min exactly on the grid and max exactly covered: z = -1, s = 0.125 at INT4
    z, s = -1.0, 0.125
    base = np.array([z, z + 15 * s] + [z + (k + 0.5) * s for k in range(14)] + [z] * 16)
    q, zz, ss = RQ.quantize(base[None, :], 4, 32)
    assert zz[0, 0] == z and ss[0, 0] == s
    assert q[0, 0] == 0 and q[0, 1] == 15
    for k in range(14):
        tie = q[0, 2 + k]
        assert tie in (k, k + 1) and tie % 2 == 0


def test_ties_are_common_with_bf16_inputs():
    # exact ties decide about 1% of INT4 codes for BF16 keys, so the tie rule matters
    rng = np.random.default_rng(12)
    x = _bf16_normal(rng, (4000, 128), outliers=4)
    q, z, s = RQ.quantize(x, 4, 32)
    t = (x.reshape(4000, 4, 32) - z[..., None]) / s[..., None]
    frac = np.mean(t - np.floor(t) == 0.5)
    assert 0.002 < frac < 0.05


def test_degenerate_group_uses_smallest_scale():
    # constant group off the FP8 grid: z rounds down, s is the smallest value covering the gap
    x = np.full((1, 32), 0.3)
    q, z, s = RQ.quantize(x, 2, 32)
    assert z[0, 0] == 0.28125 and s[0, 0] == 0.0078125     # 0.28125 + 3 * 2^-7 >= 0.3 > 0.28125 + 3 * 0.005859375
    assert np.all(np.abs(RQ.dequantize(q, z, s, 32) - 0.3) <= s[0, 0] / 2)
    # constant group on the grid (all-zero residual included): smallest scale, codes 0, exact
    for v in (0.0, 0.3125, -2.0):
        q, z, s = RQ.quantize(np.full((1, 32), v), 2, 32)
        assert z[0, 0] == v and s[0, 0] == 2.0 ** -9 and np.all(q == 0)
        assert np.all(RQ.dequantize(q, z, s, 32) == v)
