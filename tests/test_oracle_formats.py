"""Pins of the oracle's FP8 E4M3FN and BF16 codecs against torch's own dtypes,
exhaustive search and hand-built rounding cases."""
import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e4m3_table_matches_torch_float8_e4m3fn():
    raw = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.E4M3_TABLE
    assert np.array_equal(np.isnan(raw), np.isnan(ours))
    fin = ~np.isnan(raw)
    assert np.array_equal(raw[fin], ours[fin])
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


def test_e4m3_grid_shape():
    assert F.E4M3_GRID.size == 253
    assert F.E4M3_GRID.max() == 448.0 and F.E4M3_GRID.min() == -448.0
    assert F.E4M3_POSITIVE[0] == 2.0 ** -9
    assert F.E4M3_POSITIVE.size == 126


def _brute_floor(v):
    cands = [g for g in F.E4M3_GRID if g <= v]
    return max(cands)


def _brute_ceil(v):
    cands = [g for g in F.E4M3_GRID if g >= v]
    return min(cands)


def test_floor_ceil_against_exhaustive_search():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.normal(0, 3, 400), rng.normal(0, 0.01, 200), rng.uniform(-448, 448, 100),
        F.E4M3_GRID, (F.E4M3_GRID[1:] + F.E4M3_GRID[:-1]) / 2, [0.0, -0.0, 1e-30, -1e-30],
    ])
    fl = F.e4m3_floor(vals)
    ce = F.e4m3_ceil(vals)
    for v, a, b in zip(vals, fl, ce):
        assert a == _brute_floor(v)
        assert b == _brute_ceil(v)


def test_floor_out_of_range_raises():
    with pytest.raises(ValueError):
        F.e4m3_floor(-449.0)
    with pytest.raises(ValueError):
        F.e4m3_ceil(449.0)


def test_e4m3_encode_roundtrip():
    for byte in range(256):
        v = F.E4M3_TABLE[byte]
        if np.isnan(v):
            continue
        enc = int(F.e4m3_encode(v))
        expect = 0 if byte == 0x80 else byte      # -0 is stored as +0
        assert enc == expect, (byte, v, enc)
    with pytest.raises(ValueError):
        F.e4m3_encode(0.3)


def test_bf16_round_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(2)
    x32 = np.concatenate([rng.normal(0, 1, 5000), rng.normal(0, 1e-3, 1000), rng.normal(0, 1e4, 1000)]
                         ).astype(np.float32)
    # exact ties between two BF16 neighbours: low 16 bits = 0x8000
    ties = (rng.integers(0x3F000000, 0x40000000, 500, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    x32 = np.concatenate([x32, ties.view(np.float32)])
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    ours = F.bf16_round(x32.astype(np.float64))
    assert np.array_equal(ref, ours)


def test_bf16_round_is_single_rounding_from_float64():
    # 1 + 2^-8 + 2^-30: just above the midpoint between 1 and 1 + 2^-7.  Rounding once gives
    # 1 + 2^-7; going through float32 first would land on the midpoint and then on 1.
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert F.bf16_round(v) == 1.0 + 2.0 ** -7
    # exact midpoints go to the even neighbour
    assert F.bf16_round(1.0 + 2.0 ** -8) == 1.0
    assert F.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2 * 2.0 ** -7
    assert F.bf16_round(-(1.0 + 3 * 2.0 ** -8)) == -(1.0 + 2 * 2.0 ** -7)


def test_bf16_bits_roundtrip():
    rng = np.random.default_rng(3)
    v = F.bf16_round(rng.normal(0, 2, 1000))
    assert np.array_equal(F.bf16_from_bits(F.bf16_bits(v)), v)
    t = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(t, F.bf16_bits(v))
