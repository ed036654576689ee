"""Number formats used by the ResidualQuant CPU oracle: FP8 E4M3FN and BF16.

TEST INFRASTRUCTURE ONLY.  Nothing under ``oracle/`` is part of the product:
only ``tests/``, the package's ``smoke()`` check and the benchmark's CPU
baseline leg may import it.  It shares no code with the HIP path.

Everything here is derived from the format definitions, in float64:

* FP8 E4M3FN (OCP 8-bit floating point, the "e4m3" flavour without
  infinities): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent field 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; largest
  finite magnitude 448.  The arXiv digest (Figure 1 caption and main-result
  paragraph) and the explainer's worked example say each quantization group
  stores an FP8 scale and offset; this is the FP8 flavour used for them.
* BF16: 1 sign, 8 exponent bits (fp32 range), 7 stored mantissa bits.  The
  explainer's method paragraph and the digest say the per-vector least-squares
  coefficient is stored in BF16.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_SUBNORMAL = 2.0 ** -9


def _e4m3_byte_value(byte: int) -> float:
    sign = -1.0 if byte & 0x80 else 1.0
    exp = (byte >> 3) & 0xF
    man = byte & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9            # (man/8) * 2^(1-7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


#: value of each of the 256 bit patterns (NaN for 0x7F and 0xFF)
E4M3_TABLE = np.array([_e4m3_byte_value(b) for b in range(256)], dtype=np.float64)

#: the 253 distinct finite values, ascending (+0 and -0 are one value)
E4M3_GRID = np.unique(E4M3_TABLE[np.isfinite(E4M3_TABLE)])

#: positive finite values, ascending (smallest is 2^-9)
E4M3_POSITIVE = E4M3_GRID[E4M3_GRID > 0]


def e4m3_decode(codes) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.int64)]


def e4m3_floor(v) -> np.ndarray:
    """Largest E4M3 value <= v (v must be >= -448)."""
    v = np.asarray(v, dtype=np.float64)
    idx = np.searchsorted(E4M3_GRID, v, side="right") - 1
    if np.any(idx < 0) or np.any(~np.isfinite(v)):
        raise ValueError("value below the FP8 E4M3 range or not finite")
    return E4M3_GRID[idx]


def e4m3_ceil(v) -> np.ndarray:
    """Smallest E4M3 value >= v (v must be <= 448)."""
    v = np.asarray(v, dtype=np.float64)
    idx = np.searchsorted(E4M3_GRID, v, side="left")
    if np.any(idx >= E4M3_GRID.size) or np.any(~np.isfinite(v)):
        raise ValueError("value above the FP8 E4M3 range or not finite")
    return E4M3_GRID[idx]


def e4m3_encode(v) -> np.ndarray:
    """Bit pattern of values that lie on the E4M3 grid (zero is encoded as +0, 0x00)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint8)
    # positive patterns 0x00..0x7E are ascending in value; negative ones mirror them
    pos_codes = np.arange(0x7F)
    pos_vals = E4M3_TABLE[pos_codes]
    mag = np.abs(v)
    idx = np.searchsorted(pos_vals, mag)
    if np.any(idx >= pos_vals.size) or np.any(pos_vals[np.minimum(idx, 0x7E)] != mag):
        raise ValueError("value is not on the FP8 E4M3 grid")
    out[...] = pos_codes[idx]
    neg = (v < 0)
    out[neg] |= 0x80
    return out


def bf16_round(v) -> np.ndarray:
    """Round float64 values to the nearest BF16 value, ties to even, in one step
    (no intermediate rounding to float32)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = (v != 0) & np.isfinite(v)
    _, e = np.frexp(v[nz])                 # |v| in [2^(e-1), 2^e)
    exp = np.maximum(e - 1, -126)          # below 2^-126 the BF16 quantum stays 2^-133
    quantum = np.ldexp(1.0, exp - 7)
    r = np.rint(v[nz] / quantum) * quantum
    if np.any(np.abs(r) >= 2.0 ** 128):
        raise ValueError("value overflows BF16")
    out[nz] = r
    out[~np.isfinite(v)] = v[~np.isfinite(v)]
    return out


def bf16_bits(v) -> np.ndarray:
    """Bit pattern of values that are exactly representable in BF16."""
    v = np.asarray(v, dtype=np.float64)
    f = v.astype(np.float32)
    if np.any(f.astype(np.float64) != v):
        raise ValueError("value is not a BF16 value")
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value is not a BF16 value")
    return (u >> 16).astype(np.uint16)


def bf16_from_bits(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint32) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)
