"""W4A4 linear layer of a looped block with cross-loop residual activations: CPU oracle.

TEST INFRASTRUCTURE ONLY.  Nothing under ``oracle/`` is part of the product: only
``tests/``, the package's ``smoke()`` check and the benchmark's CPU baseline leg may
import it.  It shares no code with the HIP path and never takes an input or an
expected value from it.

Source: the arXiv digest (ai4snews), scope paragraph after the results ("适用场景"
paragraph: besides KV quantization the authors apply the same residual-reconstruction
principle to W4A4 activation quantization) and the caveats paragraph after it (the
activation-quantization protocol differs from the KV one).  The pages name the
transfer and nothing else; the method here is the KV method's steps applied to the
input activations of a linear layer that the looped block runs at every loop:

* weights: 4-bit codes with the KV anchor's group quantizer (groups of 32 consecutive
  input channels of one output row, FP8-E4M3 offset rounded down, smallest covering
  E4M3 scale, codes rounded half-to-even);
* activations of the anchor loop: the same 4-bit group quantizer, ``a_hat``;
* activations of every other loop of the group: least-squares coefficient
  ``c = <x, a_hat> / <a_hat, a_hat>`` rounded to BF16, residual ``x - c a_hat`` turned by
  a fixed orthogonal rotation (one 128 x 128 matrix applied to every block of 128
  input channels), 4-bit group quantizer on the rotated residual, ``r_hat``;
* output: ``y = W_hat a_hat`` at the anchor loop and
  ``y = c (W_hat a_hat) + W_R_hat r_hat`` at the others, where ``W_R_hat`` is the
  4-bit quantization of ``W R^T`` (the rotation folded into a second copy of the
  weights), so ``W_R r = W x`` before quantization and the anchor product is
  computed once per token and reused by every loop of the group.

Readings adopted where the pages are silent (each listed in the design notes):
the anchor is the *first* loop of each group, because at decode time a linear layer
of an earlier loop runs before any later loop's activation exists (the KV method can
take the last loop only because the cache is read by later tokens); the residual is
4-bit like the anchor (W4A4 names 4-bit activations); the rotation acts on blocks of
128 channels (the head size of the KV method's rotation).

Plain float64 numpy, one formula per step.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .residualquant import dequantize, ls_coefficient, quantize

GROUP = 32          # input channels per quantization group
ROT_BLOCK = 128     # input channels per rotation block
BITS = 4            # weight and activation code width
TILE_N = 16         # output rows per weight tile
QUAD = 4            # groups per weight tile column block

Quantized = Tuple[np.ndarray, np.ndarray, np.ndarray]     # codes, offsets z, scales s


def rotate_blocks(v: np.ndarray, rot: np.ndarray) -> np.ndarray:
    """R v for every block of 128 consecutive channels of the last axis."""
    v = np.asarray(v, dtype=np.float64)
    k = v.shape[-1]
    assert k % ROT_BLOCK == 0 and rot.shape == (ROT_BLOCK, ROT_BLOCK)
    vb = v.reshape(v.shape[:-1] + (k // ROT_BLOCK, ROT_BLOCK))
    return (vb @ np.asarray(rot, np.float64).T).reshape(v.shape)     # [.., b, j] = sum_i v[.., b, i] R[j, i]


def rotate_weights(w: np.ndarray, rot: np.ndarray) -> np.ndarray:
    """W R^T blockwise: (W R^T)[n, 128 b + j] = sum_i W[n, 128 b + i] R[j, i], so that
    (W R^T)(R x) = W x for the block-diagonal R."""
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    wb = w.reshape(n, k // ROT_BLOCK, ROT_BLOCK)
    return (wb @ np.asarray(rot, np.float64).T).reshape(n, k)        # [n, b, j] = sum_i W[n, b, i] R[j, i]


def quantize_weights(w: np.ndarray, rot: Optional[np.ndarray] = None) -> Quantized:
    """4-bit group quantization of W (rot None) or of W R^T."""
    w = np.asarray(w, dtype=np.float64)
    return quantize(w if rot is None else rotate_weights(w, rot), BITS, GROUP)


def dequant(q: Quantized) -> np.ndarray:
    codes, z, s = q
    return dequantize(codes, z, s, GROUP)


def anchor_activation(x: np.ndarray) -> Quantized:
    """The anchor loop's activations x [M][K]: 4-bit group quantization."""
    return quantize(np.asarray(x, np.float64), BITS, GROUP)


def residual_activation(x: np.ndarray, anchor: Quantized, rot: np.ndarray,
                        c_override: Optional[np.ndarray] = None) -> Tuple[np.ndarray, Quantized]:
    """A later loop's activations x [M][K] against the anchor: c (BF16 value per token),
    r = R (x - c a_hat) per 128-channel block, and its 4-bit group quantization.
    ``c_override`` replaces c (to judge a device's residual codes with the device's c)."""
    a_hat = dequant(anchor)
    c, _ = ls_coefficient(np.asarray(x, np.float64), a_hat)
    if c_override is not None:
        c = np.asarray(c_override, np.float64)
    r = rotate_blocks(np.asarray(x, np.float64) - c[..., None] * a_hat, rot)
    return c, quantize(r, BITS, GROUP)


def linear(wq: Quantized, act: Quantized) -> np.ndarray:
    """y[m][n] = sum_k W_hat[n][k] x_hat[m][k] (float64)."""
    return dequant(act) @ dequant(wq).T


def looped_linear(xs: np.ndarray, w: np.ndarray, rot: np.ndarray):
    """One group of loops: xs [L][M][K] activations of loops 0..L-1 (loop 0 the anchor).
    Returns the outputs y [L][M][N], the coefficients c [L][M] (1 at the anchor loop)
    and the quantized activations of every loop."""
    wq, wrq = quantize_weights(w), quantize_weights(w, rot)
    a = anchor_activation(xs[0])
    y0 = linear(wq, a)
    ys, cs, acts = [y0], [np.ones(xs.shape[1])], [a]
    for l in range(1, xs.shape[0]):
        c, r = residual_activation(xs[l], a, rot)
        ys.append(c[:, None] * y0 + linear(wrq, r))
        cs.append(c)
        acts.append(r)
    return np.stack(ys), np.stack(cs), acts


# ---------------------------------------------------------------------------
# byte layouts
# ---------------------------------------------------------------------------

def weight_bytes(n: int, k: int) -> int:
    """Packed size of an N x K weight matrix: 4-bit codes plus 2 metadata bytes per group."""
    return n * k // 2 + n * (k // GROUP) * 2


def write_weights(q: Quantized) -> np.ndarray:
    """Tile layout.  Rows in tiles of 16, groups in quads of 4; per (row tile, group quad)
    a block of 1024 code bytes then 128 metadata bytes, blocks ordered by row tile, then
    quad.  In the code block, the 16 bytes of slot (i = row in the tile, kg = quarter of
    the group) start at byte 16 (16 kg + i); inside them,
    bytes 4 j .. 4 j + 3 hold group 4 quad + j, channels 8 kg .. 8 kg + 7, channel
    8 kg + e in bits 4 e .. 4 e + 3 of the little-endian word.  Metadata: 2 bytes per
    (row i, group j) at 2 (4 i + j): offset byte, then scale byte."""
    codes, z, s = q
    n, k = codes.shape
    assert n % TILE_N == 0 and k % (GROUP * QUAD) == 0
    from .formats import e4m3_encode
    zb, sb = e4m3_encode(z), e4m3_encode(s)
    out = np.zeros(weight_bytes(n, k), np.uint8)
    nq = k // (GROUP * QUAD)
    blk = 1024 + 128
    for t in range(n // TILE_N):
        for qd in range(nq):
            base = (t * nq + qd) * blk
            for i in range(TILE_N):
                row = t * TILE_N + i
                for j in range(QUAD):
                    g = qd * QUAD + j
                    for kg in range(4):
                        word = 0
                        for e in range(8):
                            word |= int(codes[row, g * GROUP + 8 * kg + e]) << (4 * e)
                        off = base + 16 * (16 * kg + i) + 4 * j
                        out[off:off + 4] = np.frombuffer(np.uint32(word).tobytes(), np.uint8)
                    out[base + 1024 + 2 * (4 * i + j)] = zb[row, g]
                    out[base + 1024 + 2 * (4 * i + j) + 1] = sb[row, g]
    return out


def read_weights(buf: np.ndarray, n: int, k: int) -> Quantized:
    """Inverse of write_weights (the oracle's own unpacker, used on device bytes too)."""
    from .formats import e4m3_decode
    buf = np.asarray(buf, np.uint8)
    codes = np.zeros((n, k), np.int64)
    zb = np.zeros((n, k // GROUP), np.uint8)
    sb = np.zeros((n, k // GROUP), np.uint8)
    nq = k // (GROUP * QUAD)
    blk = 1024 + 128
    for t in range(n // TILE_N):
        for qd in range(nq):
            base = (t * nq + qd) * blk
            for i in range(TILE_N):
                row = t * TILE_N + i
                for j in range(QUAD):
                    g = qd * QUAD + j
                    for kg in range(4):
                        off = base + 16 * (16 * kg + i) + 4 * j
                        word = int(np.frombuffer(buf[off:off + 4].tobytes(), np.uint32)[0])
                        for e in range(8):
                            codes[row, g * GROUP + 8 * kg + e] = (word >> (4 * e)) & 15
                    zb[row, g] = buf[base + 1024 + 2 * (4 * i + j)]
                    sb[row, g] = buf[base + 1024 + 2 * (4 * i + j) + 1]
    return codes, e4m3_decode(zb), e4m3_decode(sb)


def act_bytes(m: int, k: int) -> int:
    """Packed size of M quantized activation vectors (one row per token)."""
    return m * (k // 2 + (k // GROUP) * 2)


def write_act(q: Quantized) -> np.ndarray:
    """One row per token: K/2 code bytes (channel 2 i in the low nibble of byte i,
    channel 2 i + 1 in the high nibble), then 2 bytes per group (offset, scale)."""
    from .formats import e4m3_encode
    codes, z, s = q
    m, k = codes.shape
    row = k // 2 + (k // GROUP) * 2
    out = np.zeros(m * row, np.uint8)
    zb, sb = e4m3_encode(z), e4m3_encode(s)
    for t in range(m):
        base = t * row
        for i in range(k // 2):
            out[base + i] = int(codes[t, 2 * i]) | (int(codes[t, 2 * i + 1]) << 4)
        for g in range(k // GROUP):
            out[base + k // 2 + 2 * g] = zb[t, g]
            out[base + k // 2 + 2 * g + 1] = sb[t, g]
    return out


def read_act(buf: np.ndarray, m: int, k: int) -> Quantized:
    from .formats import e4m3_decode
    buf = np.asarray(buf, np.uint8)
    row = k // 2 + (k // GROUP) * 2
    codes = np.zeros((m, k), np.int64)
    zb = np.zeros((m, k // GROUP), np.uint8)
    sb = np.zeros((m, k // GROUP), np.uint8)
    for t in range(m):
        base = t * row
        b = buf[base: base + k // 2].astype(np.int64)
        codes[t, 0::2] = b & 15
        codes[t, 1::2] = b >> 4
        zb[t] = buf[base + k // 2: base + row: 2]
        sb[t] = buf[base + k // 2 + 1: base + row: 2]
    return codes, e4m3_decode(zb), e4m3_decode(sb)


def read_weights_fast(buf: np.ndarray, n: int, k: int) -> Quantized:
    """read_weights by array reshapes (for full-size matrices); equal to read_weights."""
    from .formats import e4m3_decode
    nt, nq = n // TILE_N, k // (GROUP * QUAD)
    blk = np.asarray(buf, np.uint8)[: nt * nq * 1152].reshape(nt, nq, 1152)
    words = np.ascontiguousarray(blk[:, :, :1024]).view("<u4").reshape(nt, nq, 4, TILE_N, QUAD).astype(np.int64)
    nib = (words[..., None] >> (4 * np.arange(8))) & 15                 # [nt][nq][kg][i][j][e]
    codes = nib.transpose(0, 3, 1, 4, 2, 5).reshape(n, k)               # row (nt, i), channel (nq, j, kg, e)
    meta = blk[:, :, 1024:].reshape(nt, nq, TILE_N, QUAD, 2)
    zb = meta[..., 0].transpose(0, 2, 1, 3).reshape(n, k // GROUP)
    sb = meta[..., 1].transpose(0, 2, 1, 3).reshape(n, k // GROUP)
    return codes, e4m3_decode(zb), e4m3_decode(sb)
