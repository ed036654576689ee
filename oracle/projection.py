"""CPU oracle of the K/V projection that feeds the pending buffer.

TEST INFRASTRUCTURE ONLY.  Nothing under ``oracle/`` is part of the product:
only ``tests/``, the package's ``smoke()`` check and the benchmark's CPU
baseline leg may import it.  It shares no code with the HIP path.

Source: the ResidualQuant explainer, paragraph "Which print is the master":
while a token is still being decoded, the K and V that each loop produces are
kept in BF16 in a temporary buffer, and they are quantized only after the
group's last loop has run.  A looped Transformer runs the same layer every
loop, so loop l's K and V of the current token are that layer's K/V
projections of the loop's hidden state.

Readings adopted where the pages are silent:

* the projection is a plain linear map without bias, ``k = W_K x``,
  ``v = W_V x`` (no positional rotation: the pages describe none);
* it is computed exactly (float64 here: each product of two BF16 values is
  exact and the sums of up to a few thousand of them are correct to about
  1e-13 relative) and rounded once to BF16, half to even, which is the value a
  BF16 model stores;
* the weights are one ``[2][n_kv_heads][head_dim][hidden]`` array (the K rows,
  then the V rows, each output channel's weights contiguous over ``hidden``).

Parity of the GPU path (float32 accumulation on the matrix cores) against this
exact result is decided in the tests: identical BF16 values, except outputs
whose exact value lies next to a BF16 rounding midpoint.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .formats import bf16_round


def kv_projection(x: np.ndarray, w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """K and V of one token per batch row at one loop.

    x : [batch][hidden] float64 holding BF16 values (the loop's hidden state).
    w : [2][n_kv_heads][head_dim][hidden] float64 holding BF16 values.
    Returns (exact, rounded): both [2][batch][n_kv_heads][head_dim]; ``exact`` is the
    float64 product, ``rounded`` its BF16 rounding (half to even).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    two, hkv, d, hidden = w.shape
    if two != 2 or x.shape[1] != hidden:
        raise ValueError("shape mismatch between x and w")
    flat = w.reshape(2 * hkv * d, hidden)
    y = x @ flat.T                                   # [batch][2 * hkv * d]
    exact = y.reshape(x.shape[0], 2, hkv, d).transpose(1, 0, 2, 3).copy()
    return exact, bf16_round(exact)


def magnitude_sums(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """sum_i |x_i w_ni| for every output, [2][batch][n_kv_heads][head_dim]: the scale of the
    rounding error of any summation order of the products."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    w = np.abs(np.asarray(w, dtype=np.float64))
    two, hkv, d, hidden = w.shape
    y = x @ w.reshape(2 * hkv * d, hidden).T
    return y.reshape(x.shape[0], 2, hkv, d).transpose(1, 0, 2, 3).copy()


def write_pending(pending: np.ndarray, kv: np.ndarray, local_loop: int,
                  rows: Optional[int] = None) -> np.ndarray:
    """Store one loop's K/V ([2][batch][n_kv_heads][head_dim]) into the pending buffer
    [batch][L][2][n_kv_heads][head_dim] at loop slot ``local_loop``; other slots keep
    their contents."""
    b = kv.shape[1] if rows is None else rows
    for x in range(2):
        pending[:b, local_loop, x] = kv[x, :b]
    return pending
