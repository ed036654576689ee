"""Pins of the W4A4 oracle (cross-loop residual activations of a linear layer) against
values worked out by hand, the plain definition y = W x, brute force and the layout
written out byte by byte; none of them re-runs the oracle's own formulas."""
import numpy as np
import pytest

from oracle import w4a4 as W4
from oracle.formats import E4M3_POSITIVE, e4m3_encode


def haar(n, rng):
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))


def test_worked_example_by_hand():
    """K = 128 (one rotation block, R = I), every weight 0.5, anchor x0[k] = k mod 16.
    By hand: the weight groups are constant, so z = 0.5, s = 2^-9, codes 0 and W_hat = W;
    x0 spans 0..15 per group, so z = 0, s = 1 and a_hat = x0; y0 = 0.5 * 8 * 120 = 480.
    Loop 1, x = 2 x0: c = 2 exactly, residual 0, y = 960.  Loop 2, x = x0 + 1:
    c* = 1 + 960 / 9920, BF16 -> 1.09375; residual 1 - 0.09375 (k mod 16) lies on the grid
    z = -0.40625, s = 0.09375 (codes 15 - k mod 16), so it is exact, and
    y = 1.09375 * 480 + 0.5 * (128 - 0.09375 * 960) = 525 + 19 = 544 = W x exactly."""
    k, n = 128, 16
    w = np.full((n, k), 0.5)
    x0 = np.arange(k) % 16.0
    xs = np.stack([x0, 2 * x0, x0 + 1])[:, None, :]
    ys, cs, acts = W4.looped_linear(xs, w, np.eye(128))
    assert cs[:, 0].tolist() == [1.0, 2.0, 1.09375]
    assert np.all(ys[0] == 480.0) and np.all(ys[1] == 960.0) and np.all(ys[2] == 544.0)
    codes, z, s = acts[2]
    assert np.all(z == -0.40625) and np.all(s == 0.09375)
    assert np.array_equal(codes[0], 15 - np.arange(k) % 16)


def _on_grid(shape, rng):
    """Values z + q s per group of 32 with E4M3 z, s and codes that reach 0 and 15 in every
    group, so the quantizer must return exactly them."""
    m, k = shape
    g = k // 32
    z = rng.choice(np.concatenate([-E4M3_POSITIVE[40:90], E4M3_POSITIVE[40:90]]), size=(m, g))
    s = rng.choice(E4M3_POSITIVE[30:70], size=(m, g))
    q = rng.integers(0, 16, size=(m, g, 32))
    q[..., 0], q[..., 1] = 0, 15
    return (z[..., None] + q * s[..., None]).reshape(m, k), q.reshape(m, k)


def test_lossless_construction():
    """Weights and anchor activations on the quantizer grid, later loops equal to the
    anchor: W_hat = W, a_hat = x0, c = 1, every residual exactly zero, and every loop's
    output equals the exact product W x0 (brute force)."""
    rng = np.random.default_rng(3)
    w, wq_codes = _on_grid((16, 256), rng)
    x0, _ = _on_grid((2, 256), rng)
    rot = haar(128, rng)
    xs = np.stack([x0, x0, x0])
    ys, cs, acts = W4.looped_linear(xs, w, rot)
    assert np.array_equal(W4.quantize_weights(w)[0], wq_codes)
    exact = np.array([[sum(w[nn, kk] * x0[mm, kk] for kk in range(256)) for nn in range(16)] for mm in range(2)])
    assert np.all(cs == 1.0)
    for l in (1, 2):
        codes, z, s = acts[l]
        assert np.all(W4.dequant(acts[l]) == 0.0)
    for l in range(3):
        assert np.allclose(ys[l], exact, rtol=1e-13, atol=1e-12)


def test_rotation_direction_by_loops():
    """rotate_blocks computes R v per block (r_j = sum_i R[j, i] v_i, as the KV method's
    residual rotation) and rotate_weights W R^T, checked against explicit loops."""
    rng = np.random.default_rng(5)
    rot = rng.standard_normal((128, 128))
    v = rng.standard_normal(256)
    w = rng.standard_normal((2, 256))
    rv = W4.rotate_blocks(v, rot)
    wr = W4.rotate_weights(w, rot)
    for b in range(2):
        for j in (0, 17, 127):
            assert abs(rv[128 * b + j] - sum(rot[j, i] * v[128 * b + i] for i in range(128))) < 1e-10
            for nn in range(2):
                assert abs(wr[nn, 128 * b + j] - sum(w[nn, 128 * b + i] * rot[j, i] for i in range(128))) < 1e-10


def test_folded_rotation_reproduces_w_x():
    """With an orthogonal R, (W R^T)(R x) = W x: the rotation folded into the weights
    leaves the unquantized product unchanged (a transposed R on either side breaks it)."""
    rng = np.random.default_rng(6)
    rot = haar(128, rng)
    w = rng.standard_normal((8, 384))
    x = rng.standard_normal((3, 384))
    assert np.allclose(W4.rotate_blocks(x, rot) @ W4.rotate_weights(w, rot).T, x @ w.T, rtol=1e-12, atol=1e-12)
    assert not np.allclose(W4.rotate_blocks(x, rot.T) @ W4.rotate_weights(w, rot).T, x @ w.T, atol=1e-3)


def test_identity_rotation_brute_force():
    """R = I: y_l must be W_hat (c a_hat + r_hat), summed element by element."""
    rng = np.random.default_rng(7)
    w = rng.standard_normal((16, 128)) * 0.05
    x0 = rng.standard_normal((2, 128))
    x1 = 0.9 * x0 + 0.2 * rng.standard_normal((2, 128))
    ys, cs, acts = W4.looped_linear(np.stack([x0, x1]), w, np.eye(128))
    wh = W4.dequant(W4.quantize_weights(w))
    ah, rh = W4.dequant(acts[0]), W4.dequant(acts[1])
    for mm in range(2):
        for nn in (0, 5, 15):
            want = sum(wh[nn, kk] * (cs[1, mm] * ah[mm, kk] + rh[mm, kk]) for kk in range(128))
            assert abs(ys[1, mm, nn] - want) < 1e-12 * max(1.0, abs(want))


def test_error_against_plain_product_is_bounded():
    """y_l - W x_l = c (W_hat - W) a_hat + (W_R_hat - W R^T) r_hat + W R^T (r_hat - r), an
    identity because x_l = c a_hat + R^T r; every term is bounded by half a quantizer step
    per element, so |y_l - W x_l| <= |c| (s_w/2)|a_hat| + (s_wr/2)|r_hat| + |W R^T|(s_r/2)."""
    rng = np.random.default_rng(8)
    rot = haar(128, rng)
    w = rng.standard_normal((32, 256)) * 0.05
    x0 = rng.standard_normal((4, 256))
    x1 = 0.85 * x0 + 0.15 * rng.standard_normal((4, 256))
    ys, cs, acts = W4.looped_linear(np.stack([x0, x1]), w, rot)
    wq, wrq = W4.quantize_weights(w), W4.quantize_weights(w, rot)
    sw = np.repeat(wq[2], 32, axis=1)
    swr = np.repeat(wrq[2], 32, axis=1)
    sr = np.repeat(acts[1][2], 32, axis=1)
    ah, rh = np.abs(W4.dequant(acts[0])), np.abs(W4.dequant(acts[1]))
    wr = W4.rotate_weights(w, rot)
    bound = (np.abs(cs[1])[:, None] * (ah @ (sw / 2).T) + rh @ (swr / 2).T + (sr / 2) @ np.abs(wr).T)
    err = np.abs(ys[1] - x1 @ w.T)
    assert np.all(err <= bound * (1 + 1e-9) + 1e-12)
    assert err.max() > 0


def test_zero_anchor_gives_zero_coefficient():
    rng = np.random.default_rng(9)
    rot = haar(128, rng)
    w = rng.standard_normal((16, 128)) * 0.05
    x1 = rng.standard_normal((1, 128))
    ys, cs, acts = W4.looped_linear(np.stack([np.zeros((1, 128)), x1]), w, rot)
    assert cs[1, 0] == 0.0
    assert np.all(ys[0] == 0.0)
    # c = 0: the residual is R x itself, quantized by the same 4-bit group quantizer
    assert np.array_equal(ys[1], W4.linear(W4.quantize_weights(w, rot), W4.anchor_activation(W4.rotate_blocks(x1, rot))))


def test_weight_layout_bytes_by_hand():
    """N = 32, K = 128, one code 9 at (row 17, channel 37), offsets 0.5 and scales 2^-9
    elsewhere.  By hand: row tile 1, quad 0 -> block at 1152; row 1 of the tile, group 1
    (j = 1), quarter kg = 0, channel 5 of the quarter -> word at 1152 + 16 * 1 + 4 = 1172,
    bits 20..23 -> byte 1174, high nibble; metadata of (row 1, group 1) at 1152 + 1024 + 10."""
    codes = np.zeros((32, 128), np.int64)
    codes[17, 37] = 9
    z = np.full((32, 4), 0.5)
    s = np.full((32, 4), 2.0 ** -9)
    z[17, 1], s[17, 1] = -1.0, 0.25
    buf = W4.write_weights((codes, z, s))
    assert buf.size == W4.weight_bytes(32, 128) == 32 * 64 + 32 * 4 * 2
    assert buf[1174] == 0x90 and int(buf[1152:2176].astype(np.int64).sum()) == 0x90
    assert buf[2186] == e4m3_encode(np.array(-1.0)) and buf[2187] == e4m3_encode(np.array(0.25))
    back = W4.read_weights(buf, 32, 128)
    assert np.array_equal(back[0], codes) and np.array_equal(back[1], z) and np.array_equal(back[2], s)


def test_activation_layout_bytes_by_hand():
    """M = 2, K = 128: rows of 64 code bytes + 8 metadata bytes; token 1 channel 5 = 7 sits
    in the high nibble of byte 72 + 2."""
    codes = np.zeros((2, 128), np.int64)
    codes[1, 5] = 7
    z = np.zeros((2, 4))
    s = np.full((2, 4), 1.0)
    buf = W4.write_act((codes, z, s))
    assert buf.size == W4.act_bytes(2, 128) == 144
    assert buf[74] == 0x70 and int(buf[72:136].astype(np.int64).sum()) == 0x70
    back = W4.read_act(buf, 2, 128)
    assert np.array_equal(back[0], codes) and np.array_equal(back[2], s)


@pytest.mark.parametrize("seed", [0, 1])
def test_layout_round_trip(seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((48, 256)) * 0.05
    q = W4.quantize_weights(w)
    back = W4.read_weights(W4.write_weights(q), 48, 256)
    assert all(np.array_equal(a, b) for a, b in zip(q, back))
    a = W4.anchor_activation(rng.standard_normal((3, 256)))
    back = W4.read_act(W4.write_act(a), 3, 256)
    assert all(np.array_equal(u, v) for u, v in zip(a, back))


def test_fast_weight_reader_equals_loops():
    rng = np.random.default_rng(12)
    q = W4.quantize_weights(rng.standard_normal((32, 256)) * 0.05)
    buf = W4.write_weights(q)
    a, b = W4.read_weights(buf, 32, 256), W4.read_weights_fast(buf, 32, 256)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
