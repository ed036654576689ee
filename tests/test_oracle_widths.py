"""Pins of the oracle's per-loop residual widths (the commentary page, section "它压的根本不是
KV": the loops next to the anchor keep thinner residuals, the farther ones more bits).

A configuration gives each non-anchor loop its own residual width; the layout then has
residual planes of different sizes.  Pinned by: the storage arithmetic and byte offsets
worked out by hand, the equality of an all-equal width list with the uniform layout (bit
for bit), each loop's quantizer invariants at its own width, the error reduction a wider
loop buys, the lossless construction (plain attention), and the two algebraic forms of
decode attention agreeing on a mixed-width cache."""
import dataclasses

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

from looped_transformer_decode_amd import synth
from oracle import formats as F
from oracle import residualquant as RQ


def _cfg(widths, d=128, g=32, L=4, batch=1, ctx=100, hkv=1, hq=1, chained=False):
    return RQ.Config(d, g, 4, 2, L, 1, chained, hkv, hq, batch, ctx, 0, tuple(widths))


def test_storage_and_offsets_by_hand():
    """d = 128, g = 32, INT4 anchor, residual widths (4, 2, 2) for loops 0, 1, 2 (loop 0 is
    the farthest from the anchor, loop 3).  Per token, head and K|V:
      loop 0: 64 B codes + 8 B meta + 2 B c = 74;  loops 1, 2: 32 + 8 + 2 = 42;  anchor: 64 + 8 = 72
      = 230 B = 14.375 bits per element position over the 4 loops (BF16: 64), a 77.5% cut.
    Tiles of 64 tokens: 4736, 2688, 2688, 4608 B; with 2 tiles per plane the planes start at
    0, 9472, 14848 and 20224, and one group takes 29440 B."""
    lay = RQ.Layout(_cfg((4, 2, 2)))
    assert lay.bytes_per_token_loop() == [74, 42, 42, 72]
    assert 8 * sum(lay.bytes_per_token_loop()) / 128 == 14.375
    assert round(100 * (1 - 14.375 / 64), 1) == 77.5
    assert lay.r_tiles == [4736, 2688, 2688] and lay.a_tile == 4608 and lay.n_tiles == 2
    assert [lay.plane_offset(0, 0, 0, l) for l in range(4)] == [0, 9472, 14848, 20224]
    assert lay.group_bytes == 29440 and lay.total_bytes == 2 * 29440
    assert lay.plane_offset(0, 0, 1, 0) == 29440


def test_equal_widths_give_the_uniform_layout_bit_for_bit():
    wl = synth.WORKLOADS["tiny_d64_t256"]
    inp = synth.generate(wl, seed=60, ctx=150)
    kv = inp.kv.double().numpy()
    rot = inp.rot.double().numpy()
    base = RQ.Config(64, 32, 4, 2, 4, 1, False, 2, 2, 1, 151)
    for widths in ((2, 2, 2), (4, 4, 4)):
        explicit = dataclasses.replace(base, resid_bits_loop=widths)
        uniform = dataclasses.replace(base, resid_bits=widths[0])
        a = RQ.pack_context(kv, rot, explicit, 150)
        b = RQ.pack_context(kv, rot, uniform, 150)
        assert RQ.Layout(explicit).total_bytes == RQ.Layout(uniform).total_bytes
        assert np.array_equal(a, b)


def _loops(seed, n, d, a=(0.85, 0.9, 0.95)):
    rng = np.random.default_rng(seed)
    anchor = rng.normal(0, 1, (n, d))
    anchor[:, rng.choice(d, 4, replace=False)] *= 8
    xs = [a[l] * anchor + 0.15 * rng.normal(0, 1, (n, d)) for l in range(3)] + [anchor]
    return F.bf16_round(np.stack(xs))


def test_each_loop_is_quantized_at_its_own_width():
    xs = _loops(61, 400, 128)
    rot = synth.haar_rotations(1, 128, 62)[0, 0].double().numpy()
    wide = RQ.encode(xs, rot, _cfg((4, 2, 2)))
    narrow = RQ.encode(xs, rot, _cfg((2, 2, 2)))
    for l, bits in ((0, 4), (1, 2), (2, 2)):
        q, z, s, c = wide.resid[l]
        assert q.min() >= 0 and q.max() <= 2 ** bits - 1
        assert q.max() > 3 if bits == 4 else True                 # the 4-bit loop uses its range
        r = (xs[l] - c[:, None] * RQ.dequantize(*wide.anchor, 32)) @ rot.T
        rg, qg = r.reshape(400, 4, 32), q.reshape(400, 4, 32)
        assert np.all(z <= rg.min(-1)) and np.all(z + (2 ** bits - 1) * s >= rg.max(-1))
        assert np.all(np.abs(rg - (z[..., None] + qg * s[..., None])) <= s[..., None] / 2)
    # loops 1 and 2 are the same whatever loop 0's width
    for l in (1, 2):
        for u, v in zip(wide.resid[l], narrow.resid[l]):
            assert np.array_equal(u, v)
    # a 4-bit residual scale is about a fifth of the 2-bit one: the rebuilt loop 0 is much closer
    cfg_w, cfg_n = _cfg((4, 2, 2)), _cfg((2, 2, 2))
    e_w = np.linalg.norm(xs[0] - RQ.reconstruct(wide, 0, rot, cfg_w), axis=-1)
    e_n = np.linalg.norm(xs[0] - RQ.reconstruct(narrow, 0, rot, cfg_n), axis=-1)
    assert e_w.mean() < 0.35 * e_n.mean()


def test_bytes_round_trip_with_mixed_widths():
    wl = synth.WORKLOADS["tiny_d64_t256"]
    inp = synth.generate(wl, seed=63, ctx=130)
    kv = inp.kv.double().numpy()
    rot = inp.rot.double().numpy()
    cfg = RQ.Config(64, 32, 4, 2, 4, 1, False, 2, 2, 1, 131, 0, (4, 4, 2))
    cache = RQ.pack_context(kv, rot, cfg, 130)
    lay = RQ.Layout(cfg)
    for h in range(2):
        for x in range(2):
            enc = RQ.encode(kv[0, :, x, 0, h, :130], rot[h, x], cfg)
            back = RQ.read_tokens(cache, lay, 0, h, x, 0, 130)
            for u, v in zip(enc.anchor, back.anchor):
                assert np.array_equal(u, v)
            for ru, rv in zip(enc.resid, back.resid):
                for u, v in zip(ru, rv):
                    assert np.array_equal(u, v)


def test_mixed_widths_lossless_construction_and_factored_form():
    """Anchor on the INT4 grid and the other loops equal to it: c = 1, zero residuals, so
    attention at every loop is torch's softmax attention over the values; and on a
    generated cache the brute-force and factored forms agree."""
    rng = np.random.default_rng(64)
    B, Hkv, T, d, L = 1, 2, 90, 64, 4
    codes = rng.integers(0, 16, size=(2, B, Hkv, T + 1, d))
    codes[..., 0::32] = 0
    codes[..., 1::32] = 15
    vals = -1.0 + codes / 8.0
    kv = np.broadcast_to(vals[None, None], (1, L) + vals.shape).copy()
    rot = synth.haar_rotations(Hkv, d, 65).double().numpy()
    cfg = RQ.Config(d, 32, 4, 2, L, 1, False, Hkv, Hkv, B, T + 1, 0, (4, 2, 4))
    cache = RQ.pack_context(kv, rot, cfg, T)
    lay = RQ.Layout(cfg)
    q = rng.normal(size=(B, Hkv, d))
    for loop in range(L):
        kc, vc = kv[0, loop, 0, :, :, T], kv[0, loop, 1, :, :, T]
        o = RQ.decode_attention(cache, lay, loop, q, kc, vc, [T], rot, 0.125)
        keys = torch.from_numpy(vals[0, :, :, :T + 1].copy())
        values = torch.from_numpy(vals[1, :, :, :T + 1].copy())
        keys[:, :, T] = torch.from_numpy(kc)
        values[:, :, T] = torch.from_numpy(vc)
        ref = Fnn.scaled_dot_product_attention(torch.from_numpy(q)[:, :, None], keys, values, scale=0.125)[:, :, 0]
        assert np.allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)
    wl = synth.WORKLOADS["tiny_d64_t256"]
    inp = synth.generate(wl, seed=66, ctx=120)
    kv = inp.kv.double().numpy()
    rot = inp.rot.double().numpy()
    cfg = RQ.Config(64, 32, 4, 2, 4, 1, False, 2, 2, 1, 121, 0, (4, 2, 2))
    cache = RQ.pack_context(kv, rot, cfg, 120)
    lay = RQ.Layout(cfg)
    qq = inp.q.double().numpy()
    for loop in range(4):
        kc, vc = kv[0, loop, 0, :, :, 120], kv[0, loop, 1, :, :, 120]
        o = RQ.decode_attention(cache, lay, loop, qq[loop], kc, vc, [120], rot, 0.125)
        for h in range(2):
            ek = RQ.read_tokens(cache, lay, 0, h, 0, 0, 120)
            ev = RQ.read_tokens(cache, lay, 0, h, 1, 0, 120)
            of = RQ.decode_attention_factored(ek, ev, loop, qq[loop][0, h], kc[0, h], vc[0, h], rot[h, 0],
                                              rot[h, 1], 0.125, cfg)
            assert np.allclose(o[0, h], of, rtol=1e-12, atol=1e-12 * np.abs(of).max())
