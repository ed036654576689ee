"""Pins of the oracle's decode attention: torch's scaled_dot_product_attention, closed
forms (q = 0), a lossless construction that reduces RQ attention to plain attention,
and the rearranged (factored) form a kernel evaluates."""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

from looped_transformer_decode_amd import synth
from oracle import formats as F
from oracle import residualquant as RQ


def _cfg(wl, chained=False):
    return RQ.Config(wl.head_dim, wl.group, wl.anchor_bits, wl.resid_bits, wl.loops_per_group,
                     wl.n_groups, chained, wl.n_kv_heads, wl.n_q_heads, wl.batch, wl.ctx + 1)


def _sdpa(q, keys, values, scale, gqa=1):
    """torch reference: q (B, Hq, d), keys/values (B, Hkv, n, d) -> (B, Hq, d)."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[:, :, None, :]
    k = torch.from_numpy(np.asarray(keys, np.float64)).repeat_interleave(gqa, dim=1)
    v = torch.from_numpy(np.asarray(values, np.float64)).repeat_interleave(gqa, dim=1)
    return Fnn.scaled_dot_product_attention(qt, k, v, scale=scale)[:, :, 0, :].numpy()


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(30)
    q = rng.normal(size=(1, 1, 64))
    keys = rng.normal(size=(1, 1, 300, 64)) * 3
    values = rng.normal(size=(1, 1, 300, 64))
    ours = RQ.attention(q[0, 0], keys[0, 0], values[0, 0], 0.125)
    assert np.allclose(ours, _sdpa(q, keys, values, 0.125)[0, 0], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("chained", [False, True])
def test_brute_force_equals_factored_form(chained):
    wl = synth.WORKLOADS["tiny_d64_t256"]
    inp = synth.generate(wl, seed=31)
    cfg = _cfg(wl, chained)
    kv = inp.kv.double().numpy()
    rot = inp.rot.double().numpy()
    T = wl.ctx
    cache = RQ.pack_context(kv, rot, cfg, T)
    lay = RQ.Layout(cfg)
    q = inp.q.double().numpy()
    sc = synth.sm_scale(wl.head_dim)
    for loop in range(4):
        kc, vc = kv[0, loop, 0, :, :, T], kv[0, loop, 1, :, :, T]
        o = RQ.decode_attention(cache, lay, loop, q[loop], kc, vc, [T], rot, sc)
        for h in range(2):
            ek = RQ.read_tokens(cache, lay, 0, h, 0, 0, T)
            ev = RQ.read_tokens(cache, lay, 0, h, 1, 0, T)
            of = RQ.decode_attention_factored(ek, ev, loop, q[loop][0, h], kc[0, h], vc[0, h],
                                              rot[h, 0], rot[h, 1], sc, cfg)
            assert np.allclose(o[0, h], of, rtol=1e-12, atol=1e-12 * np.abs(of).max())


def test_zero_query_gives_mean_of_rebuilt_values():
    wl = synth.WORKLOADS["tiny_d64_t256"]
    inp = synth.generate(wl, seed=32)
    cfg = _cfg(wl)
    kv = inp.kv.double().numpy()
    rot = inp.rot.double().numpy()
    T = 100
    cache = RQ.pack_context(kv, rot, cfg, T)
    lay = RQ.Layout(cfg)
    q = np.zeros((1, 2, 64))
    for loop in (0, 3):
        vc = kv[0, loop, 1, :, :, T]
        o = RQ.decode_attention(cache, lay, loop, q, kv[0, loop, 0, :, :, T], vc, [T], rot, 0.125)
        for h in range(2):
            ev = RQ.read_tokens(cache, lay, 0, h, 1, 0, T)
            vals = np.concatenate([RQ.reconstruct(ev, loop, rot[h, 1], cfg), vc[0, h][None]])
            assert np.allclose(o[0, h], vals.mean(axis=0), rtol=1e-12, atol=1e-13)


def test_anchor_loop_is_plain_attention_over_dequantized_anchor():
    wl = synth.WORKLOADS["tiny_d64_t256"]
    inp = synth.generate(wl, seed=33)
    cfg = _cfg(wl)
    kv = inp.kv.double().numpy()
    rot = inp.rot.double().numpy()
    T = wl.ctx
    cache = RQ.pack_context(kv, rot, cfg, T)
    lay = RQ.Layout(cfg)
    q = inp.q.double().numpy()[3]
    kc, vc = kv[0, 3, 0, :, :, T], kv[0, 3, 1, :, :, T]
    o = RQ.decode_attention(cache, lay, 3, q, kc, vc, [T], rot, 0.125)
    keys = np.empty((1, 2, T + 1, 64))
    vals = np.empty((1, 2, T + 1, 64))
    for h in range(2):
        for x, dst, cur in ((0, keys, kc), (1, vals, vc)):
            qa, za, sa = RQ.quantize(kv[0, 3, x, 0, h, :T], 4, 32)      # same definition, recomputed
            dst[0, h, :T] = RQ.dequantize(qa, za, sa, 32)
            dst[0, h, T] = cur[0, h]
    assert np.allclose(o, _sdpa(q, keys, vals, 0.125), rtol=1e-12, atol=1e-13)


def _lossless_inputs(rng, B, Hkv, T, d, L):
    """K/V whose anchor lies on the INT4 grid of every group (z = -1, s = 1/8, codes 0..15
    with both ends present) and whose other loops equal the anchor: then c = 1, the
    residual is exactly zero and RQ reconstruction is exact."""
    codes = rng.integers(0, 16, size=(2, B, Hkv, T + 1, d))
    codes[..., 0::32] = 0
    codes[..., 1::32] = 15
    vals = -1.0 + codes / 8.0                     # exactly representable in BF16
    kv = np.broadcast_to(vals[None, None], (1, L) + vals.shape).copy()
    return kv


@pytest.mark.parametrize("gqa", [1, 4])
@pytest.mark.parametrize("chained", [False, True])
def test_lossless_construction_reduces_to_plain_attention(gqa, chained):
    rng = np.random.default_rng(34 + gqa)
    B, Hkv, T, d, L = 2, 2, 130, 64, 4
    Hq = Hkv * gqa
    cfg = RQ.Config(d, 32, 4, 2, L, 1, chained, Hkv, Hq, B, T + 1)
    kv = _lossless_inputs(rng, B, Hkv, T, d, L)
    rot = synth.haar_rotations(Hkv, d, 35).double().numpy()
    cache = RQ.pack_context(kv, rot, cfg, T)
    lay = RQ.Layout(cfg)
    enc = RQ.read_tokens(cache, lay, 1, 1, 0, 0, T)
    assert np.all(enc.resid[0][3] == 1.0)                     # c = 1
    assert np.all(enc.resid[0][0] == 0) and np.all(enc.resid[1][1] == 0)   # zero residual codes
    q = rng.normal(size=(B, Hq, d))
    ctx = [T, 77]
    for loop in range(L):
        kc, vc = kv[0, loop, 0, :, :, T], kv[0, loop, 1, :, :, T]
        o = RQ.decode_attention(cache, lay, loop, q, kc, vc, ctx, rot, 0.125)
        for b in range(B):
            n = ctx[b]
            keys = np.concatenate([kv[0, loop, 0, b:b + 1, :, :n], kc[b:b + 1, :, None]], axis=2)
            vals = np.concatenate([kv[0, loop, 1, b:b + 1, :, :n], vc[b:b + 1, :, None]], axis=2)
            ref = _sdpa(q[b:b + 1], keys, vals, 0.125, gqa=gqa)
            assert np.allclose(o[b], ref[0], rtol=1e-12, atol=1e-13)


def test_empty_context_returns_current_value():
    wl = synth.WORKLOADS["tiny_d64_t256"]
    inp = synth.generate(wl, seed=36)
    cfg = _cfg(wl)
    kv = inp.kv.double().numpy()
    rot = inp.rot.double().numpy()
    cache = np.zeros(RQ.Layout(cfg).total_bytes, dtype=np.uint8)
    vc = kv[0, 1, 1, :, :, 0]
    o = RQ.decode_attention(cache, RQ.Layout(cfg), 1, inp.q.double().numpy()[1],
                            kv[0, 1, 0, :, :, 0], vc, [0], rot, 0.125)
    assert np.array_equal(o, vc)


@pytest.mark.parametrize("chained", [False, True])
def test_token_permutation_invariance(chained):
    """Softmax attention does not depend on the order of the context tokens.  Packing the
    same tokens in another order must give the same output at every loop (this catches a
    key scored against another token's value, coefficient or metadata)."""
    wl = synth.WORKLOADS["tiny_d64_t256"]
    inp = synth.generate(wl, seed=36)
    cfg = _cfg(wl, chained)
    kv = inp.kv.double().numpy()
    rot = inp.rot.double().numpy()
    T = 150
    perm = np.random.default_rng(37).permutation(T)
    kvp = kv.copy()
    kvp[..., :T, :] = kv[..., perm, :]
    lay = RQ.Layout(cfg)
    c0 = RQ.pack_context(kv, rot, cfg, T)
    c1 = RQ.pack_context(kvp, rot, cfg, T)
    assert not np.array_equal(c0, c1)
    q = inp.q.double().numpy()
    for loop in range(4):
        kc, vc = kv[0, loop, 0, :, :, T], kv[0, loop, 1, :, :, T]
        o0 = RQ.decode_attention(c0, lay, loop, q[loop], kc, vc, [T], rot, 0.125)
        o1 = RQ.decode_attention(c1, lay, loop, q[loop], kc, vc, [T], rot, 0.125)
        assert np.allclose(o0, o1, rtol=1e-12, atol=1e-13)
