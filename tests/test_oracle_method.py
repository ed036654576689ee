"""Pins of the oracle's encoding: least-squares coefficient, rotation, reconstruction
bounds, chained-variant special cases, byte layout and the pages' storage arithmetic."""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

from looped_transformer_decode_amd import synth
from oracle import formats as F
from oracle import residualquant as RQ

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cfg(wl, chained=False, batch=None, ctx=None, L=None):
    return RQ.Config(wl.head_dim, wl.group, wl.anchor_bits, wl.resid_bits,
                     L or wl.loops_per_group, wl.n_groups, chained, wl.n_kv_heads, wl.n_q_heads,
                     batch or wl.batch, ctx or wl.ctx + 1)


def _loops(seed, n_tok, d, L=4, a=(0.5, 0.7, 0.9), noise=0.15, outliers=4):
    rng = np.random.default_rng(seed)
    anchor = rng.normal(0, 1, (n_tok, d))
    anchor[:, rng.choice(d, outliers, replace=False)] *= 8
    xs = [a[l] * anchor + noise * rng.normal(0, 1, (n_tok, d)) for l in range(L - 1)] + [anchor]
    return F.bf16_round(np.stack(xs))


def test_ls_coefficient_normal_equation_and_rounding():
    xs = _loops(20, 500, 128)
    q, z, s = RQ.quantize(xs[3], 4, 32)
    a_hat = RQ.dequantize(q, z, s, 32)
    for l in range(3):
        c, exact = RQ.ls_coefficient(xs[l], a_hat)
        resid = np.sum((xs[l] - exact[:, None] * a_hat) * a_hat, axis=-1)
        scale = np.sum(np.abs(xs[l] * a_hat), axis=-1)
        assert np.all(np.abs(resid) <= 1e-12 * scale)
        # c is the BF16 value nearest c*: within half a BF16 ulp
        ulp = 2.0 ** (np.floor(np.log2(np.abs(exact))) - 7)
        assert np.all(np.abs(c - exact) <= ulp / 2)
        F.bf16_bits(c)


def test_ls_coefficient_zero_reference():
    c, exact = RQ.ls_coefficient(np.ones((1, 8)), np.zeros((1, 8)))
    assert c[0] == 0 and exact[0] == 0


def test_norm_ratio_coefficient_matches_norms():
    """Norm ratio: |c*| * ||ref|| = ||x|| for every vector (the defining property), c* >= 0,
    c = BF16(c*) within half an ulp."""
    xs = _loops(21, 400, 128)
    q, z, s = RQ.quantize(xs[3], 4, 32)
    a_hat = RQ.dequantize(q, z, s, 32)
    for l in range(3):
        c, exact = RQ.norm_ratio_coefficient(xs[l], a_hat)
        lhs = exact * np.linalg.norm(a_hat, axis=-1)
        assert np.all(np.abs(lhs - np.linalg.norm(xs[l], axis=-1)) <= 1e-13 * lhs)
        assert np.all(exact >= 0)
        ulp = 2.0 ** (np.floor(np.log2(exact)) - 7)
        assert np.all(np.abs(c - exact) <= ulp / 2)


def test_norm_ratio_special_cases():
    """x = k * ref with k > 0: both rules give k; x = -ref: least squares gives -1, the norm
    ratio 1; x orthogonal to ref: least squares gives 0, the norm ratio ||x||/||ref||;
    ref = 0: both give 0."""
    rng = np.random.default_rng(3)
    ref = rng.normal(size=(5, 64))
    for k in (0.5, 1.0, 3.0):
        for fn in (RQ.ls_coefficient, RQ.norm_ratio_coefficient):
            _, exact = fn(k * ref, ref)
            assert np.allclose(exact, k, rtol=1e-14, atol=0)
    assert np.allclose(RQ.ls_coefficient(-ref, ref)[1], -1.0, rtol=1e-14)
    assert np.allclose(RQ.norm_ratio_coefficient(-ref, ref)[1], 1.0, rtol=1e-14)
    e1 = np.zeros((1, 8)); e1[0, 0] = 2.0
    e2 = np.zeros((1, 8)); e2[0, 1] = 0.5
    assert RQ.ls_coefficient(e1, e2)[1][0] == 0.0
    assert RQ.norm_ratio_coefficient(e1, e2)[1][0] == 4.0
    c, exact = RQ.norm_ratio_coefficient(np.ones((1, 8)), np.zeros((1, 8)))
    assert c[0] == 0 and exact[0] == 0


def test_encode_uses_the_configured_rule():
    """A configuration with the norm-ratio rule stores ||x||/||a_hat|| (rounded to BF16) as c
    and quantizes x - c * a_hat; the default stores the least-squares c."""
    wl = synth.WORKLOADS["tiny_d64_t256"]
    xs = _loops(22, 50, 64)
    rot = synth.haar_rotations(1, 64, 9).double().numpy()[0, 0]
    for rule, fn in ((0, RQ.ls_coefficient), (1, RQ.norm_ratio_coefficient)):
        cfg = dataclasses.replace(_cfg(wl), scale_rule=rule)
        enc = RQ.encode(xs, rot, cfg)
        a_hat = RQ.dequantize(*enc.anchor, wl.group)
        for l in range(3):
            c_exp, _ = fn(xs[l], a_hat)
            assert np.array_equal(enc.resid[l][3], c_exp)
            r = (xs[l] - c_exp[:, None] * a_hat) @ rot.T
            qr, zr, sr = RQ.quantize(r, wl.resid_bits, wl.group)
            assert np.array_equal(enc.resid[l][0], qr)
    # the two rules give different c on these inputs
    c0 = RQ.encode(xs, rot, _cfg(wl)).resid[0][3]
    c1 = RQ.encode(xs, rot, dataclasses.replace(_cfg(wl), scale_rule=1)).resid[0][3]
    assert not np.array_equal(c0, c1)


def test_synthetic_rotations_are_orthogonal():
    rot = synth.haar_rotations(3, 128, 5).double().numpy()
    for h in range(3):
        for x in range(2):
            R = rot[h, x]
            assert np.abs(R.T @ R - np.eye(128)).max() <= 1e-6
            assert abs(abs(np.linalg.det(R)) - 1) <= 1e-5
            y = np.random.default_rng(h).normal(size=128)
            assert abs(np.linalg.norm(R @ y) - np.linalg.norm(y)) <= 1e-6 * np.linalg.norm(y)
    # two different heads get different rotations
    assert np.abs(rot[0, 0] - rot[1, 0]).max() > 0.1


def _recon_bound(s, group, y_norm):
    return np.sqrt(np.sum(group * (s / 2) ** 2, axis=-1)) * (1 + 1e-6) + 2e-6 * y_norm


@pytest.mark.parametrize("chained", [False, True])
def test_reconstruction_error_within_quantizer_bound(chained):
    wl = synth.WORKLOADS["ouro_b4_t8192"]
    cfg = _cfg(wl, chained=chained, batch=1, ctx=256)
    rot = synth.haar_rotations(1, 128, 9)[0, 0].double().numpy()
    xs = _loops(21, 256, 128)
    enc = RQ.encode(xs, rot, cfg)
    qa, za, sa = enc.anchor
    a_hat = RQ.dequantize(qa, za, sa, 32)
    # anchor: per-element bound s/2
    assert np.all(np.abs(xs[3] - a_hat).reshape(256, 4, 32) <= sa[..., None] / 2)
    for l in range(3):
        xh = RQ.reconstruct(enc, l, rot, cfg)
        err = np.linalg.norm(xs[l] - xh, axis=-1)
        bound = _recon_bound(enc.resid[l][2], 32, np.linalg.norm(xs[l], axis=-1))
        assert np.all(err <= bound), (l, (err / bound).max())
        # reconstruction is much better than using the anchor alone
        assert err.mean() < 0.5 * np.linalg.norm(xs[l] - a_hat, axis=-1).mean()


def test_chained_equals_shared_on_loop_next_to_anchor_and_for_two_loops():
    wl = synth.WORKLOADS["int2g16_b4_t16384"]
    rot = synth.haar_rotations(1, 128, 4)[0, 1].double().numpy()
    xs = _loops(22, 128, 128)
    sh = RQ.encode(xs, rot, _cfg(wl, chained=False, batch=1, ctx=128))
    ch = RQ.encode(xs, rot, _cfg(wl, chained=True, batch=1, ctx=128))
    for a, b in zip(sh.anchor, ch.anchor):
        assert np.array_equal(a, b)
    for a, b in zip(sh.resid[2], ch.resid[2]):
        assert np.array_equal(a, b)
    # the other loops differ (they reference rebuilt neighbours)
    assert not np.array_equal(sh.resid[0][0], ch.resid[0][0])
    xs2 = xs[2:]
    sh2 = RQ.encode(xs2, rot, _cfg(wl, chained=False, batch=1, ctx=128, L=2))
    ch2 = RQ.encode(xs2, rot, _cfg(wl, chained=True, batch=1, ctx=128, L=2))
    for a, b in zip(sh2.resid[0], ch2.resid[0]):
        assert np.array_equal(a, b)


def test_storage_accounting_matches_worked_example():
    with open(os.path.join(GOLDEN, "storage_worked_example.json")) as f:
        gold = json.load(f)
    wl = synth.WORKLOADS["ouro_b4_t8192"]
    cfg = _cfg(wl)
    lay = RQ.Layout(cfg)
    a, r = lay.bytes_per_token_head()
    assert (a, r) == (72, 42)            # 64 B codes + 8 B FP8 meta; 32 B codes + 8 B meta + 2 B c
    L = cfg.loops_per_group
    code_bits = cfg.anchor_bits + (L - 1) * cfg.resid_bits
    assert code_bits == gold["rq_code_bits_all_loops"]
    assert 16 * L == gold["bf16_bits_all_loops"]
    assert code_bits / L == gold["bits_per_element_before_metadata"]
    assert 16 * L / code_bits == gold["ratio_before_metadata"]
    bits = 8 * (a + (L - 1) * r) / cfg.head_dim      # stored bits per element position, all loops
    assert bits == 12.375
    assert round(16 * L / bits, 1) == gold["ratio_with_metadata_rounded_1dp"]
    assert round(100 * (1 - bits / (16 * L)), 1) == gold["storage_cut_percent_rounded_1dp"]
    # whole-cache size: 198 B per token per KV head per K|V at 64-token tiles
    assert lay.n_tiles == 129            # 8192 context tokens + the current one
    assert lay.total_bytes == 4 * 16 * 2 * 129 * (4608 + 3 * 2688)


def test_layout_byte_counts_other_configs():
    lay3 = RQ.Layout(_cfg(synth.WORKLOADS["int2g16_b4_t16384"]))
    assert lay3.bytes_per_token_head() == (48, 50)
    assert (lay3.a_tile, lay3.r_tile) == (3072, 3200)
    lay0 = RQ.Layout(_cfg(synth.WORKLOADS["tiny_d64_t256"]))
    assert lay0.bytes_per_token_head() == (36, 22)
    assert (lay0.a_tile, lay0.r_tile) == (2304, 1408)


def test_layout_hand_built_token_bytes():
    cfg = RQ.Config(64, 32, 4, 2, 2, 1, False, 1, 1, 1, 64)
    lay = RQ.Layout(cfg)
    cache = np.zeros(lay.total_bytes, dtype=np.uint8)
    qa = np.arange(64)[None, :] % 16
    qr = np.arange(64)[None, :] % 4
    enc = RQ.Encoded((qa, np.array([[-1.0, 0.5]]), np.array([[0.125, 2.0 ** -9]])),
                     [(qr, np.array([[0.0, -0.25]]), np.array([[1.0, 448.0]]), np.array([0.75]))])
    RQ.write_tokens(cache, lay, 0, 0, 0, 0, np.array([5]), enc)
    a_off = lay.plane_offset(0, 0, 0, 1)
    r_off = lay.plane_offset(0, 0, 0, 0)
    assert r_off == 0 and a_off == lay.n_tiles * lay.r_tile
    row = cache[a_off + 5 * 32: a_off + 6 * 32]
    assert list(row[:8]) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    meta = cache[a_off + 64 * 32 + 5 * 4: a_off + 64 * 32 + 6 * 4]
    assert list(meta) == [0xB8, 0x20, 0x30, 0x01]      # -1.0, 0.125, 0.5, 2^-9
    rrow = cache[r_off + 5 * 16: r_off + 6 * 16]
    assert list(rrow[:2]) == [0xE4, 0xE4]                # codes 0,1,2,3 at bits 0,2,4,6
    rmeta = cache[r_off + 64 * 16 + 5 * 4: r_off + 64 * 16 + 6 * 4]
    assert list(rmeta) == [0x00, 0x38, 0xA8, 0x7E]      # 0, 1.0, -0.25, 448
    cb = cache[r_off + 64 * 20 + 10: r_off + 64 * 20 + 12]
    assert list(cb) == [0x40, 0x3F]                      # BF16 0.75 = 0x3F40 little-endian
    back = RQ.read_tokens(cache, lay, 0, 0, 0, 0, 6)
    assert np.array_equal(back.anchor[0][5], qa[0]) and np.array_equal(back.resid[0][0][5], qr[0])
    assert back.resid[0][3][5] == 0.75


def test_pack_context_roundtrip_through_bytes():
    wl = synth.WORKLOADS["tiny_d64_t256"]
    inp = synth.generate(wl, seed=3)
    for chained in (False, True):
        cfg = _cfg(wl, chained=chained)
        kv = inp.kv.double().numpy()
        rot = inp.rot.double().numpy()
        cache = RQ.pack_context(kv, rot, cfg, wl.ctx + 1)
        lay = RQ.Layout(cfg)
        for h in range(2):
            for x in range(2):
                enc = RQ.encode(kv[0, :, x, 0, h, :wl.ctx + 1], rot[h, x], cfg)
                back = RQ.read_tokens(cache, lay, 0, h, x, 0, wl.ctx + 1)
                for a, b in zip(enc.anchor, back.anchor):
                    assert np.array_equal(a, b)
                for ra, rb in zip(enc.resid, back.resid):
                    for a, b in zip(ra, rb):
                        assert np.array_equal(a, b)
