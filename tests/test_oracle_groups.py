"""Pins of the oracle's grouped-anchor path (several anchor groups per layer).

The digest's Huginn-3.5B setting runs 32 loops as 8 groups of 4: the last loop of each
group is that group's anchor and the group's other loops are residuals against it.  The
oracle handles this with the group term of ``Layout.plane_offset``, the group loop of
``pack_context`` and the ``divmod(loop, L)`` group selection of ``decode_attention``.
These tests pin each of them against something other than the oracle's own formula:
literal byte offsets worked out by hand, the non-overlap of every plane, a direct
``encode`` of each group's own data, and plain softmax attention (torch's) over values
that the quantizer reproduces exactly.  Each group is given different data, so a group
index that is dropped anywhere (every loop reading group 0, say) fails them."""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

from looped_transformer_decode_amd import synth
from oracle import residualquant as RQ


def _sdpa(q, keys, values, scale, gqa=1):
    qt = torch.from_numpy(np.asarray(q, np.float64))[:, :, None, :]
    k = torch.from_numpy(np.asarray(keys, np.float64)).repeat_interleave(gqa, dim=1)
    v = torch.from_numpy(np.asarray(values, np.float64)).repeat_interleave(gqa, dim=1)
    return Fnn.scaled_dot_product_attention(qt, k, v, scale=scale)[:, :, 0, :].numpy()


def test_plane_offsets_of_three_groups_by_hand():
    """d = 64, g = 32, INT4 anchor / INT2 residuals, L = 4, 3 groups, 2 KV heads, 2 rows,
    100 slots (2 tiles of 64 tokens).  By hand:
      anchor tile   = 64 * (32 B codes + 4 B meta)          = 2304 B
      residual tile = 64 * (16 B codes + 4 B meta + 2 B c)  = 1408 B
      one group     = 2 tiles * (2304 + 3 * 1408)           = 13056 B
      one block     = 3 groups * 13056                      = 39168 B
      cache         = 2 rows * 2 heads * 2 (K|V) * 39168    = 313344 B"""
    cfg = RQ.Config(64, 32, 4, 2, 4, 3, False, 2, 2, 2, 100)
    lay = RQ.Layout(cfg)
    assert (lay.a_tile, lay.r_tile, lay.group_bytes, lay.block_bytes, lay.total_bytes) == \
        (2304, 1408, 13056, 39168, 313344)
    # (b, h, x, global loop) -> offset
    # block index ((b*2 + h)*2 + x); group k = loop // 4; local loop l = loop % 4, whose plane
    # follows the l residual planes (2 tiles of 1408 B each) before it in its group
    cases = {
        (0, 0, 0, 0): 0,
        (0, 0, 0, 3): 3 * 2816,                               # group 0's anchor plane
        (0, 0, 0, 4): 13056,                                  # group 1, loop 0
        (1, 0, 1, 5): 5 * 39168 + 13056 + 2816,               # block 5, group 1, loop 1
        (0, 1, 0, 11): 2 * 39168 + 2 * 13056 + 3 * 2816,      # block 2, group 2's anchor
        (1, 1, 1, 10): 7 * 39168 + 2 * 13056 + 2 * 2816,      # last block, group 2, loop 2
    }
    for key, off in cases.items():
        assert lay.plane_offset(*key) == off, key
    assert cases[(1, 0, 1, 5)] == 211712 and cases[(0, 1, 0, 11)] == 112896


def test_planes_of_every_group_tile_the_cache_exactly():
    """Every (row, head, K|V, loop) plane has its own byte range; together they cover the
    cache once.  An offset that ignores the group would make groups overlap."""
    cfg = RQ.Config(128, 32, 4, 2, 4, 8, False, 3, 12, 2, 200)
    lay = RQ.Layout(cfg)
    cover = np.zeros(lay.total_bytes, dtype=np.int32)
    for b in range(2):
        for h in range(3):
            for x in range(2):
                for loop in range(cfg.n_loops):
                    size = lay.n_tiles * (lay.a_tile if loop % 4 == 3 else lay.r_tile)
                    off = lay.plane_offset(b, h, x, loop)
                    cover[off: off + size] += 1
    assert np.all(cover == 1)


def _grouped_inputs(seed, n_groups, L, B, Hkv, T, d):
    """Synthetic loops whose groups all differ: each group has its own anchor draw."""
    wl = synth.WORKLOADS["tiny_d64_t256"].with_(n_groups=n_groups, loops_per_group=L,
                                                 loop_scale="uniform(0.8,1.0)", n_kv_heads=Hkv,
                                                 n_q_heads=Hkv, head_dim=d)
    inp = synth.generate(wl, seed=seed, batch=B, ctx=T)
    return inp.kv.double().numpy(), inp.rot.double().numpy()


@pytest.mark.parametrize("chained", [False, True])
def test_pack_context_stores_each_groups_own_encoding(chained):
    n_groups, L, B, Hkv, T, d = 3, 4, 2, 2, 70, 64
    kv, rot = _grouped_inputs(40, n_groups, L, B, Hkv, T, d)
    cfg = RQ.Config(d, 32, 4, 2, L, n_groups, chained, Hkv, Hkv, B, T + 1)
    lay = RQ.Layout(cfg)
    cache = RQ.pack_context(kv, rot, cfg, T)
    for b in range(B):
        for h in range(Hkv):
            for x in range(2):
                encs = []
                for k in range(n_groups):
                    direct = RQ.encode(kv[k, :, x, b, h, :T], rot[h, x], cfg)
                    back = RQ.read_tokens(cache, lay, b, h, x, k, T)
                    for u, v in zip(direct.anchor, back.anchor):
                        assert np.array_equal(u, v), (b, h, x, k)
                    for ru, rv in zip(direct.resid, back.resid):
                        for u, v in zip(ru, rv):
                            assert np.array_equal(u, v), (b, h, x, k)
                    encs.append(back)
                # the groups' stored encodings differ from each other
                for k in range(1, n_groups):
                    assert not np.array_equal(encs[k].anchor[0], encs[0].anchor[0])


@pytest.mark.parametrize("chained", [False, True])
def test_grouped_decode_equals_single_group_run_on_that_group(chained):
    """decode_attention at global loop k*L + l of a 3-group cache equals a one-group oracle
    run, at loop l, on group k's K/V alone (its own cache, packed separately)."""
    n_groups, L, B, Hkv, T, d = 3, 4, 1, 2, 90, 64
    gqa = 2
    kv, rot = _grouped_inputs(41, n_groups, L, B, Hkv, T, d)
    cfg = RQ.Config(d, 32, 4, 2, L, n_groups, chained, Hkv, Hkv * gqa, B, T + 1)
    cfg1 = RQ.Config(d, 32, 4, 2, L, 1, chained, Hkv, Hkv * gqa, B, T + 1)
    cache = RQ.pack_context(kv, rot, cfg, T)
    rng = np.random.default_rng(42)
    q = rng.normal(size=(n_groups * L, B, Hkv * gqa, d))
    outs = {}
    for k in range(n_groups):
        single = RQ.pack_context(kv[k:k + 1], rot, cfg1, T)
        for l in range(L):
            loop = k * L + l
            kc, vc = kv[k, l, 0, :, :, T], kv[k, l, 1, :, :, T]
            o = RQ.decode_attention(cache, RQ.Layout(cfg), loop, q[loop], kc, vc, [T], rot, 0.125)
            o1 = RQ.decode_attention(single, RQ.Layout(cfg1), l, q[loop], kc, vc, [T], rot, 0.125)
            assert np.array_equal(o, o1), (k, l)
            outs[(k, l)] = o
    # with the same query, the same local loop of two groups gives different outputs
    kc, vc = kv[0, 1, 0, :, :, T], kv[0, 1, 1, :, :, T]
    o_g0 = RQ.decode_attention(cache, RQ.Layout(cfg), 1, q[1], kc, vc, [T], rot, 0.125)
    o_g2 = RQ.decode_attention(cache, RQ.Layout(cfg), 2 * L + 1, q[1], kc, vc, [T], rot, 0.125)
    assert np.abs(o_g0 - o_g2).max() > 1e-3


@pytest.mark.parametrize("chained", [False, True])
def test_grouped_lossless_construction_is_plain_attention_over_that_group(chained):
    """Each group's anchor lies on the INT4 grid (z = -1, s = 1/8, codes 0..15 with both ends
    present in every channel group) and the group's other loops equal its anchor, so
    c = 1, the residual is zero and the group is stored without loss.  Attention at global
    loop k*L + l must then be torch's softmax attention over group k's values (and not over
    any other group's: each group draws its own codes)."""
    rng = np.random.default_rng(43)
    n_groups, L, B, Hkv, T, d, gqa = 3, 4, 2, 2, 80, 64, 2
    codes = rng.integers(0, 16, size=(n_groups, 2, B, Hkv, T + 1, d))
    codes[..., 0::32] = 0
    codes[..., 1::32] = 15
    vals = -1.0 + codes / 8.0
    kv = np.broadcast_to(vals[:, None], (n_groups, L) + vals.shape[1:]).copy()
    rot = synth.haar_rotations(Hkv, d, 44).double().numpy()
    cfg = RQ.Config(d, 32, 4, 2, L, n_groups, chained, Hkv, Hkv * gqa, B, T + 1)
    cache = RQ.pack_context(kv, rot, cfg, T)
    lay = RQ.Layout(cfg)
    q = rng.normal(size=(B, Hkv * gqa, d))
    ctx = [T, 51]
    for k in range(n_groups):
        for l in (0, L - 1):
            loop = k * L + l
            kc, vc = kv[k, l, 0, :, :, T], kv[k, l, 1, :, :, T]
            o = RQ.decode_attention(cache, lay, loop, q, kc, vc, ctx, rot, 0.125)
            for b in range(B):
                n = ctx[b]
                keys = np.concatenate([vals[k, 0, b:b + 1, :, :n], kc[b:b + 1, :, None]], axis=2)
                values = np.concatenate([vals[k, 1, b:b + 1, :, :n], vc[b:b + 1, :, None]], axis=2)
                ref = _sdpa(q[b:b + 1], keys, values, 0.125, gqa=gqa)
                assert np.allclose(o[b], ref[0], rtol=1e-12, atol=1e-13), (k, l, b)
