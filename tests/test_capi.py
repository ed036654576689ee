"""Host-side checks of librq.so that need no GPU: every symbol declared in include/rq.h
is exported, the size queries agree with the oracle's byte layout, and invalid
arguments are rejected on the host with the documented status (nothing launched)."""
import ctypes
import os
import re

import pytest

from looped_transformer_decode_amd import synth
from oracle import residualquant as RQ

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "looped_transformer_decode_amd", "librq.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="librq.so not built")


@pytest.fixture(scope="module")
def B():
    from looped_transformer_decode_amd import binding
    return binding


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "rq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rq_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(B):
    lib = ctypes.CDLL(LIB)
    declared = _declared_symbols()
    assert len(declared) >= 7
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(B.EXPORTS)


def _oracle_cfg(wl, chained):
    return RQ.Config(wl.head_dim, wl.group, wl.anchor_bits, wl.resid_bits, wl.loops_per_group,
                     wl.n_groups, chained, wl.n_kv_heads, wl.n_q_heads, wl.batch, wl.ctx + 1)


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
@pytest.mark.parametrize("chained", [False, True])
def test_cache_bytes_match_oracle_layout(B, name, chained):
    wl = synth.WORKLOADS[name]
    if chained and wl.loops_per_group > 4:
        pytest.skip("chained needs L <= 4")
    cfg = B.config_for(wl, chained=chained)
    assert B.rq_cache_bytes(cfg) == RQ.Layout(_oracle_cfg(wl, chained)).total_bytes
    assert B.rq_workspace_bytes(cfg) > 0


def test_invalid_configs_have_no_size(B):
    wl = synth.WORKLOADS["ouro_b4_t8192"]
    for field, bad in (("head_dim", 96), ("group", 24), ("anchor_bits", 3), ("resid_bits", 3),
                       ("resid_bits", 8), ("loops_per_group", 1), ("loops_per_group", 17), ("n_q_heads", 17),
                       ("max_batch", 0), ("max_ctx", 0), ("scale_rule", 2), ("scale_rule", -1)):
        cfg = B.config_for(wl)
        setattr(cfg, field, bad)
        assert B.rq_cache_bytes(cfg) == 0, field
        assert B.rq_workspace_bytes(cfg) == 0, field
    cfg = B.config_for(wl.with_(loops_per_group=8), chained=True)
    assert B.rq_cache_bytes(cfg) == 0                    # chained reads at most 3 residual planes
    cfg = B.config_for(wl.with_(resid_bits=4), chained=True)
    assert B.rq_cache_bytes(cfg) == 0                    # 4-bit residuals: shared anchor only
    assert B.rq_bf16_workspace_bytes(B.rq_bf16_config(96, 1, 1, 1, 64)) == 0


@pytest.mark.parametrize("variant", [dict(resid_bits=4), dict(loops_per_group=16, loop_scale="uniform(0.8,1.0)"),
                                     dict(loops_per_group=8, loop_scale="uniform(0.8,1.0)"), dict(scale_rule=1),
                                     dict(group=16, anchor_bits=4, resid_bits=2)])
def test_variant_configs_match_oracle_layout(B, variant):
    """The precision, group-length and scale-rule settings are supported tuples whose cache
    size is the oracle layout's."""
    wl = synth.WORKLOADS["ouro_b4_t8192"].with_(**variant)
    cfg = B.config_for(wl)
    ocfg = RQ.Config(wl.head_dim, wl.group, wl.anchor_bits, wl.resid_bits, wl.loops_per_group, wl.n_groups,
                     False, wl.n_kv_heads, wl.n_q_heads, wl.batch, wl.ctx + 1, wl.scale_rule)
    assert B.rq_cache_bytes(cfg) == RQ.Layout(ocfg).total_bytes > 0


@pytest.mark.parametrize("widths", [(4, 2, 2), (4, 4, 2), (2, 2, 2), (2, 4, 2)])
def test_per_loop_widths_match_oracle_layout(B, widths):
    wl = synth.WORKLOADS["ouro_b4_t8192"].with_(resid_bits_loop=widths)
    cfg = B.config_for(wl)
    ocfg = RQ.Config(wl.head_dim, wl.group, wl.anchor_bits, wl.resid_bits, wl.loops_per_group, wl.n_groups,
                     False, wl.n_kv_heads, wl.n_q_heads, wl.batch, wl.ctx + 1, 0, widths)
    assert B.rq_cache_bytes(cfg) == RQ.Layout(ocfg).total_bytes > 0
    # the paged block holds one tile of every plane: the oracle's group bytes per tile
    assert B.rq_paged_block_bytes(cfg) == 16 * 2 * RQ.Layout(ocfg).group_bytes // RQ.Layout(ocfg).n_tiles


def test_invalid_per_loop_widths_are_rejected(B):
    wl = synth.WORKLOADS["ouro_b4_t8192"]
    for widths in ((3, 2, 2), (8, 2, 2), (2, 2, 2, 4), (-2, 2, 2)):
        cfg = B.config_for(wl.with_(resid_bits_loop=widths))
        assert B.rq_cache_bytes(cfg) == 0, widths
    assert B.rq_cache_bytes(B.config_for(wl.with_(resid_bits_loop=(4, 2, 2)), chained=True)) == 0
    assert B.rq_cache_bytes(B.config_for(wl.with_(resid_bits_loop=(2, 2, 2)), chained=True)) > 0


def test_status_strings(B):
    assert B.rq_status_str(0) == "ok"
    assert "workspace" in B.rq_status_str(4)


# Fake, 256-byte aligned device addresses: every call below must fail its host checks
# before touching them.
A = 0x7F0000000000


def _decode(B, cfg, **kw):
    args = dict(cache=A, loop=0, q=A, q_bf16=1, k_cur=A, v_cur=A, pending=None, ctx_len=A, ctx_bound=64,
                rot=A, sm_scale=0.1, out=A, ws=A, ws_bytes=1 << 40, batch=1, n_splits=0)
    args.update(kw)
    return B._lib.rq_decode_attention(ctypes.byref(cfg), args["cache"], args["loop"], args["q"],
                                      args["q_bf16"], args["k_cur"], args["v_cur"], args["pending"],
                                      args["ctx_len"], args["ctx_bound"], args["rot"], args["sm_scale"],
                                      args["out"], args["ws"], args["ws_bytes"], args["batch"],
                                      args["n_splits"], None)


def test_decode_attention_rejects_bad_arguments(B):
    wl = synth.WORKLOADS["ouro_b4_t8192"]
    cfg = B.config_for(wl)
    need = B.rq_workspace_bytes(cfg)
    assert _decode(B, B.rq_config()) == 2                # all-zero config: unsupported
    assert _decode(B, cfg, cache=None) == 1
    assert _decode(B, cfg, loop=4) == 1
    assert _decode(B, cfg, loop=-1) == 1
    assert _decode(B, cfg, batch=5) == 1
    assert _decode(B, cfg, ctx_bound=wl.ctx + 2) == 1
    assert _decode(B, cfg, n_splits=65) == 1
    assert _decode(B, cfg, sm_scale=0.0) == 1
    assert _decode(B, cfg, q_bf16=2) == 1
    assert _decode(B, cfg, q=A + 8) == 3
    assert _decode(B, cfg, pending=A + 4) == 3
    assert _decode(B, cfg, ws=None) == 4
    assert _decode(B, cfg, ws_bytes=need - 1) == 4


def test_noalloc_decode_rejects_bad_arguments_and_oversize(B):
    """The entry point without a workspace checks the same arguments, and rejects more than
    4096 (row, query head) pairs or an explicit split count whose records do not fit its 4 MiB,
    all on the host before looking up its device array."""
    f = B._lib.rq_decode_attention_noalloc

    def call(cfg, loop=0, q=A, batch=1, n_splits=0, ctx_bound=64):
        return f(ctypes.byref(cfg), A, loop, q, 1, A, A, None, A, ctx_bound, A, 0.1, A, batch, n_splits, None)

    wl = synth.WORKLOADS["ouro_b4_t8192"]
    cfg = B.config_for(wl)
    assert call(B.rq_config()) == 2
    assert call(cfg, loop=4) == 1
    assert call(cfg, batch=5) == 1
    assert call(cfg, q=A + 8) == 3
    assert call(cfg, n_splits=65) == 1
    # 4 rows x 16 heads x 64 splits x (2 * 128 + 4) floats = 4.26 MB > 4 MiB
    assert call(cfg, batch=4, n_splits=64) == 4
    big = B.config_for(wl.with_(batch=257))              # 257 x 16 = 4112 pairs > 4096
    assert call(big, batch=257) == 4


def test_quantize_token_rejects_bad_arguments(B):
    wl = synth.WORKLOADS["ouro_b4_t8192"]
    cfg = B.config_for(wl)
    f = B._lib.rq_quantize_token
    ok = dict(cache=A, pending=A, st=None, grp=0, pos=A, rot=A, batch=4, n=1)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(ctypes.byref(cfg), a["cache"], a["pending"], a["st"], a["grp"], a["pos"], a["rot"],
                 a["batch"], a["n"], None)

    assert call(cache=None) == 1
    assert call(grp=1) == 1
    assert call(batch=0) == 1
    assert call(batch=5) == 1
    assert call(n=0) == 1
    assert call(cache=A + 8) == 3
    assert call(pending=A + 1) == 3
    bad = (ctypes.c_int64 * 5)(1, 1, -1, 1, 1)
    assert call(st=bad) == 1
    bad = B.config_for(wl)
    bad.head_dim = 96
    assert f(ctypes.byref(bad), A, A, None, 0, A, A, 1, 1, None) == 2


def test_bf16_decode_rejects_bad_arguments(B):
    cfg = B.rq_bf16_config(128, 16, 16, 4, 8193)
    need = B.rq_bf16_workspace_bytes(cfg)
    f = B._lib.rq_bf16_decode_attention

    def call(cfg=cfg, k=A, v=A, q=A, ctx_bound=8192, ws=A, ws_bytes=1 << 40, batch=4):
        return f(ctypes.byref(cfg), k, v, q, 1, A, A, 0, A, ctx_bound, 0.1, A, ws, ws_bytes, batch, 0, None)

    assert call(k=None) == 1
    assert call(ctx_bound=8194) == 1
    assert call(batch=5) == 1
    assert call(q=A + 2) == 3
    assert call(ws_bytes=need - 1) == 4
    assert call(cfg=B.rq_bf16_config(128, 16, 24, 4, 8193)) == 2


def test_unpack_debug_rejects_bad_arguments(B):
    wl = synth.WORKLOADS["ouro_b4_t8192"]
    cfg = B.config_for(wl)
    f = B._lib.rq_unpack_debug

    def call(cfg=cfg, cache=A, loop=0, rot=A, t0=0, t1=64, batch=4, out=A):
        return f(ctypes.byref(cfg), cache, loop, rot, t0, t1, batch, out, None)

    assert call(cfg=B.rq_config()) == 2
    assert call(cache=None) == 1
    assert call(loop=4) == 1
    assert call(t0=-1) == 1
    assert call(t0=64, t1=64) == 1
    assert call(t1=wl.ctx + 2) == 1
    assert call(batch=5) == 1
    assert call(out=A + 4) == 3


def test_stream_read_rejects_bad_arguments(B):
    f = B._lib.rq_stream_read
    assert f(None, 1 << 20, A, 1 << 20, None) == 1
    assert f(A, 0, A, 1 << 20, None) == 1
    assert f(A, 100, A, 1 << 20, None) == 1
    assert f(A + 8, 1 << 20, A, 1 << 20, None) == 3
    assert f(A, 1 << 20, A, (1 << 20) - 1, None) == 4


def test_paged_entry_points_reject_bad_arguments(B):
    wl = synth.WORKLOADS["ouro_b4_t8192"]
    cfg = B.config_for(wl)
    tiles = (cfg.max_ctx + 63) // 64
    blk = B.rq_paged_block_bytes(cfg)
    # one block holds a tile of every (head, K|V, group, plane): 16 * 2 * (4608 + 3 * 2688) bytes
    assert blk == 16 * 2 * (4608 + 3 * 2688)
    bad = B.config_for(wl)
    bad.head_dim = 96
    assert B.rq_paged_block_bytes(bad) == 0
    fq = B._lib.rq_quantize_token_paged

    def q(n_blocks=8, table=A, stride=tiles, batch=4):
        return fq(ctypes.byref(cfg), A, n_blocks, table, stride, A, None, 0, A, A, batch, 1, None)

    assert q(n_blocks=0) == 1
    assert q(table=None) == 1
    assert q(stride=tiles - 1) == 1
    assert q(table=A + 2) == 3
    assert q(batch=5) == 1
    fd = B._lib.rq_decode_attention_paged

    def d(n_blocks=8, table=A, stride=tiles, loop=0):
        return fd(ctypes.byref(cfg), A, n_blocks, table, stride, loop, A, 1, A, A, None, A, 64, A, 0.1, A, A,
                  1 << 40, 1, 0, None)

    assert d(n_blocks=0) == 1
    assert d(stride=0) == 1
    assert d(table=A + 1) == 3
    assert d(loop=4) == 1


def test_kv_project_rejects_bad_arguments(B):
    wl = synth.WORKLOADS["ouro_b4_t8192"]
    cfg = B.config_for(wl)
    f = B._lib.rq_kv_project

    def call(cfg=cfg, x=A, stride=2048, hidden=2048, w=A, loop=0, k=A, v=A, pending=A, batch=4):
        return f(ctypes.byref(cfg), x, stride, hidden, w, loop, k, v, pending, batch, None)

    assert call(cfg=B.rq_config()) == 2
    assert call(x=None) == 1
    assert call(w=None) == 1
    assert call(k=None, v=None, pending=None) == 1
    assert call(loop=4) == 1
    assert call(loop=-1) == 1
    assert call(batch=0) == 1
    assert call(batch=5) == 1
    assert call(hidden=2000) == 1                   # not a multiple of 32
    assert call(hidden=16) == 1
    assert call(stride=1024) == 1                   # rows overlap
    assert call(stride=2052) == 3                   # rows not 16-byte aligned
    assert call(x=A + 8) == 3
    assert call(w=A + 2) == 3
    assert call(pending=A + 4) == 3
    big = B.config_for(wl, max_batch=80)
    assert call(cfg=big, batch=65) == 2             # more than four 16-row tiles


def test_kv_project_binding_rejects_wrong_shapes(B):
    """The binding refuses output tensors whose shape would let the kernel write past them
    (CPU tensors suffice: the checks run before any pointer reaches the library)."""
    import torch
    wl = synth.WORKLOADS["tiny_d64_t256"]
    cfg = B.config_for(wl, max_batch=2)
    bf = torch.bfloat16
    x = torch.zeros(2, 128, dtype=bf)
    w = torch.zeros(2, 2, 64, 128, dtype=bf)
    k = torch.zeros(2, 2, 64, dtype=bf)
    pend = torch.zeros(2, 4, 2, 2, 64, dtype=bf)
    with pytest.raises(ValueError):
        B.rq_kv_project(cfg, x, torch.zeros(2, 2, 64, 96, dtype=bf), 0, k, k, pend, 2)
    with pytest.raises(ValueError):
        B.rq_kv_project(cfg, x, w, 0, torch.zeros(1, 2, 64, dtype=bf), k, pend, 2)
    with pytest.raises(ValueError):
        B.rq_kv_project(cfg, x, w, 0, k, torch.zeros(2, 2, 32, dtype=bf), pend, 2)
    with pytest.raises(ValueError):
        B.rq_kv_project(cfg, x, w, 0, k, k, torch.zeros(2, 3, 2, 2, 64, dtype=bf), 2)
    with pytest.raises(ValueError):
        B.rq_kv_project(cfg, x, w, 0, k, k, pend, 3)
    with pytest.raises(ValueError):
        B.rq_kv_project(cfg, x.float(), w, 0, k, k, pend, 2)


@pytest.mark.parametrize("k", [128, 640, 1024, 2048, 3072, 4096, 5632, 8192, 16384])
def test_w4a4_sizes_follow_the_layouts(B, k):
    """Weight and activation bytes of any K that is a multiple of 128 up to 16384 follow the
    oracle's layouts; the workspace holds X, c, the activation rows and, for a K off the four
    fast sizes that needs more than one 4096-channel slice, the slices' partial products."""
    from oracle import w4a4 as W4
    n, m = 48, 10
    cfg = B.w4a4_config(k, n, m)
    assert B.rq_w4_weight_bytes(cfg) == W4.weight_bytes(n, k)
    assert B.rq_w4a4_act_bytes(cfg) == W4.act_bytes(m, k)
    r = lambda b: (b + 255) // 256 * 256
    base = r(m * (k // 32) * 4) + r(m * 4) + r(W4.act_bytes(m, k))
    splits = 1 if k in (1024, 2048, 3072, 4096) else -(-k // 4096)
    assert B.rq_w4a4_workspace_bytes(cfg) == base + (r(splits * m * n * 4) if splits > 1 else 0)


@pytest.mark.parametrize("k,n,m", [(0, 16, 1), (64, 16, 1), (1000, 16, 1), (16512, 16, 1), (1024, 8, 1),
                                   (1024, 16, 0), (1024, 16, 65)])
def test_w4a4_invalid_sizes_have_no_size(B, k, n, m):
    cfg = B.w4a4_config(k, n, m)
    assert B.rq_w4_weight_bytes(cfg) == 0 and B.rq_w4a4_workspace_bytes(cfg) == 0
