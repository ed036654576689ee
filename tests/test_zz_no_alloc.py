"""The decode entry point that allocates nothing (rq_decode_attention_noalloc) against the
one that takes a workspace (rq_decode_attention), through the C ABI: two calls in a row on
the same GPU, the second with a smaller input (fewer rows, shorter contexts, another loop),
each compared with the workspace entry point on the same inputs and with the oracle."""
import numpy as np
import pytest
import torch

from looped_transformer_decode_amd import synth
from oracle import residualquant as RQ

from _support import close, gpu_pack, say, setup_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from looped_transformer_decode_amd import binding
    return binding


def _call_pair(B, wl, inp, cfg, ocfg, ctx, T, loop, n_splits, tag):
    dev = inp.kv.device
    L, d = wl.loops_per_group, wl.head_dim
    grp, l = divmod(loop, L)
    cache = gpu_pack(B, cfg, inp.kv, inp.rot, T)
    ctx_len = torch.tensor(ctx, dtype=torch.int32, device=dev)
    k_cur = inp.kv[grp, l, 0, :, :, T].contiguous()
    v_cur = inp.kv[grp, l, 1, :, :, T].contiguous()
    q = inp.q[loop].contiguous()
    sc = synth.sm_scale(d)
    ws = torch.zeros(B.rq_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    outs, pends = [], []
    for which in ("workspace", "noalloc"):
        out = torch.full((wl.batch, wl.n_q_heads, d), float("nan"), device=dev)
        pend = torch.zeros(wl.batch, L, 2, wl.n_kv_heads, d, dtype=torch.bfloat16, device=dev)
        say(f"[noalloc] {tag} entry={which} batch={wl.batch} ctx={ctx} loop={loop} n_splits={n_splits}")
        if which == "workspace":
            B.rq_decode_attention(cfg, cache, loop, q, k_cur, v_cur, pend, ctx_len, T, inp.rot, sc, out, ws,
                                  wl.batch, n_splits=n_splits)
        else:
            B.rq_decode_attention_noalloc(cfg, cache, loop, q, k_cur, v_cur, pend, ctx_len, T, inp.rot, sc, out,
                                          wl.batch, n_splits=n_splits)
        torch.cuda.synchronize()
        outs.append(out)
        pends.append(pend)
    assert bool(torch.isfinite(outs[1]).all())
    # same kernels and split count: the same float32 results, bit for bit, and the same pending write
    assert torch.equal(outs[0], outs[1]), tag
    assert torch.equal(pends[0], pends[1]), tag
    kv = inp.kv.double().cpu().numpy()
    ref = RQ.decode_attention(cache.cpu().numpy(), RQ.Layout(ocfg), loop, q.double().cpu().numpy(),
                              kv[grp, l, 0, :, :, T], kv[grp, l, 1, :, :, T], ctx, inp.rot.double().cpu().numpy(), sc)
    err = close(outs[1].double().cpu().numpy(), ref)
    say(f"    err/bound vs oracle={err:.3f}")
    assert err <= 1.0


@pytest.mark.parametrize("n_splits", [0, 3])
def test_noalloc_matches_workspace_entry_on_two_calls(B, n_splits):
    wl0 = synth.WORKLOADS["ouro_b4_t8192"]
    wl, inp, cfg, ocfg, ctx, T = setup_case(B, wl0, False, 4, [300, 64, 1, 257], 2, 2, seed=21)
    _call_pair(B, wl, inp, cfg, ocfg, ctx, T, 0, n_splits, "call 1")
    # second call: fewer rows, shorter contexts, the anchor loop
    wl, inp, cfg, ocfg, ctx, T = setup_case(B, wl0, False, 2, [100, 40], 2, 2, seed=22)
    _call_pair(B, wl, inp, cfg, ocfg, ctx, T, 3, n_splits, "call 2")


def test_noalloc_grouped_queries(B):
    """The grouped-query kernel (4 query heads per KV head) takes its records from the same
    static array."""
    wl0 = synth.WORKLOADS["huginn_gqa4_b8_t8192"].with_(n_groups=2)
    wl, inp, cfg, ocfg, ctx, T = setup_case(B, wl0, False, 2, [190, 77], 2, 8, seed=23)
    _call_pair(B, wl, inp, cfg, ocfg, ctx, T, 5, 0, "gqa call 1")
    wl, inp, cfg, ocfg, ctx, T = setup_case(B, wl0, False, 1, [70], 2, 8, seed=24)
    _call_pair(B, wl, inp, cfg, ocfg, ctx, T, 2, 0, "gqa call 2")


def test_noalloc_rejects_sizes_beyond_its_array(B):
    """More (row, query head) pairs than the array holds counters for, or an explicit split
    count whose records do not fit: RQ_ERR_WORKSPACE before anything is launched."""
    dev = torch.device("cuda")
    wl = synth.WORKLOADS["ouro_b4_t8192"].with_(batch=300, n_kv_heads=16, n_q_heads=16, ctx=64)
    cfg = B.config_for(wl)
    d = wl.head_dim
    cache = torch.zeros(16, dtype=torch.uint8, device=dev)          # never read: rejected first
    q = torch.zeros(wl.batch, wl.n_q_heads, d, dtype=torch.bfloat16, device=dev)
    kc = torch.zeros(wl.batch, wl.n_kv_heads, d, dtype=torch.bfloat16, device=dev)
    ctx_len = torch.zeros(wl.batch, dtype=torch.int32, device=dev)
    rot = torch.zeros(wl.n_kv_heads, 2, d, d, device=dev)
    out = torch.zeros(wl.batch, wl.n_q_heads, d, device=dev)
    with pytest.raises(B.RQError) as e:
        B.rq_decode_attention_noalloc(cfg, cache, 0, q, kc, kc, None, ctx_len, 64, rot, 0.1, out, wl.batch)
    assert "workspace" in str(e.value)
    # 64 rows x 16 heads x 64 splits x 1040 B = 68 MB of records: too many splits
    with pytest.raises(B.RQError):
        B.rq_decode_attention_noalloc(cfg, cache, 0, q[:64], kc[:64], kc[:64], None, ctx_len[:64], 64, rot, 0.1,
                                      out[:64], 64, n_splits=64)
