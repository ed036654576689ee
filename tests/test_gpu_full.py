"""GPU parity at the full workload sizes, in the launch configuration the benchmark times
(automatic split count, every row at the full context), on sampled (row, KV head) pairs
that the float64 oracle can check one by one:

* the bulk-packed cache bytes of each sampled pair against the oracle's encoding rules;
* decode attention at every loop of the first, middle and last anchor groups, for every
  query head of the sampled KV heads, against the oracle's decode of the GPU's own bytes
  and of the oracle's own encoding;
* the current token that each loop-step writes into the BF16 pending buffer, and, after a
  group's anchor loop, the per-step pack of that finished token into the last slot of the
  cache (slot T, in the last tile), against the oracle's encoding rules;
* the BF16 baseline against float64 softmax attention on sampled heads.
"""
import numpy as np
import pytest
import torch

from looped_transformer_decode_amd import synth
from oracle import residualquant as RQ

from _support import (assert_stats, check_encoding, check_pack_block, close, device_block, gpu_pack, new_stats,
                      oracle_cfg, record_margin, say, slice_enc, sub_cache)

pytestmark = pytest.mark.gpu

FULL = [
    ("ouro_b4_t8192", False),
    ("ouro_b16_t8192", False),
    ("int2g16_b4_t16384", False),
    ("int2g16_b4_t16384", True),
    ("huginn_gqa4_b8_t8192", False),
    ("ouro_b4_t8192+widths422", False),     # residual widths 4, 2, 2 (more bits far from the anchor)
]
VARIANTS = {"widths422": dict(resid_bits_loop=(4, 2, 2))}


def _workload(name):
    base, _, var = name.partition("+")
    wl = synth.WORKLOADS[base]
    return wl.with_(name=name, **VARIANTS[var]) if var else wl


def _pairs(wl, rng):
    pairs = {(0, 0), (wl.batch - 1, wl.n_kv_heads - 1)}
    pairs.add((int(rng.integers(wl.batch)), int(rng.integers(wl.n_kv_heads))))
    return sorted(pairs)


def _loops(wl):
    L, G = wl.loops_per_group, wl.n_groups
    groups = sorted({0, G // 2, G - 1})
    return [k * L + l for k in groups for l in range(L)]


@pytest.mark.parametrize("name,chained", FULL, ids=[f"{n}{'_chained' if c else ''}" for n, c in FULL])
def test_full_size_parity(name, chained):
    from looped_transformer_decode_amd import binding as B
    wl = _workload(name).with_(chained=chained)
    T, L, d = wl.ctx, wl.loops_per_group, wl.head_dim
    gqa = wl.n_q_heads // wl.n_kv_heads
    say(f"[full] {name} chained={chained}: generating")
    inp = synth.generate(wl, seed=4242, device="cuda")
    cfg = B.config_for(wl)
    ocfg = oracle_cfg(wl)
    say(f"[full] {name} chained={chained}: bulk pack of {T} tokens")
    cache = gpu_pack(B, cfg, inp.kv, inp.rot, T)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    pairs = _pairs(wl, rng)
    rot = inp.rot.double().cpu().numpy()
    sc = synth.sm_scale(d)

    # current token of every loop, and the outputs of the sampled loops at the benchmark's split count
    loops = _loops(wl)
    ws = torch.zeros(B.rq_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    ctx_len = torch.full((wl.batch,), T, dtype=torch.int32, device="cuda")
    pending = torch.zeros(wl.batch, L, 2, wl.n_kv_heads, d, dtype=torch.bfloat16, device="cuda")
    outs = {}
    for loop in loops:
        grp, l = divmod(loop, L)
        out = torch.full((wl.batch, wl.n_q_heads, d), float("nan"), device="cuda")
        say(f"[full] {name} chained={chained}: decode loop {loop}")
        B.rq_decode_attention(cfg, cache, loop, inp.q[loop].contiguous(),
                              inp.kv[grp, l, 0, :, :, T].contiguous(), inp.kv[grp, l, 1, :, :, T].contiguous(),
                              pending, ctx_len, T, inp.rot, sc, out, ws, wl.batch, n_splits=0)
        torch.cuda.synchronize()
        outs[loop] = out.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(outs[loop]))
        if l == L - 1:
            # the pending buffer holds this group's current token of every loop; drain it into slot T
            assert torch.equal(pending, inp.kv[grp, :, :, :, :, T].permute(2, 0, 1, 3, 4))
            say(f"[full] {name} chained={chained}: per-step pack of group {grp} into slot {T}")
            B.rq_quantize_token(cfg, cache, pending, grp, ctx_len, inp.rot, wl.batch, 1)
            torch.cuda.synchronize()

    stats = new_stats()
    worst = 0.0
    for b, h in pairs:
        say(f"[full] {name} chained={chained}: oracle checks of row {b}, KV head {h}")
        kv = inp.kv[:, :, :, b, h].double().cpu().numpy()          # [G][L][2][T+1][d]
        block = device_block(cache, ocfg, b, h)
        _, sub = sub_cache(np.zeros(0, np.uint8), ocfg, b, h)
        xs = [[kv[k, :, x, :T] for x in range(2)] for k in range(wl.n_groups)]
        check_pack_block(block, sub, xs, rot[h], T, stats)
        for grp in sorted({lp // L for lp in loops}):
            for x in range(2):
                enc = RQ.read_tokens(block, RQ.Layout(sub), 0, 0, x, grp, T + 1)
                check_encoding(slice_enc(enc, slice(T, T + 1)), kv[grp, :, x, T:T + 1], rot[h, x], sub, stats)
        own = RQ.pack_context(kv[:, :, :, None, None], rot[h:h + 1], sub, T)
        lay = RQ.Layout(sub)
        for loop in loops:
            grp, l = divmod(loop, L)
            qh = inp.q[loop][b:b + 1, h * gqa:(h + 1) * gqa].double().cpu().numpy()
            kc, vc = kv[grp, l, 0, T][None, None], kv[grp, l, 1, T][None, None]
            ref_gpu = RQ.decode_attention(block, lay, loop, qh, kc, vc, [T], rot[h:h + 1], sc)
            ref_own = RQ.decode_attention(own, lay, loop, qh, kc, vc, [T], rot[h:h + 1], sc)
            o = outs[loop][b:b + 1, h * gqa:(h + 1) * gqa]
            e1, e2 = close(o, ref_gpu), close(o, ref_own)
            worst = max(worst, e1, e2)
            assert e1 <= 1.0 and e2 <= 1.0, (loop, b, h, e1, e2)
    say(f"[full] {name} chained={chained}: pack stats {stats}, worst err/bound {worst:.3f}")
    record_margin(f"full size {name}{' chained' if chained else ''}", worst)
    assert_stats(stats, wl.group)


@pytest.mark.parametrize("name", ["ouro_b4_t8192", "huginn_gqa4_b8_t8192"])
def test_bf16_full_size_parity(name):
    """The BF16 baseline at the full workload size, in the benchmark's launch configuration
    (automatic split count), with row lengths that end on a full tile, one token past it,
    mid-tile and at a single token, against float64 softmax attention on sampled heads."""
    from looped_transformer_decode_amd import binding as B
    wl = synth.WORKLOADS[name]
    T, d = wl.ctx, wl.head_dim
    gqa = wl.n_q_heads // wl.n_kv_heads
    say(f"[bf16 full] {name}: generating")
    g = torch.Generator().manual_seed(515)
    K = torch.randn(wl.batch, wl.n_kv_heads, T + 1, d, generator=g).to(torch.bfloat16)
    V = torch.randn(wl.batch, wl.n_kv_heads, T + 1, d, generator=g).to(torch.bfloat16)
    q = torch.randn(wl.batch, wl.n_q_heads, d, generator=g)
    lens = [T, T - 63, 4097, 1, T - 1, 65, 2048, 7][:wl.batch]
    Kd, Vd, qd = K.cuda(), V.cuda(), q.cuda()
    k_cur, v_cur = Kd[:, :, T].contiguous(), Vd[:, :, T].contiguous()
    bcfg = B.bf16_config_for(wl)
    ws = torch.zeros(B.rq_bf16_workspace_bytes(bcfg), dtype=torch.uint8, device="cuda")
    ctx_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = torch.full((wl.batch, wl.n_q_heads, d), float("nan"), device="cuda")
    sc = synth.sm_scale(d)
    say(f"[bf16 full] {name}: decode, rows {lens}")
    B.rq_bf16_decode_attention(bcfg, Kd, Vd, qd, k_cur, v_cur, False, ctx_len, T, sc, out, ws, wl.batch,
                               n_splits=0)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o))
    rng = np.random.default_rng(11)
    worst = 0.0
    for b in range(wl.batch):
        h = int(rng.integers(wl.n_kv_heads)) if 0 < b < wl.batch - 1 else (0 if b == 0 else wl.n_kv_heads - 1)
        n = lens[b]
        keys = np.concatenate([K[b, h, :n].double().numpy(), K[b, h, T][None].double().numpy()])
        vals = np.concatenate([V[b, h, :n].double().numpy(), V[b, h, T][None].double().numpy()])
        for hq in range(h * gqa, (h + 1) * gqa):
            ref = RQ.attention(q[b, hq].double().numpy(), keys, vals, sc)
            e = close(o[b, hq][None], ref[None])
            worst = max(worst, e)
            assert e <= 1.0, (b, h, hq, n, e)
    say(f"[bf16 full] {name}: worst err/bound {worst:.2e}")
    record_margin(f"bf16 full size {name}", worst)
