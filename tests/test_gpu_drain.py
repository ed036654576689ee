"""The per-step drain (a few finished tokens, shared anchor) has two kernels: one residual
loop per workgroup while its workgroups fit one round on the chip, else every residual loop
of a token per workgroup with R staged in LDS.  Both take the same float64 steps in the
same order, so their bytes must be identical: here 8 tokens packed in one call (enough
workgroups for the LDS kernel) are compared byte for byte with the same tokens packed by one
call per token (the one-loop kernel), and every code, FP8 offset/scale and c is checked
against the oracle's rules."""
import numpy as np
import pytest
import torch

from looped_transformer_decode_amd import synth

from _support import check_pack_block, device_block, new_stats, oracle_cfg, pending_strides, say, assert_stats, \
    sub_cache

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
U = "uniform(0.8,1.0)"
N_TOK = 8
CASES = {
    # name: (workload, batch, n_kv_heads)
    "d128g32_L4": (W["ouro_b4_t8192"], 4, 16),
    "d128g32_L2": (W["ouro_b4_t8192"].with_(loops_per_group=2, loop_scale=U), 4, 16),
    "d128g32_two_groups": (W["ouro_b4_t8192"].with_(n_groups=2), 3, 16),
    "d64g16_L8_int4": (W["tiny_d64_t256"].with_(group=16, loops_per_group=8, resid_bits=4, loop_scale=U), 4, 8),
    "d128g16_widths_422_norm_ratio": (W["int2g16_b4_t16384"].with_(anchor_bits=4, scale_rule=1,
                                                                   resid_bits_loop=(4, 2, 2)), 4, 16),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_drain_kernels_agree(name):
    from looped_transformer_decode_amd import binding as B
    wl, batch, hkv = CASES[name]
    wl = wl.with_(batch=batch, ctx=N_TOK, chained=False, n_kv_heads=hkv, n_q_heads=hkv)
    L = wl.loops_per_group
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    # the one-call pack takes the LDS kernel, the per-token packs the one-loop kernel
    assert L <= 8 and N_TOK * batch * hkv * 2 * (L - 1) > 3 * n_cu
    assert batch * hkv * 2 * (L - 1) <= 3 * n_cu
    inp = synth.generate(wl, seed=606, device="cuda")
    cfg = B.config_for(wl)
    ocfg = oracle_cfg(wl)
    one_call = torch.zeros(B.rq_cache_bytes(cfg), dtype=torch.uint8, device="cuda")
    per_tok = torch.zeros_like(one_call)
    say(f"[drain] case={name} batch={batch} hkv={hkv} L={L}: {N_TOK} tokens in one call")
    for grp in range(wl.n_groups):
        kv = inp.kv[grp]
        pos = torch.zeros(batch, dtype=torch.int32, device="cuda")
        B.rq_quantize_token(cfg, one_call, kv, grp, pos, inp.rot, batch, N_TOK, pending_strides=pending_strides(kv))
    say(f"[drain] case={name}: one call per token")
    for grp in range(wl.n_groups):
        for t in range(N_TOK):
            kv = inp.kv[grp, :, :, :, :, t:t + 1]
            pos = torch.full((batch,), t, dtype=torch.int32, device="cuda")
            B.rq_quantize_token(cfg, per_tok, kv, grp, pos, inp.rot, batch, 1, pending_strides=pending_strides(kv))
    torch.cuda.synchronize()
    assert torch.equal(one_call, per_tok), int((one_call != per_tok).sum())
    kvd = inp.kv.double().cpu().numpy()
    rot = inp.rot.double().cpu().numpy()
    stats = new_stats()
    _, sub = sub_cache(np.zeros(0, np.uint8), ocfg, 0, 0)
    for b in range(batch):
        for h in range(hkv):
            xs = [[kvd[k, :, x, b, h, :N_TOK] for x in range(2)] for k in range(wl.n_groups)]
            check_pack_block(device_block(one_call, ocfg, b, h), sub, xs, rot[h], N_TOK, stats)
    say(f"[drain] case={name} stats={stats}")
    assert_stats(stats, wl.group)


def test_drain_through_block_tables():
    """The LDS drain kernel through a shuffled block table: the gathered bytes equal the
    contiguous drain of the same tokens."""
    from looped_transformer_decode_amd import binding as B
    from test_gpu_paged import gather
    wl, batch, hkv = CASES["d128g32_L4"]
    wl = wl.with_(batch=batch, ctx=N_TOK, chained=False, n_kv_heads=hkv, n_q_heads=hkv)
    inp = synth.generate(wl, seed=607, device="cuda")
    cfg = B.config_for(wl)
    ocfg = oracle_cfg(wl)
    n_tiles = (cfg.max_ctx + 63) // 64
    n_blocks = batch * n_tiles + 3
    table_np = np.random.default_rng(5).permutation(n_blocks)[: batch * n_tiles].reshape(batch, n_tiles)
    table = torch.from_numpy(table_np.astype(np.int32)).to("cuda")
    bb = B.rq_paged_block_bytes(cfg)
    pool = torch.zeros(n_blocks * bb, dtype=torch.uint8, device="cuda")
    flat = torch.zeros(B.rq_cache_bytes(cfg), dtype=torch.uint8, device="cuda")
    pos = torch.zeros(batch, dtype=torch.int32, device="cuda")
    say(f"[drain] paged: batch={batch} hkv={hkv} blocks={n_blocks}")
    kv = inp.kv[0]
    B.rq_quantize_token_paged(cfg, pool, n_blocks, table, kv, 0, pos, inp.rot, batch, N_TOK,
                              pending_strides=pending_strides(kv))
    B.rq_quantize_token(cfg, flat, kv, 0, pos, inp.rot, batch, N_TOK, pending_strides=pending_strides(kv))
    torch.cuda.synchronize()
    assert np.array_equal(gather(pool.cpu().numpy(), table_np, ocfg, bb), flat.cpu().numpy())


def test_drain_past_max_ctx():
    """Tokens whose slot lies past max_ctx are skipped by the LDS drain kernel as by the
    one-loop kernel: 8 tokens from slot max_ctx - 3, in one call and one call per token, give
    the same bytes, and the slots before the first token stay untouched."""
    from looped_transformer_decode_amd import binding as B
    wl, batch, hkv = CASES["d128g32_L4"]
    wl = wl.with_(batch=batch, ctx=N_TOK, chained=False, n_kv_heads=hkv, n_q_heads=hkv)
    inp = synth.generate(wl, seed=608, device="cuda")
    cfg = B.config_for(wl)
    p0 = cfg.max_ctx - 3
    one_call = torch.full((B.rq_cache_bytes(cfg),), 0x5A, dtype=torch.uint8, device="cuda")
    per_tok = one_call.clone()
    untouched = one_call.clone()
    kv = inp.kv[0]
    say(f"[drain] past max_ctx: first slot {p0}, max_ctx {cfg.max_ctx}")
    B.rq_quantize_token(cfg, one_call, kv, 0, torch.full((batch,), p0, dtype=torch.int32, device="cuda"), inp.rot,
                        batch, N_TOK, pending_strides=pending_strides(kv))
    for t in range(N_TOK):
        kt = inp.kv[0, :, :, :, :, t:t + 1]
        B.rq_quantize_token(cfg, per_tok, kt, 0, torch.full((batch,), p0 + t, dtype=torch.int32, device="cuda"),
                            inp.rot, batch, 1, pending_strides=pending_strides(kt))
    torch.cuda.synchronize()
    assert torch.equal(one_call, per_tok)
    # only the three token rows at slots p0 .. max_ctx - 1 changed: the rest of every tile keeps 0x5A
    changed = int((one_call != untouched).sum())
    assert 0 < changed <= 3 * batch * hkv * 2 * (72 + 3 * (40 + 2)), changed


@pytest.mark.parametrize("kind", ["zero", "constant", "large", "zero_anchor"])
def test_drain_kernels_agree_on_edge_inputs(kind):
    """Degenerate inputs through both drain kernels: all zeros (zero anchor, c = 0, zero ranges),
    one constant per vector (zero group ranges, the smallest scale), values near the E4M3 range
    (offsets at -448, scales near 448) and a zero anchor under nonzero loops (c = 0, the residual
    is R x).  The bytes must be identical and the encoding follow the oracle's rules."""
    from looped_transformer_decode_amd import binding as B
    wl, batch, hkv = CASES["d128g32_L4"]
    wl = wl.with_(batch=batch, ctx=N_TOK, chained=False, n_kv_heads=hkv, n_q_heads=hkv)
    inp = synth.generate(wl, seed=609, device="cuda")
    kv = inp.kv
    if kind == "zero":
        kv.zero_()
    elif kind == "constant":
        kv.copy_(torch.linspace(-3.0, 3.0, kv.shape[5], device="cuda").view(1, 1, 1, 1, 1, -1, 1).expand_as(kv))
    elif kind == "large":
        kv.copy_((kv.float().clamp(-1.0, 1.0) * 380.0).to(kv.dtype))
    else:
        kv[:, wl.loops_per_group - 1].zero_()
    cfg = B.config_for(wl)
    ocfg = oracle_cfg(wl)
    one_call = torch.zeros(B.rq_cache_bytes(cfg), dtype=torch.uint8, device="cuda")
    per_tok = torch.zeros_like(one_call)
    say(f"[drain] edge inputs: {kind}")
    k0 = kv[0]
    B.rq_quantize_token(cfg, one_call, k0, 0, torch.zeros(batch, dtype=torch.int32, device="cuda"), inp.rot, batch,
                        N_TOK, pending_strides=pending_strides(k0))
    for t in range(N_TOK):
        kt = kv[0, :, :, :, :, t:t + 1]
        B.rq_quantize_token(cfg, per_tok, kt, 0, torch.full((batch,), t, dtype=torch.int32, device="cuda"), inp.rot,
                            batch, 1, pending_strides=pending_strides(kt))
    torch.cuda.synchronize()
    assert torch.equal(one_call, per_tok)
    kvd = kv.double().cpu().numpy()
    rot = inp.rot.double().cpu().numpy()
    stats = new_stats()
    _, sub = sub_cache(np.zeros(0, np.uint8), ocfg, 0, 0)
    for b in range(batch):
        for h in range(0, hkv, 5):
            xs = [[kvd[0, :, x, b, h, :N_TOK] for x in range(2)]]
            check_pack_block(device_block(one_call, ocfg, b, h), sub, xs, rot[h], N_TOK, stats)
    say(f"[drain] edge {kind} stats={stats}")
    assert_stats(stats, wl.group)
