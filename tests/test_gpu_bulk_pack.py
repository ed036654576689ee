"""GPU parity of the many-token pack paths (16 tokens per workgroup, used for 16 or more
tokens) on the cases the default workloads do not reach.  Shared anchor: 2, 6 and 8 loops
per anchor group (one, two and three residual batches of the rotation product, the last
one partial), head_dim 64 and 128, INT4 and INT2 anchors.  Chained: 2, 3 and 4 loops per
group (one to three links of the chain), head_dim 64 and 128, g = 16 and 32, both
coefficient rules, a start slot that is not a multiple of 16.  Both: a token count that
is not a multiple of 16, and a start slot so close to max_ctx that the last tokens have no
slot (they must be skipped: nothing written, nothing else touched).  Every stored code,
FP8 offset/scale and c is checked against the float64 oracle under the parity rules."""
import numpy as np
import pytest
import torch

from looped_transformer_decode_amd import synth
from oracle import residualquant as RQ

from _support import (assert_stats, check_encoding, device_block, gpu_pack, new_stats, oracle_cfg, pending_strides,
                      say, slice_enc, sub_cache)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
U = "uniform(0.8,1.0)"
CASES = {
    # name: (workload, batch, tokens, n_kv_heads, first slot, max_ctx or None)
    "L2_d128g32": (W["ouro_b4_t8192"].with_(loops_per_group=2, loop_scale=U), 2, 100, 2, 0, None),
    "chained_L2_d128g32": (W["ouro_b4_t8192"].with_(loops_per_group=2, loop_scale=U, chained=True), 2, 100, 2, 0,
                           None),
    "chained_L3_d64g16_offset": (W["tiny_d64_t256"].with_(group=16, loops_per_group=3, loop_scale=U, chained=True), 2,
                                 45, 2, 5, None),
    "chained_L4_d128g32_past_max_ctx": (W["ouro_b4_t8192"].with_(chained=True), 2, 50, 1, 51, 96),
    "chained_norm_ratio_d64g32": (W["tiny_d64_t256"].with_(scale_rule=1, chained=True), 1, 70, 2, 0, None),
    "L6_d128g16int2": (W["int2g16_b4_t16384"].with_(loops_per_group=6, loop_scale=U), 1, 70, 2, 0, None),
    "L8_d64": (W["tiny_d64_t256"].with_(loops_per_group=8, loop_scale=U), 1, 40, 2, 0, None),
    "past_max_ctx": (W["ouro_b4_t8192"], 2, 50, 1, 51, 96),
    "L6_widths_d128g32": (W["ouro_b4_t8192"].with_(loops_per_group=6, loop_scale=U, resid_bits_loop=(4, 4, 2, 2, 2)),
                          2, 90, 2, 0, None),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_bulk_pack_parity(name):
    from looped_transformer_decode_amd import binding as B
    wl, batch, T, hkv, pos0, max_ctx = CASES[name]
    wl = wl.with_(batch=batch, ctx=T, n_kv_heads=hkv, n_q_heads=hkv)
    max_ctx = max_ctx or pos0 + T
    say(f"[bulk] case={name} tokens={T} first slot={pos0} max_ctx={max_ctx} L={wl.loops_per_group}")
    inp = synth.generate(wl, seed=321, device="cuda")
    cfg = B.config_for(wl, max_ctx=max_ctx)
    ocfg = oracle_cfg(wl, max_ctx=max_ctx)
    cache = gpu_pack(B, cfg, inp.kv, inp.rot, T, pos0=pos0)
    torch.cuda.synchronize()
    n = min(T, max_ctx - pos0)                      # tokens that have a slot
    kv = inp.kv.double().cpu().numpy()
    rot = inp.rot.double().cpu().numpy()
    stats = new_stats()
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            block = device_block(cache, ocfg, b, h)
            _, sub = sub_cache(np.zeros(0, np.uint8), ocfg, b, h)
            lay = RQ.Layout(sub)
            for k in range(wl.n_groups):
                for x in range(2):
                    enc = RQ.read_tokens(block, lay, 0, 0, x, k, pos0 + n)
                    check_encoding(slice_enc(enc, slice(pos0, pos0 + n)), kv[k, :, x, b, h, :n], rot[h, x], sub, stats)
                    if pos0 > 0:                    # slots before the first one are untouched
                        head = slice_enc(enc, slice(0, pos0))
                        assert not np.any(head.anchor[0]) and not np.any(head.anchor[1])
    say(f"[bulk] case={name} stats={stats}")
    assert_stats(stats, wl.group)


@pytest.mark.parametrize("chained", [False, True], ids=["shared", "chained"])
def test_bulk_pack_rows_start_at_their_own_slots(chained):
    """Each batch row packs from its own first slot (pos[b]): row 0 from slot 0, row 1 from
    slot 37, so that its 40 tokens straddle a 64-token tile boundary.  Every stored value is
    checked against the oracle, and the slots before a row's first one stay untouched."""
    from looped_transformer_decode_amd import binding as B
    wl = W["ouro_b4_t8192"].with_(batch=2, ctx=40, n_kv_heads=2, n_q_heads=2, chained=chained)
    T, starts = 40, [0, 37]
    max_ctx = max(starts) + T
    say(f"[bulk] rows from slots {starts}, {T} tokens, chained={chained}")
    inp = synth.generate(wl, seed=331, device="cuda")
    cfg = B.config_for(wl, max_ctx=max_ctx)
    ocfg = oracle_cfg(wl, max_ctx=max_ctx)
    cache = torch.zeros(B.rq_cache_bytes(cfg), dtype=torch.uint8, device="cuda")
    pos = torch.tensor(starts, dtype=torch.int32, device="cuda")
    for grp in range(wl.n_groups):
        B.rq_quantize_token(cfg, cache, inp.kv[grp], grp, pos, inp.rot, wl.batch, T,
                            pending_strides=pending_strides(inp.kv[grp]))
    torch.cuda.synchronize()
    kv = inp.kv.double().cpu().numpy()
    rot = inp.rot.double().cpu().numpy()
    stats = new_stats()
    for b, p0 in enumerate(starts):
        for h in range(wl.n_kv_heads):
            block = device_block(cache, ocfg, b, h)
            _, sub = sub_cache(np.zeros(0, np.uint8), ocfg, b, h)
            lay = RQ.Layout(sub)
            for k in range(wl.n_groups):
                for x in range(2):
                    enc = RQ.read_tokens(block, lay, 0, 0, x, k, p0 + T)
                    check_encoding(slice_enc(enc, slice(p0, p0 + T)), kv[k, :, x, b, h, :T], rot[h, x], sub, stats)
                    if p0 > 0:
                        head = slice_enc(enc, slice(0, p0))
                        assert not np.any(head.anchor[0]) and not np.any(head.anchor[1])
    say(f"[bulk] rows from their own slots stats={stats}")
    assert_stats(stats, wl.group)
