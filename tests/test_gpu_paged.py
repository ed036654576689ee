"""GPU parity of the paged cache (block tables): tiles live in a pool of 64-token blocks in
a shuffled order (plus blocks no row uses).  The pool is packed through the paged entry
points, gathered back into the contiguous layout on the host with the block table, and
then checked like the contiguous path:

* every code, FP8 offset/scale and c of the bulk-packed context against the oracle's
  encoding rules;
* decode attention at every loop, through the block table, against the oracle's decode of
  the gathered bytes, with ragged (and empty) contexts;
* the per-step drain of the current token into its slot through the block table.

The gathered bytes must also equal those of the contiguous pack of the same tokens, and
the paged decode must give the contiguous decode's outputs to the bit (same kernels, same
split count)."""
import numpy as np
import pytest
import torch

from looped_transformer_decode_amd import synth
from oracle import residualquant as RQ

from _support import (assert_stats, check_encoding, check_pack_block, close, gpu_pack, new_stats, oracle_cfg,
                      pending_strides, say, slice_enc, sub_cache)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
CASES = {
    # name: (workload, chained, batch, ctx_len per row, n_kv_heads, n_q_heads)
    "d128g32_ragged": (W["ouro_b4_t8192"], False, 3, [300, 0, 130], 2, 2),
    "d128g16int2_chained": (W["int2g16_b4_t16384"], True, 2, [65, 200], 2, 2),
    "gqa4_two_groups": (W["huginn_gqa4_b8_t8192"].with_(n_groups=2), False, 2, [190, 77], 2, 8),
    "d64": (W["tiny_d64_t256"], False, 1, [150], 2, 2),
    "widths_422_d128g32": (W["ouro_b4_t8192"].with_(resid_bits_loop=(4, 2, 2)), False, 2, [190, 64], 2, 2),
}


def gather(pool: np.ndarray, table: np.ndarray, cfg: RQ.Config, block_bytes: int) -> np.ndarray:
    """The contiguous cache that holds the tiles the block table points at."""
    lay = RQ.Layout(cfg)
    L, G = cfg.loops_per_group, cfg.n_groups
    g_tile = lay.a_tile + sum(lay.r_tiles)
    pre = [sum(lay.r_tiles[:l]) for l in range(L)]          # tile bytes before plane l in a block
    cache = np.zeros(lay.total_bytes, np.uint8)
    for b in range(cfg.max_batch):
        for t in range(lay.n_tiles):
            blk = int(table[b, t])
            for h in range(cfg.n_kv_heads):
                for x in range(2):
                    for k in range(G):
                        base = blk * block_bytes + ((h * 2 + x) * G + k) * g_tile
                        for l in range(L):
                            size = lay.a_tile if l == L - 1 else lay.r_tiles[l]
                            dst = lay.plane_offset(b, h, x, k * L + l) + t * size
                            cache[dst: dst + size] = pool[base + pre[l]: base + pre[l] + size]
    return cache


@pytest.mark.parametrize("name", sorted(CASES))
def test_paged_pack_and_decode(name):
    from looped_transformer_decode_amd import binding as B
    wl, chained, batch, ctx, hkv, hq = CASES[name]
    T = max(ctx)
    wl = wl.with_(batch=batch, ctx=T, chained=chained, n_kv_heads=hkv, n_q_heads=hq)
    say(f"[paged] case={name} T={T} ctx={ctx}")
    dev = torch.device("cuda")
    inp = synth.generate(wl, seed=555, device=dev)
    cfg = B.config_for(wl)
    ocfg = oracle_cfg(wl)
    n_tiles = (cfg.max_ctx + 63) // 64
    n_blocks = batch * n_tiles + 5
    rng = np.random.default_rng(11)
    table_np = rng.permutation(n_blocks)[: batch * n_tiles].reshape(batch, n_tiles).astype(np.int32)
    table = torch.from_numpy(table_np).to(dev)
    bb = B.rq_paged_block_bytes(cfg)
    pool = torch.zeros(n_blocks * bb, dtype=torch.uint8, device=dev)
    pos0 = torch.zeros(batch, dtype=torch.int32, device=dev)
    for grp in range(wl.n_groups):
        B.rq_quantize_token_paged(cfg, pool, n_blocks, table, inp.kv[grp], grp, pos0, inp.rot, batch, T,
                                  pending_strides=pending_strides(inp.kv[grp]))
    torch.cuda.synchronize()
    cache_np = gather(pool.cpu().numpy(), table_np, ocfg, bb)
    kv = inp.kv.double().cpu().numpy()
    rot = inp.rot.double().cpu().numpy()
    # the same tokens packed into the contiguous cache give the same bytes
    flat = gpu_pack(B, cfg, inp.kv, inp.rot, T)
    torch.cuda.synchronize()
    assert np.array_equal(flat.cpu().numpy(), cache_np), "paged pack differs from the contiguous pack"

    # the packed context
    stats = new_stats()
    for b in range(batch):
        for h in range(hkv):
            block, sub = sub_cache(cache_np, ocfg, b, h)
            xs = [[kv[k, :, x, b, h, :T] for x in range(2)] for k in range(wl.n_groups)]
            check_pack_block(block, sub, xs, rot[h], T, stats)
    say(f"[paged] case={name} pack stats {stats}")
    assert_stats(stats, wl.group)

    # decode at every loop through the block table, then the drain of the current token
    L, d = wl.loops_per_group, wl.head_dim
    lay = RQ.Layout(ocfg)
    ctx_len = torch.tensor(ctx, dtype=torch.int32, device=dev)
    ws = torch.zeros(B.rq_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    pending = torch.zeros(batch, L, 2, hkv, d, dtype=torch.bfloat16, device=dev)
    sc = synth.sm_scale(d)
    worst = 0.0
    for loop in range(wl.n_loops):
        grp, l = divmod(loop, L)
        q = inp.q[loop].contiguous()
        kc = torch.stack([inp.kv[grp, l, 0, b, :, ctx[b]] for b in range(batch)]).contiguous()
        vc = torch.stack([inp.kv[grp, l, 1, b, :, ctx[b]] for b in range(batch)]).contiguous()
        out = torch.full((batch, hq, d), float("nan"), device=dev)
        B.rq_decode_attention_paged(cfg, pool, n_blocks, table, loop, q, kc, vc, pending, ctx_len, T, inp.rot, sc,
                                    out, ws, batch)
        out_flat = torch.full_like(out, float("nan"))
        B.rq_decode_attention(cfg, flat, loop, q, kc, vc, None, ctx_len, T, inp.rot, sc, out_flat, ws, batch)
        torch.cuda.synchronize()
        # same kernel arithmetic and split count: the outputs agree to the bit
        assert torch.equal(out, out_flat), (loop, (out - out_flat).abs().max().item())
        ref = RQ.decode_attention(cache_np, lay, loop, q.double().cpu().numpy(), kc.double().cpu().numpy(),
                                  vc.double().cpu().numpy(), ctx, rot, sc)
        e = close(out.double().cpu().numpy(), ref)
        worst = max(worst, e)
        assert e <= 1.0, (loop, e)
        if l == L - 1:
            B.rq_quantize_token_paged(cfg, pool, n_blocks, table, pending, grp, ctx_len, inp.rot, batch, 1)
    torch.cuda.synchronize()
    say(f"[paged] case={name} decode worst err/bound {worst:.3f}")

    # the drained token of every row sits in its slot ctx[b] of the gathered cache
    cache_np = gather(pool.cpu().numpy(), table_np, ocfg, bb)
    stats = new_stats()
    for b in range(batch):
        for h in range(hkv):
            block, sub = sub_cache(cache_np, ocfg, b, h)
            slay = RQ.Layout(sub)
            for k in range(wl.n_groups):
                for x in range(2):
                    enc = RQ.read_tokens(block, slay, 0, 0, x, k, ctx[b] + 1)
                    check_encoding(slice_enc(enc, slice(ctx[b], ctx[b] + 1)), kv[k, :, x, b, h, ctx[b]: ctx[b] + 1],
                                   rot[h, x], sub, stats)
    assert_stats(stats, wl.group)
