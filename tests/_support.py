"""Helpers for the GPU parity tests: run the HIP path through the C ABI and compare it
with the float64 oracle under the parity rules.

Parity rules (written here, checked by the tests):
* anchor codes and FP8 metadata: bit-exact;
* c: within 1 BF16 ulp of the oracle's c computed from the GPU's own reference vector;
* residual codes and metadata are checked conditionally on the GPU's upstream choices
  (its c and, for the chained layout, its rebuilt neighbour): a metadata mismatch is
  allowed only where the oracle's group minimum (offset) or (max - z)/n (scale) lies
  within 1e-6 relative of an E4M3 grid point, and a code mismatch only where
  (x - z)/s lies within 1e-6 * max(1, |t|) of a rounding tie; such near-ties are counted
  and must stay below 1e-5 of all codes;
* attention outputs: max|o_gpu - o_oracle| <= 1e-3 * max|o_oracle| + 1e-5 per output tensor.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from looped_transformer_decode_amd import synth
from oracle import formats as F
from oracle import residualquant as RQ

ATOL_REL, ATOL_ABS = 1e-3, 1e-5
NEAR = 1e-6


#: (case, worst err/bound) of every parity check, printed at the end of the run
MARGINS = []


def record_margin(tag: str, worst: float) -> None:
    MARGINS.append((tag, float(worst)))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_cfg(wl, chained=None, max_batch=None, max_ctx=None, n_kv_heads=None, n_q_heads=None):
    return RQ.Config(wl.head_dim, wl.group, wl.anchor_bits, wl.resid_bits, wl.loops_per_group,
                     wl.n_groups, bool(wl.chained if chained is None else chained),
                     n_kv_heads or wl.n_kv_heads, n_q_heads or wl.n_q_heads,
                     max_batch or wl.batch, max_ctx or wl.ctx + 1, wl.scale_rule, tuple(wl.resid_bits_loop))


def pending_strides(kv: torch.Tensor):
    """Strides (token, batch, loop, K|V, head) of one group slice kv[grp], shaped
    [L][2][B][Hkv][T+1][d], of the generator's K/V tensor."""
    assert kv.dim() == 6
    st = kv.stride()
    return (st[4], st[2], st[0], st[1], st[3])


def gpu_pack(B, cfg, kv: torch.Tensor, rot: torch.Tensor, n_tokens: int, cache=None, pos0=0):
    """Quantize tokens [0, n_tokens) of every anchor group on the GPU; returns the cache."""
    if cache is None:
        cache = torch.zeros(B.rq_cache_bytes(cfg), dtype=torch.uint8, device=kv.device)
    batch = kv.shape[3]
    pos = torch.full((batch,), pos0, dtype=torch.int32, device=kv.device)
    for grp in range(kv.shape[0]):
        B.rq_quantize_token(cfg, cache, kv[grp], grp, pos, rot, batch, n_tokens,
                            pending_strides=pending_strides(kv[grp]))
    return cache


def sub_cache(cache_np: np.ndarray, cfg: RQ.Config, b: int, h: int):
    """Bytes of one (batch row, KV head) as a cache of a 1-row, 1-head configuration."""
    lay = RQ.Layout(cfg)
    start = (b * cfg.n_kv_heads + h) * 2 * lay.block_bytes
    sub = RQ.Config(cfg.head_dim, cfg.group, cfg.anchor_bits, cfg.resid_bits, cfg.loops_per_group,
                    cfg.n_groups, cfg.chained, 1, cfg.n_q_heads // cfg.n_kv_heads, 1, cfg.max_ctx, cfg.scale_rule,
                    cfg.resid_bits_loop)
    return np.ascontiguousarray(cache_np[start: start + 2 * lay.block_bytes]), sub


def device_block(cache: torch.Tensor, cfg: RQ.Config, b: int, h: int) -> np.ndarray:
    lay = RQ.Layout(cfg)
    start = (b * cfg.n_kv_heads + h) * 2 * lay.block_bytes
    return cache[start: start + 2 * lay.block_bytes].cpu().numpy()


def _ulp_bf16(v):
    v = np.abs(v)
    e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    return np.where(v > 0, 2.0 ** (np.maximum(e, -126) - 7), 2.0 ** -133)


def _near_grid(v):
    g = F.E4M3_GRID
    idx = np.clip(np.searchsorted(g, v), 1, g.size - 1)
    d = np.minimum(np.abs(v - g[idx - 1]), np.abs(g[idx] - v))
    return d <= NEAR * np.maximum(np.abs(v), 2.0 ** -9)


def slice_enc(enc: RQ.Encoded, idx) -> RQ.Encoded:
    return RQ.Encoded(tuple(a[idx] for a in enc.anchor), [tuple(a[idx] for a in r) for r in enc.resid])


def check_encoding(enc: RQ.Encoded, xs: np.ndarray, R: np.ndarray, sub: RQ.Config, stats: dict):
    """Check the GPU's encoding `enc` (tokens on the leading axis) of inputs xs
    (L, n, d) float64 for one (row, KV head, K|V, anchor group); R = (d, d) float64."""
    L, g = sub.loops_per_group, sub.group
    qa, za, sa = RQ.quantize(xs[L - 1], sub.anchor_bits, g)
    ga, gz, gs = enc.anchor
    assert np.array_equal(ga, qa), "anchor codes differ"
    assert np.array_equal(gz, za) and np.array_equal(gs, sa), "anchor metadata differs"
    stats["codes"] += qa.size
    a_hat = RQ.dequantize(qa, za, sa, g)
    for l in range(L - 2, -1, -1):
        ref = RQ.reconstruct(enc, l + 1, R, sub) if sub.chained else a_hat
        c_exp, _ = RQ.coefficient(xs[l], ref, sub)
        qg, zg, sg, cg = enc.resid[l]
        dc = np.abs(cg - c_exp)
        assert np.all(dc <= _ulp_bf16(c_exp)), f"c off by more than 1 ulp: {dc.max()}"
        stats["c_diff"] += int(np.count_nonzero(dc))
        stats["c_total"] += cg.size
        y = xs[l] - cg[:, None] * ref
        r = y @ R.T
        qe, ze, se = RQ.quantize(r, sub.rbits(l), g)
        rg = r.reshape(r.shape[0], -1, g)
        bad_meta = (ze != zg) | (se != sg)
        if np.any(bad_meta):
            lo = rg.min(-1)
            n = 2 ** sub.rbits(l) - 1
            need = (rg.max(-1) - ze) / n
            ok = _near_grid(lo) | _near_grid(need)
            assert np.all(ok[bad_meta]), "residual metadata differs away from a grid point"
            stats["near_meta"] += int(np.count_nonzero(bad_meta))
        # codes, judged with the metadata the GPU stored
        t = (rg - zg[..., None]) / sg[..., None]
        q_with_gpu_meta = np.clip(np.rint(t), 0, 2 ** sub.rbits(l) - 1).reshape(qg.shape)
        bad = q_with_gpu_meta != qg
        if np.any(bad):
            tt = t.reshape(qg.shape)[bad]
            dist = np.abs(tt - (np.floor(tt) + 0.5))
            assert np.all(dist <= NEAR * np.maximum(1.0, np.abs(tt))), "residual code differs away from a tie"
            stats["near_ties"] += int(np.count_nonzero(bad))
        stats["codes"] += qg.size


def check_pack_block(gpu_block: np.ndarray, sub: RQ.Config, xs_groups, rot2, n_tokens: int, stats: dict):
    """Check tokens [0, n_tokens) of one (row, KV head) block.  xs_groups[k][x] =
    (L, n_tokens, d) float64 inputs of anchor group k, K|V x; rot2 = (2, d, d) float64."""
    lay = RQ.Layout(sub)
    for k in range(sub.n_groups):
        for x in range(2):
            enc = RQ.read_tokens(gpu_block, lay, 0, 0, x, k, n_tokens)
            check_encoding(enc, xs_groups[k][x], rot2[x], sub, stats)


def new_stats():
    return dict(codes=0, near_ties=0, near_meta=0, c_diff=0, c_total=0)


def assert_stats(stats, group: int = 32):
    """Near-ties, plus every code of a group whose metadata the GPU took differently next to
    a grid point, must stay below 1e-5 of all codes."""
    charged = stats["near_ties"] + stats["near_meta"] * group
    assert charged <= 1e-5 * max(stats["codes"], 1), stats


def close(o_gpu: np.ndarray, o_ref: np.ndarray) -> float:
    """Return max|diff| / bound; <= 1 passes."""
    bound = ATOL_REL * np.abs(o_ref).max() + ATOL_ABS
    return float(np.abs(o_gpu - o_ref).max() / bound)


def setup_case(B, wl, chained, batch, ctx, hkv=None, hq=None, seed=1234):
    """Workload of a small parity case: batch rows with context lengths ctx (the largest is
    the packed context T), seeded inputs on the GPU, the library and oracle configurations."""
    T = max(ctx)
    wl = wl.with_(batch=batch, ctx=T, chained=chained,
                  n_kv_heads=hkv or wl.n_kv_heads, n_q_heads=hq or wl.n_q_heads)
    inp = synth.generate(wl, seed=seed, device="cuda")
    return wl, inp, B.config_for(wl), oracle_cfg(wl), ctx, T


def run_pack_parity(B, name, wl, inp, cfg, ocfg, T):
    """Pack the whole context of every group on the GPU and check every stored code,
    FP8 offset/scale and c against the oracle's rules."""
    say(f"[pack] case={name} T={T} batch={wl.batch}")
    cache = gpu_pack(B, cfg, inp.kv, inp.rot, T)
    torch.cuda.synchronize()
    kv = inp.kv.double().cpu().numpy()
    rot = inp.rot.double().cpu().numpy()
    stats = new_stats()
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            block = device_block(cache, ocfg, b, h)
            _, sub = sub_cache(np.zeros(0, np.uint8), ocfg, 0, 0)
            xs = [[kv[k, :, x, b, h, :T] for x in range(2)] for k in range(wl.n_groups)]
            check_pack_block(block, sub, xs, rot[h], T, stats)
    say(f"[pack] case={name} stats={stats}")
    assert_stats(stats, wl.group)


def run_decode_step_parity(B, name, wl, inp, cfg, ocfg, ctx, T, loops=None):
    """One decode step through every loop (or the listed ones, then only the drains of
    groups whose loops all ran): attention at each loop with the current token written to
    the pending buffer, compared with the oracle on the GPU's bytes and on the oracle's own
    pack, at several split counts; after a group's last loop, the finished token packed from
    that buffer and checked."""
    say(f"[decode] case={name} T={T} ctx={ctx}")
    dev = inp.kv.device
    L, d, Hq, Hkv = wl.loops_per_group, wl.head_dim, wl.n_q_heads, wl.n_kv_heads
    cache = gpu_pack(B, cfg, inp.kv, inp.rot, T)
    ctx_len = torch.tensor(ctx, dtype=torch.int32, device=dev)
    ws = torch.zeros(B.rq_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    pending = torch.zeros(wl.batch, L, 2, Hkv, d, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    cache_np = cache.cpu().numpy()
    kv = inp.kv.double().cpu().numpy()
    rot = inp.rot.double().cpu().numpy()
    own = RQ.pack_context(kv, rot, ocfg, T)
    lay = RQ.Layout(ocfg)
    sc = synth.sm_scale(d)
    n_tiles = -(-T // 64)
    run = list(range(wl.n_loops)) if loops is None else list(loops)
    worst = 0.0
    for loop in run:
        grp, l = divmod(loop, L)
        k_cur = inp.kv[grp, l, 0, :, :, T].contiguous()
        v_cur = inp.kv[grp, l, 1, :, :, T].contiguous()
        q = inp.q[loop].contiguous()
        ref_gpu = RQ.decode_attention(cache_np, lay, loop, q.double().cpu().numpy(), kv[grp, l, 0, :, :, T],
                                      kv[grp, l, 1, :, :, T], ctx, rot, sc)
        ref_own = RQ.decode_attention(own, lay, loop, q.double().cpu().numpy(), kv[grp, l, 0, :, :, T],
                                      kv[grp, l, 1, :, :, T], ctx, rot, sc)
        for ns in sorted({0, 1, min(3, n_tiles), n_tiles}):
            out = torch.full((wl.batch, Hq, d), float("nan"), dtype=torch.float32, device=dev)
            say(f"[decode] case={name} loop={loop} n_splits={ns}")
            B.rq_decode_attention(cfg, cache, loop, q, k_cur, v_cur, pending, ctx_len, T, inp.rot, sc, out,
                                  ws, wl.batch, n_splits=ns)
            torch.cuda.synchronize()
            o = out.double().cpu().numpy()
            assert np.all(np.isfinite(o))
            e1, e2 = close(o, ref_gpu), close(o, ref_own)
            worst = max(worst, e1, e2)
            say(f"    err/bound vs oracle(gpu cache)={e1:.3f} vs oracle(own cache)={e2:.3f}")
            assert e1 <= 1.0 and e2 <= 1.0
        if l == L - 1 and all(grp * L + m in run for m in range(L)):
            # pending now holds the current token of every loop of this group
            want = inp.kv[grp, :, :, :, :, T].permute(2, 0, 1, 3, 4)
            assert torch.equal(pending, want)
            say(f"[decode] case={name} pack finished token of group {grp}")
            B.rq_quantize_token(cfg, cache, pending, grp, ctx_len, inp.rot, wl.batch, 1)
            torch.cuda.synchronize()
            cache_np = cache.cpu().numpy()
            stats = new_stats()
            for b in range(wl.batch):
                for h in range(Hkv):
                    block, sub = sub_cache(cache_np, ocfg, b, h)
                    for x in range(2):
                        enc = RQ.read_tokens(block, RQ.Layout(sub), 0, 0, x, grp, ctx[b] + 1)
                        check_encoding(slice_enc(enc, slice(ctx[b], ctx[b] + 1)),
                                       kv[grp, :, x, b, h, T:T + 1], rot[h, x], sub, stats)
            assert_stats(stats, wl.group)
    record_margin(f"decode step {name}", worst)
