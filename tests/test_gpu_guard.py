"""Guard bands around every device buffer the library writes or reads, at one full-size
workload (4 rows x 16 KV heads x 8192 context tokens, head_dim 128, INT4/INT2): each
buffer sits inside a larger allocation whose bytes before and after it hold a fixed
pattern, and after the bulk pack, decode attention at every loop (with the pending
write), the per-step pack, the paged pack and decode, the K/V projection, the decode
entry point without a workspace and the BF16 baseline (with its append) those bytes must
be unchanged: no kernel reads or writes past the buffers it is given."""
import pytest
import torch

from looped_transformer_decode_amd import synth

from _support import pending_strides, say

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes of pattern on each side (keeps the buffer 4096-byte aligned)
PATTERN = 0xA5


class Guarded:
    def __init__(self):
        self.bufs = []

    def new(self, shape, dtype, name, init=None):
        n = int(torch.Size(shape).numel()) * torch.empty(0, dtype=dtype).element_size()
        raw = torch.full((n + 2 * GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        view = raw[GUARD:GUARD + n].view(dtype).view(shape)
        if init is None:
            view.zero_()
        else:
            view.copy_(init)
        self.bufs.append((name, raw, n))
        return view

    def check(self, stage):
        torch.cuda.synchronize()
        for name, raw, n in self.bufs:
            for side, band in (("before", raw[:GUARD]), ("after", raw[GUARD + n:])):
                bad = int((band != PATTERN).sum())
                assert bad == 0, f"{stage}: {bad} guard bytes {side} {name} changed"
        say(f"[guard] {stage}: {len(self.bufs)} buffers intact")


def test_guard_bands_full_size():
    from looped_transformer_decode_amd import binding as B
    wl = synth.WORKLOADS["ouro_b4_t8192"]
    T, L, d, Bt, Hkv, Hq = wl.ctx, wl.loops_per_group, wl.head_dim, wl.batch, wl.n_kv_heads, wl.n_q_heads
    say("[guard] generating")
    inp = synth.generate(wl, seed=77, device="cuda")
    cfg = B.config_for(wl)
    g = Guarded()
    kv = g.new(inp.kv.shape, torch.bfloat16, "kv", inp.kv)
    rot = g.new(inp.rot.shape, torch.float32, "rot", inp.rot)
    cache = g.new((B.rq_cache_bytes(cfg),), torch.uint8, "cache")
    pos0 = g.new((Bt,), torch.int32, "pos0")
    say("[guard] bulk pack")
    B.rq_quantize_token(cfg, cache, kv[0], 0, pos0, rot, Bt, T, pending_strides=pending_strides(kv[0]))
    g.check("bulk pack")

    q = [g.new(inp.q[i].shape, inp.q.dtype, f"q{i}", inp.q[i]) for i in range(L)]
    kc = [g.new((Bt, Hkv, d), torch.bfloat16, f"k_cur{i}", inp.kv[0, i, 0, :, :, T]) for i in range(L)]
    vc = [g.new((Bt, Hkv, d), torch.bfloat16, f"v_cur{i}", inp.kv[0, i, 1, :, :, T]) for i in range(L)]
    ctx_len = g.new((Bt,), torch.int32, "ctx_len", torch.tensor([T, T - 1, 4097, 65], dtype=torch.int32))
    pending = g.new((Bt, L, 2, Hkv, d), torch.bfloat16, "pending")
    out = g.new((Bt, Hq, d), torch.float32, "out")
    ws = g.new((B.rq_workspace_bytes(cfg),), torch.uint8, "workspace")
    sc = synth.sm_scale(d)
    for loop in range(L):
        say(f"[guard] decode loop {loop}")
        B.rq_decode_attention(cfg, cache, loop, q[loop], kc[loop], vc[loop], pending, ctx_len, T, rot, sc, out, ws, Bt)
        g.check(f"decode loop {loop}")
    say("[guard] per-step pack")
    B.rq_quantize_token(cfg, cache, pending, 0, ctx_len, rot, Bt, 1)
    g.check("per-step pack")
    say("[guard] decode without a workspace")
    B.rq_decode_attention_noalloc(cfg, cache, 1, q[1], kc[1], vc[1], pending, ctx_len, T, rot, sc, out, Bt)
    g.check("decode without a workspace")

    # paged: every tile of every row in its own block, in reverse order
    n_tiles = (cfg.max_ctx + 63) // 64
    n_blocks = Bt * n_tiles
    table = g.new((Bt, n_tiles), torch.int32, "block table",
                  torch.arange(n_blocks - 1, -1, -1, dtype=torch.int32).view(Bt, n_tiles))
    pool = g.new((n_blocks * B.rq_paged_block_bytes(cfg),), torch.uint8, "pool")
    say("[guard] paged pack")
    B.rq_quantize_token_paged(cfg, pool, n_blocks, table, kv[0], 0, pos0, rot, Bt, T,
                              pending_strides=pending_strides(kv[0]))
    g.check("paged pack")
    for loop in (0, L - 1):
        say(f"[guard] paged decode loop {loop}")
        B.rq_decode_attention_paged(cfg, pool, n_blocks, table, loop, q[loop], kc[loop], vc[loop], pending, ctx_len,
                                    T, rot, sc, out, ws, Bt)
        g.check(f"paged decode loop {loop}")

    say("[guard] K/V projection")
    pin_ = synth.projection_inputs(wl, seed=78, device="cuda")
    x = g.new(pin_.x[0].shape, torch.bfloat16, "hidden", pin_.x[0])
    w = g.new(pin_.w.shape, torch.bfloat16, "weights", pin_.w)
    pk = g.new((Bt, Hkv, d), torch.bfloat16, "proj k")
    pv = g.new((Bt, Hkv, d), torch.bfloat16, "proj v")
    B.rq_kv_project(cfg, x, w, 2, pk, pv, pending, Bt)
    g.check("K/V projection")

    say("[guard] BF16 baseline with append")
    bcfg = B.bf16_config_for(wl)
    K = g.new((Bt, Hkv, T + 1, d), torch.bfloat16, "bf16 K", inp.kv[0, 0, 0])
    V = g.new((Bt, Hkv, T + 1, d), torch.bfloat16, "bf16 V", inp.kv[0, 0, 1])
    bws = g.new((B.rq_bf16_workspace_bytes(bcfg),), torch.uint8, "bf16 workspace")
    B.rq_bf16_decode_attention(bcfg, K, V, q[0], kc[0], vc[0], True, ctx_len, T, sc, out, bws, Bt)
    g.check("BF16 decode with append")
    assert bool(torch.isfinite(out).all())
