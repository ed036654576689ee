"""A decode step captured in a HIP graph (torch.cuda.CUDAGraph) replays to the same
outputs as eager launches: every replay, with eager work and synchronisations in
between, is compared with the eager result.  The library enqueues no allocation,
memset or synchronisation, so it can be captured."""
import pytest
import torch

from looped_transformer_decode_amd import synth

from _support import gpu_pack, say

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    from looped_transformer_decode_amd import binding as B
    wl = synth.WORKLOADS["ouro_b4_t8192"].with_(batch=2, ctx=700, n_kv_heads=4, n_q_heads=4)
    dev = torch.device("cuda:0")
    inp = synth.generate(wl, seed=21, device=dev)
    cfg = B.config_for(wl)
    T, L, d = wl.ctx, wl.loops_per_group, wl.head_dim
    cache = gpu_pack(B, cfg, inp.kv, inp.rot, T)
    ws = torch.zeros(B.rq_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    pending = torch.zeros(wl.batch, L, 2, wl.n_kv_heads, d, dtype=torch.bfloat16, device=dev)
    ctx_len = torch.tensor([T, 333], dtype=torch.int32, device=dev)
    outs = [torch.empty(wl.batch, wl.n_q_heads, d, device=dev) for _ in range(L)]
    q = [inp.q[l].contiguous() for l in range(L)]
    kc = [inp.kv[0, l, 0, :, :, T].contiguous() for l in range(L)]
    vc = [inp.kv[0, l, 1, :, :, T].contiguous() for l in range(L)]

    def step():
        for l in range(L):
            B.rq_decode_attention(cfg, cache, l, q[l], kc[l], vc[l], pending, ctx_len, T, inp.rot, 0.088, outs[l],
                                  ws, wl.batch, n_splits=3)
        B.rq_quantize_token(cfg, cache, pending, 0, ctx_len, inp.rot, wl.batch, 1)

    say("[graph] eager")
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    cache_want = cache.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        say(f"[graph] replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o, w)
        assert torch.equal(cache, cache_want)
        step()                                   # eager work between replays
        torch.cuda.synchronize()


def test_graph_replay_with_projection_matches_eager():
    """A decode step that starts every loop with rq_kv_project (current-token K/V into the
    decode inputs and the pending slot) replays from a graph to the eager result."""
    from looped_transformer_decode_amd import binding as B
    wl = synth.WORKLOADS["ouro_b4_t8192"].with_(batch=3, ctx=500, n_kv_heads=4, n_q_heads=4)
    dev = torch.device("cuda:0")
    inp = synth.generate(wl, seed=22, device=dev)
    pin = synth.projection_inputs(wl, seed=23, device=dev, hidden=512)
    cfg = B.config_for(wl)
    T, L, d = wl.ctx, wl.loops_per_group, wl.head_dim
    cache = gpu_pack(B, cfg, inp.kv, inp.rot, T)
    ws = torch.zeros(B.rq_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    pending = torch.zeros(wl.batch, L, 2, wl.n_kv_heads, d, dtype=torch.bfloat16, device=dev)
    ctx_len = torch.tensor([T, 17, 400], dtype=torch.int32, device=dev)
    outs = [torch.empty(wl.batch, wl.n_q_heads, d, device=dev) for _ in range(L)]
    q = [inp.q[l].contiguous() for l in range(L)]
    kc = torch.empty(wl.batch, wl.n_kv_heads, d, dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)

    def step():
        for l in range(L):
            B.rq_kv_project(cfg, pin.x[l], pin.w, l, kc, vc, pending, wl.batch)
            B.rq_decode_attention(cfg, cache, l, q[l], kc, vc, None, ctx_len, T, inp.rot, 0.088, outs[l], ws,
                                  wl.batch)
        B.rq_quantize_token(cfg, cache, pending, 0, ctx_len, inp.rot, wl.batch, 1)

    say("[graph+projection] eager")
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    cache_want = cache.clone()
    pend_want = pending.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        pending.zero_()
        say(f"[graph+projection] replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o, w)
        assert torch.equal(cache, cache_want)
        assert torch.equal(pending.view(torch.int16), pend_want.view(torch.int16))
        step()
        torch.cuda.synchronize()


def test_pack_beside_anchor_attention_matches_sequential():
    """With the projection in front of every loop, the pack of the finished token reads only the
    pending buffer, so it may run on a second stream beside the anchor loop's attention: that
    attention reads token slots below ctx_len, the pack writes slot ctx_len.  The overlapped step
    (fork/join in a HIP graph, replayed several times) gives the sequential step's outputs and
    cache bytes exactly, for shared anchors and for the grouped-query kernel."""
    from looped_transformer_decode_amd import binding as B
    dev = torch.device("cuda:0")
    for wl in (synth.WORKLOADS["ouro_b4_t8192"].with_(batch=3, ctx=333, n_kv_heads=4, n_q_heads=4),
               synth.WORKLOADS["huginn_gqa4_b8_t8192"].with_(batch=2, ctx=200, n_kv_heads=2, n_q_heads=8,
                                                            n_groups=2)):
        say(f"[pack beside anchor] {wl.name} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} groups={wl.n_groups}")
        inp = synth.generate(wl, seed=31, device=dev)
        pin = synth.projection_inputs(wl, seed=32, device=dev, hidden=256)
        cfg = B.config_for(wl)
        T, L, d = wl.ctx, wl.loops_per_group, wl.head_dim
        cache0 = gpu_pack(B, cfg, inp.kv, inp.rot, T)
        cache = cache0.clone()
        ws = torch.zeros(B.rq_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
        pending = torch.zeros(wl.batch, L, 2, wl.n_kv_heads, d, dtype=torch.bfloat16, device=dev)
        ctx_len = torch.tensor([T, 64, 129][:wl.batch], dtype=torch.int32, device=dev)
        outs = [torch.empty(wl.batch, wl.n_q_heads, d, device=dev) for _ in range(wl.n_loops)]
        q = [inp.q[l].contiguous() for l in range(wl.n_loops)]
        kc = torch.empty(wl.batch, wl.n_kv_heads, d, dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        side = torch.cuda.Stream()

        def step(overlap):
            main = torch.cuda.current_stream()
            for l in range(wl.n_loops):
                B.rq_kv_project(cfg, pin.x[l], pin.w, l, kc, vc, pending, wl.batch)
                anchor = l % L == L - 1
                if anchor and overlap:
                    fork = torch.cuda.Event()
                    fork.record(main)
                    side.wait_event(fork)
                    B.rq_quantize_token(cfg, cache, pending, l // L, ctx_len, inp.rot, wl.batch, 1, stream=side)
                B.rq_decode_attention(cfg, cache, l, q[l], kc, vc, None, ctx_len, T, inp.rot, 0.088, outs[l], ws,
                                      wl.batch)
                if anchor and overlap:
                    join = torch.cuda.Event()
                    join.record(side)
                    main.wait_event(join)
                elif anchor:
                    B.rq_quantize_token(cfg, cache, pending, l // L, ctx_len, inp.rot, wl.batch, 1)

        step(False)
        torch.cuda.synchronize()
        want = [o.clone() for o in outs]
        cache_want = cache.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(True)
        torch.cuda.synchronize()
        for rep in range(3):
            cache.copy_(cache0)
            for o in outs:
                o.fill_(float("nan"))
            torch.cuda.synchronize()
            say(f"[pack beside anchor] replay {rep}")
            g.replay()
            torch.cuda.synchronize()
            for o, w in zip(outs, want):
                assert torch.equal(o, w)
            assert torch.equal(cache, cache_want)
