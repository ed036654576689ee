"""Benchmark of the ResidualQuant decode hot path on one MI355X.

One step = one layer's decode step of one token through every loop of the workload:
for each loop, fused RQ decode attention (which also writes the current token into the
BF16 pending buffer); after each anchor loop, rq_quantize_token packs the finished token
of that anchor group.  Inputs (packed context, queries, current-token K/V) are resident
in HBM before the timed region.  The BF16 decode kernel is timed on the same K/V.

To measure HBM rather than the 256 MB Infinity Cache, every loop-step reads its own
replica of the packed cache (replicas rotate; the same replica comes back only after
more than 256 MB of other reads), which is what a multi-layer model sees between two
loops of one layer.  Warm (single replica) figures are reported separately.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "ouro_b16_t8192"
CSRC = os.path.join(ROOT, "looped_transformer_decode_amd", "csrc")
# sources of the decode kernels (split-K with the merge in the last workgroup): the one-query
# kernel, and the grouped-query kernel that serves the query heads of a KV head together
DECODE_SOURCES = ("rq_api.hip", "rq_decode.hip", "rq_args.hpp", "rq_common.hpp",
                  "rq_splitk.hpp", "rq_stage.hpp")
GQA_SOURCES = ("rq_api.hip", "rq_decode_gqa.hip", "rq_args.hpp", "rq_common.hpp",
               "rq_merge_group.hpp", "rq_splitk.hpp", "rq_stage.hpp")
PROFILES = os.path.join(ROOT, "profiles")


def traffic_profile(workload: str) -> str:
    return os.path.join(PROFILES, f"rq_decode_residual_{workload}_hbm_traffic.txt")


def grouped_kernel(wl) -> bool:
    """Whether the library runs this workload's residual loop-steps on the grouped-query kernel:
    head_dim 128, g = 32, INT4 anchor, 2-bit residual planes read one at a time (not chained),
    2 or 4 query heads per KV head (the routing rule of rq_decode_attention)."""
    gq = wl.n_q_heads // wl.n_kv_heads
    return (wl.head_dim == 128 and wl.group == 32 and wl.anchor_bits == 4 and not wl.chained
            and all(b == 2 for b in (wl.resid_bits_loop or (wl.resid_bits,))) and gq in (2, 4))


def decode_source_digest(wl=None) -> str:
    """Digest of the sources of the kernel that runs the workload's residual loop-steps."""
    h = hashlib.sha256()
    for name in (GQA_SOURCES if wl is not None and grouped_kernel(wl) else DECODE_SOURCES):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per residual loop-step from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None when it was taken on other kernel sources or another workload."""
    try:
        with open(traffic_profile(workload)) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    from looped_transformer_decode_amd import synth
    wl = synth.WORKLOADS.get(workload)
    if wl is None or kv.get("source_digest") != decode_source_digest(wl) or kv.get("workload") != workload:
        return None
    return int(float(kv["traffic_bytes_per_loop_step"]))


def algorithmic_bytes(wl, loop_local: int, chained: bool) -> int:
    """Compressed bytes one loop-step must read: codes + FP8 metadata + BF16 c of every
    plane the loop needs, for K and V, for all context tokens of all (row, KV head)."""
    d, g = wl.head_dim, wl.group
    A = d * wl.anchor_bits // 8 + 2 * d // g
    L = wl.loops_per_group
    widths = wl.resid_bits_loop or (wl.resid_bits,) * (L - 1)
    planes = [] if loop_local == L - 1 else (list(range(loop_local, L - 1)) if chained else [loop_local])
    R = sum(d * widths[l] // 8 + 2 * d // g + 2 for l in planes)
    return 2 * (A + R) * wl.batch * wl.ctx * wl.n_kv_heads


def bf16_bytes(wl) -> int:
    return 2 * 2 * wl.head_dim * wl.batch * wl.ctx * wl.n_kv_heads


def bulk_in_bytes(wl) -> int:
    """BF16 K/V of every loop of every anchor group, read once by the bulk context pack."""
    return wl.batch * wl.ctx * wl.n_loops * 2 * wl.n_kv_heads * wl.head_dim * 2


def rotation_fma(wl) -> int:
    """Float64 FMAs of the d x d products in a bulk pack of the whole context: R y of every
    residual vector, and in the chained layout also the rebuilt reference c ref + R^T r_hat
    of every residual loop but the group's first (the last loop stored needs no successor)."""
    n_prod = wl.n_groups * (wl.loops_per_group - 1)
    if wl.chained:
        n_prod += wl.n_groups * (wl.loops_per_group - 2)
    return wl.batch * wl.ctx * wl.n_kv_heads * 2 * n_prod * wl.head_dim * wl.head_dim


def _oracle_worker(args):
    """One worker of the CPU baseline: the float64 oracle's residual loop-step of decode
    attention for one (row, KV head) at the full context, repeated until the deadline."""
    wl, seed, deadline = args
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from looped_transformer_decode_amd import synth
    from oracle import residualquant as RQ

    torch.set_num_threads(1)
    with threadpool_limits(limits=1):
        T = wl.ctx
        small = wl.with_(batch=1, n_kv_heads=1, n_q_heads=wl.n_q_heads // wl.n_kv_heads)
        inp = synth.generate(small, seed=seed, device="cpu")
        cfg = RQ.Config(small.head_dim, small.group, small.anchor_bits, small.resid_bits, small.loops_per_group,
                        small.n_groups, small.chained, 1, small.n_q_heads, 1, T + 1, small.scale_rule,
                        tuple(small.resid_bits_loop))
        kv = inp.kv.double().numpy()
        rot = inp.rot.double().numpy()
        tp = time.perf_counter()
        cache = RQ.pack_context(kv, rot, cfg, T)
        pack_s = time.perf_counter() - tp
        lay = RQ.Layout(cfg)
        q = inp.q.double().numpy()
        sc = synth.sm_scale(small.head_dim)
        reps = 0
        t0 = time.perf_counter()
        while True:
            RQ.decode_attention(cache, lay, 0, q[0], kv[0, 0, 0, :, :, T], kv[0, 0, 1, :, :, T], [T], rot, sc)
            reps += 1
            if time.time() >= deadline:
                break
        return reps, time.perf_counter() - t0, pack_s


def cpu_baseline(wl, budget_s: float = 15.0, workers: int = 0):
    """Time the float64 oracle (as it is) on a bounded sample of the same workload: one
    (row, KV head) per worker process, each running the residual loop-step of decode
    attention at the full context until a common deadline.  All workers run at once, one
    BLAS thread each, so the figure is the host's whole-socket oracle rate on this sample."""
    import multiprocessing as mp

    n = workers or min(16, os.cpu_count() or 1)
    pairs = n
    deadline = time.time() + budget_s
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(n) as pool:
        res = pool.map(_oracle_worker, [(wl, 1000 + i, deadline) for i in range(pairs)])
    wall = time.perf_counter() - t0
    reps = sum(r[0] for r in res)
    per_head_bytes = algorithmic_bytes(wl.with_(batch=1, n_kv_heads=1), 0, wl.chained)
    decode_s = max(r[1] for r in res)
    pack_s = sum(r[2] for r in res) / len(res)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": round(per_head_bytes * reps / decode_s / 1e9, 4),
        "unit": "GB/s",
        "cores": n,
        "host_cpus": os.cpu_count(),
        "cpu_model": model,
        "kind": "oracle",
        "sample": f"{reps} residual loop-steps of float64 oracle decode attention, one (row, KV head) at "
                  f"{wl.ctx} context tokens per worker process, {n} processes at once with one BLAS thread "
                  f"each, {decode_s:.1f} s ({wall:.1f} s with input generation and the pack)",
        "kv_tokens_per_s": round(wl.ctx * reps / decode_s, 1),
        "pack": {"token_heads_per_s": round(n * wl.ctx / pack_s, 1),
                 "sample": f"float64 oracle pack of {wl.ctx} tokens of one (row, KV head), K and V, all "
                           f"{wl.n_loops} loops, in each of the {n} processes ({pack_s:.1f} s each)"},
    }



def w4a4_bytes(wl, residual: bool) -> int:
    """Algorithmic bytes of one loop-step of the W4A4 layer: the packed weights, the BF16
    activations, the 4-bit activation rows written (and the anchor rows read at a residual
    loop), the float32 output and the anchor product (written at the anchor loop, read at
    the others)."""
    K, N, M = wl.in_features, wl.out_features, wl.tokens
    rows = M * (K // 2 + K // 16)
    weights = N * K // 2 + N * (K // 32) * 2
    return weights + M * K * 2 + rows * (2 if residual else 1) + 2 * M * N * 4


def measure_w4a4(B, dev, sink, eager: bool = False, name: str = "ouro_up_b16") -> dict:
    """The W4A4 layer with cross-loop residual activations at one MLP up projection
    (ouro_up_b16: K 2048 -> N 8192 for a decode batch of 16; huginn_up_b8: K 4096 -> N 16384
    for a batch of 8): anchor and residual loop-steps replayed from HIP graphs over cold
    weight copies (beyond the 256 MB Infinity Cache), next to a plain load loop over the
    same weight bytes and a BF16 linear layer of the same shape (hipBLASLt through torch)
    over cold BF16 weight copies."""
    import torch
    from looped_transformer_decode_amd import synth
    wl = synth.W4A4_WORKLOADS[name]
    K, N, M, L = wl.in_features, wl.out_features, wl.tokens, wl.loops
    inp = synth.w4a4_inputs(wl, device=dev)
    cfg = B.w4a4_config(K, N, M)
    wb = B.rq_w4_weight_bytes(cfg)
    wq = torch.empty(wb, dtype=torch.uint8, device=dev)
    wrq = torch.empty_like(wq)
    B.rq_w4_quantize_weights(cfg, inp.w, None, wq)
    B.rq_w4_quantize_weights(cfg, inp.w, inp.rot, wrq)
    n_rep = max(2, math.ceil(600e6 / (2 * wb)))
    reps_a = [wq.clone() for _ in range(n_rep)]
    reps_r = [wrq.clone() for _ in range(n_rep)]
    anchor = torch.zeros(B.rq_w4a4_act_bytes(cfg), dtype=torch.uint8, device=dev)
    act = torch.zeros_like(anchor)
    ws = torch.zeros(B.rq_w4a4_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    y0 = torch.zeros(M, N, device=dev)
    y = torch.zeros(M, N, device=dev)
    xs = [inp.x[l].contiguous() for l in range(L)]
    B.rq_w4a4_linear(cfg, wq, xs[0], 0, anchor, None, None, None, y0, y0, M, ws)
    if eager:
        # plain launches (for counter runs, which attribute per dispatch): a group of loops per replica
        for i in range(n_rep):
            B.rq_w4a4_linear(cfg, reps_a[i], xs[0], 0, anchor, None, None, None, y0, y0, M, ws)
            for l in range(1, L):
                B.rq_w4a4_linear(cfg, reps_r[i], xs[l], l, anchor, act, inp.rot, None, y0, y, M, ws)
        torch.cuda.synchronize()
        return {"workload": wl.name, "launch": "eager", "weight_replicas": n_rep}

    def graph_ms(call, reps):
        for i in range(2):
            call(i)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                call(i + 2)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    reps = 3 * n_rep
    ms_anchor = graph_ms(lambda i: B.rq_w4a4_linear(cfg, reps_a[i % n_rep], xs[0], 0, anchor, None, None, None,
                                                    y0, y, M, ws), reps)
    ms_resid = graph_ms(lambda i: B.rq_w4a4_linear(cfg, reps_r[i % n_rep], xs[1 + i % (L - 1)], 1 + i % (L - 1),
                                                   anchor, act, inp.rot, None, y0, y, M, ws), reps)
    ms_stream = graph_ms(lambda i: B.rq_stream_read(reps_a[i % n_rep], wb, sink), reps)
    del reps_a, reps_r
    w16 = inp.w.contiguous()
    n16 = max(2, math.ceil(600e6 / w16.numel() / 2))
    reps16 = [w16.clone() for _ in range(n16)]
    out16 = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    ms_bf16 = graph_ms(lambda i: torch.matmul(xs[0], reps16[i % n16].t(), out=out16), 3 * n16)
    del reps16
    ba, br = w4a4_bytes(wl, False), w4a4_bytes(wl, True)
    group_ms = ms_anchor + (L - 1) * ms_resid
    return {"workload": wl.name, "in_features": K, "out_features": N, "tokens": M, "loops": L,
            "weight_bytes": wb, "weight_replicas": n_rep,
            "anchor_loop": {"bytes": ba, "ms": round(ms_anchor, 5), "gbps": round(ba / (ms_anchor * 1e-3) / 1e9, 1),
                            "frac_of_hbm_peak": round(ba / (ms_anchor * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
            "residual_loop": {"bytes": br, "ms": round(ms_resid, 5), "gbps": round(br / (ms_resid * 1e-3) / 1e9, 1),
                              "frac_of_hbm_peak": round(br / (ms_resid * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
            "group_of_loops_ms": round(group_ms, 5),
            "stream_read_same_weight_bytes_ms": round(ms_stream, 5),
            "bf16_linear_ms": round(ms_bf16, 5),
            "speedup_vs_bf16_linear": round(ms_bf16 * L / group_ms, 3),
            "timing": "HIP graph replay of back-to-back calls over cold weight copies, one event pair; "
                      "each call = activation quantizer + GEMM kernels"}

def measure_loop_steps(B, dev, name: str, splits: int = 0) -> dict:
    """Residual and anchor loop-steps of a second workload (the batch-4 case beside the batch-16
    default), each launched back to back over cold cache replicas with one event pair per
    repeat, and the BF16 kernel's loop-step on the same K/V."""
    import torch
    from looped_transformer_decode_amd import synth
    wl = synth.WORKLOADS[name]
    L, d, T, Bt = wl.loops_per_group, wl.head_dim, wl.ctx, wl.batch
    inp = synth.generate(wl, seed=20261202, device=dev)
    cfg = B.config_for(wl)
    cache_bytes = B.rq_cache_bytes(cfg)
    cache = torch.zeros(cache_bytes, dtype=torch.uint8, device=dev)
    pos0 = torch.zeros(Bt, dtype=torch.int32, device=dev)
    for grp in range(wl.n_groups):
        st = inp.kv[grp].stride()
        B.rq_quantize_token(cfg, cache, inp.kv[grp], grp, pos0, inp.rot, Bt, T,
                            pending_strides=(st[4], st[2], st[0], st[1], st[3]))
    n_rep = max(2, min(16, math.ceil(1.6e9 / cache_bytes)))
    caches = [cache] + [cache.clone() for _ in range(n_rep - 1)]
    q = [inp.q[i].contiguous() for i in range(L)]
    k_cur = [inp.kv[0, i, 0, :, :, T].contiguous() for i in range(L)]
    v_cur = [inp.kv[0, i, 1, :, :, T].contiguous() for i in range(L)]
    ctx_len = torch.full((Bt,), T, dtype=torch.int32, device=dev)
    ws = torch.zeros(B.rq_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    out = torch.empty(Bt, wl.n_q_heads, d, dtype=torch.float32, device=dev)
    sc = synth.sm_scale(d)
    stream = torch.cuda.current_stream()

    def back_to_back(loops, calls):
        reps = []
        for r in range(4):                        # the first repeat warms up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(calls):
                loop = loops[i % len(loops)]
                B.rq_decode_attention(cfg, caches[i % n_rep], loop, q[loop], k_cur[loop], v_cur[loop], None, ctx_len,
                                      T, inp.rot, sc, out, ws, Bt, n_splits=splits, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1) / calls)
        return sum(reps[1:]) / 3

    res_ms = back_to_back(list(range(L - 1)), 6 * n_rep)
    anc_ms = back_to_back([L - 1], 2 * n_rep)
    res_bytes = algorithmic_bytes(wl, 0, False)
    anc_bytes = algorithmic_bytes(wl, L - 1, False)
    bcfg = B.bf16_config_for(wl)
    bws = torch.zeros(B.rq_bf16_workspace_bytes(bcfg), dtype=torch.uint8, device=dev)
    Ks = [inp.kv[0, l, 0] for l in range(L)]
    Vs = [inp.kv[0, l, 1] for l in range(L)]
    bre = []
    for r in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(2 * L):
            l = i % L
            B.rq_bf16_decode_attention(bcfg, Ks[l], Vs[l], q[l], k_cur[l], v_cur[l], False, ctx_len, T, sc, out, bws,
                                       Bt, n_splits=splits, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        bre.append(e0.elapsed_time(e1) / (2 * L))
    bf16_ms = sum(bre[1:]) / 3
    return {"workload": name, "batch": Bt, "ctx": T, "cache_replicas": n_rep,
            "residual_loop_step": {"bytes": res_bytes, "ms": round(res_ms, 4),
                                   "gbps": round(res_bytes / (res_ms * 1e-3) / 1e9, 1),
                                   "frac_of_hbm_peak": round(res_bytes / (res_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
            "anchor_loop_step": {"bytes": anc_bytes, "ms": round(anc_ms, 4),
                                 "gbps": round(anc_bytes / (anc_ms * 1e-3) / 1e9, 1),
                                 "frac_of_hbm_peak": round(anc_bytes / (anc_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
            "bf16": {"bytes": bf16_bytes(wl), "ms_per_loop_step": round(bf16_ms, 4),
                     "gbps": round(bf16_bytes(wl) / (bf16_ms * 1e-3) / 1e9, 1),
                     "speedup_rq_residual_vs_bf16": round(bf16_ms / res_ms, 3)},
            "timing": "HIP events around back-to-back loop-steps over cold cache replicas (mean of 3 repeats "
                      "after one warm-up repeat); BF16 loop-steps back to back on the same K/V"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--chained", action="store_true")
    ap.add_argument("--resid-bits", type=int, default=0, help="4: uniform INT4 (with 4-bit anchors)")
    ap.add_argument("--loops-per-group", type=int, default=0, help="loop group length (8 or 16: the larger groups)")
    ap.add_argument("--scale-rule", type=int, default=0, help="1: norm-ratio coefficient")
    ap.add_argument("--resid-widths", default="", help="residual width per loop of a group, e.g. 4,2,2 "
                    "(more bits far from the anchor)")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-w4a4", action="store_true", help="skip the W4A4 layer measurement")
    ap.add_argument("--no-batch4", action="store_true",
                    help="skip the batch-4 loop-steps measured beside the default batch-16 workload")
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="time the CPU oracle on the workload and print its JSON (no GPU use)")
    ap.add_argument("--replicas", type=int, default=0)
    ap.add_argument("--eager-only", action="store_true",
                    help="time whole steps from eager launches instead of HIP graph replay "
                         "(for profilers that cannot follow graph launches)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode hot path has no cross-GPU step here "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    from looped_transformer_decode_amd import synth

    wl = synth.WORKLOADS[args.workload]
    if args.chained:
        wl = wl.with_(chained=True)
    if args.resid_bits:
        wl = wl.with_(resid_bits=args.resid_bits)
    if args.loops_per_group:
        wl = wl.with_(loops_per_group=args.loops_per_group, loop_scale="uniform(0.8,1.0)",
                      n_groups=max(1, wl.n_loops // args.loops_per_group))
    if args.scale_rule:
        wl = wl.with_(scale_rule=args.scale_rule)
    widths = tuple(int(v) for v in args.resid_widths.split(",")) if args.resid_widths else ()
    if widths:
        wl = wl.with_(resid_bits_loop=widths)
    variant = "".join(t for t, on in (("+int4", args.resid_bits == 4), (f"+L{args.loops_per_group}", args.loops_per_group),
                                      ("+norm_ratio", args.scale_rule == 1),
                                      ("+widths" + "".join(map(str, widths)), bool(widths))) if on)
    if variant:
        wl = wl.with_(name=wl.name + variant)
    if args.cpu_baseline_only:
        print(json.dumps(cpu_baseline(wl)))
        return
    cpu_base = None
    if not args.no_cpu_baseline:
        # The oracle runs in a child process started before this one touches the GPU; its
        # worker processes never use the GPU.
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        child = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-only"] +
                               [a for a in sys.argv[1:] if a != "--cpu-baseline-only"],
                               stdout=subprocess.PIPE, text=True, timeout=300)
        if child.returncode != 0:
            print("[bench] CPU baseline failed", file=sys.stderr)
            sys.exit(child.returncode or 1)
        cpu_base = json.loads(child.stdout.strip().splitlines()[-1])

    import torch

    from looped_transformer_decode_amd import binding as B

    dev = torch.device("cuda:0")
    L, d, T, Bt = wl.loops_per_group, wl.head_dim, wl.ctx, wl.batch
    print(f"[bench] workload={wl.name} chained={wl.chained}: generating inputs", file=sys.stderr, flush=True)
    inp = synth.generate(wl, seed=20261202, device=dev)
    cfg = B.config_for(wl)
    cache_bytes = B.rq_cache_bytes(cfg)
    cache = torch.zeros(cache_bytes, dtype=torch.uint8, device=dev)
    pos0 = torch.zeros(Bt, dtype=torch.int32, device=dev)
    for grp in range(wl.n_groups):
        st = inp.kv[grp].stride()
        B.rq_quantize_token(cfg, cache, inp.kv[grp], grp, pos0, inp.rot, Bt, T,
                            pending_strides=(st[4], st[2], st[0], st[1], st[3]))
    torch.cuda.synchronize()
    # bulk pack of the whole context (the step before decode), timed on a second run that
    # rewrites the same bytes
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record()
    for grp in range(wl.n_groups):
        st = inp.kv[grp].stride()
        B.rq_quantize_token(cfg, cache, inp.kv[grp], grp, pos0, inp.rot, Bt, T,
                            pending_strides=(st[4], st[2], st[0], st[1], st[3]))
    b1.record()
    torch.cuda.synchronize()
    bulk_ms = b0.elapsed_time(b1)
    n_rep = args.replicas or max(2, min(16, math.ceil(1.6e9 / cache_bytes)))
    caches = [cache] + [cache.clone() for _ in range(n_rep - 1)]
    print(f"[bench] packed context ({cache_bytes/1e6:.1f} MB), {n_rep} replicas", file=sys.stderr, flush=True)

    q = [inp.q[i].contiguous() for i in range(wl.n_loops)]
    k_cur = [inp.kv[i // L, i % L, 0, :, :, T].contiguous() for i in range(wl.n_loops)]
    v_cur = [inp.kv[i // L, i % L, 1, :, :, T].contiguous() for i in range(wl.n_loops)]
    ctx_len = torch.full((Bt,), T, dtype=torch.int32, device=dev)
    pending = torch.zeros(Bt, L, 2, wl.n_kv_heads, d, dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(B.rq_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    out = torch.empty(Bt, wl.n_q_heads, d, dtype=torch.float32, device=dev)
    sc = synth.sm_scale(d)
    n_loops = wl.n_loops
    ev = {}

    def step(s, timed):
        stream = torch.cuda.current_stream()
        for loop in range(n_loops):
            c = caches[(s * n_loops + loop) % n_rep]
            if timed:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            B.rq_decode_attention(cfg, c, loop, q[loop], k_cur[loop], v_cur[loop], pending, ctx_len, T, inp.rot,
                                  sc, out, ws, Bt, n_splits=args.splits, stream=stream)
            if timed:
                e1.record(stream)
                ev.setdefault(("dec", loop % L), []).append((e0, e1))
            if loop % L == L - 1:
                if timed:
                    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    p0.record(stream)
                B.rq_quantize_token(cfg, c, pending, loop // L, ctx_len, inp.rot, Bt, 1, stream=stream)
                if timed:
                    p1.record(stream)
                    ev.setdefault(("pack",), []).append((p0, p1))

    # per-kernel durations: eager steps with events around each call
    for s in range(args.warmup):
        step(s, False)
    for s in range(args.steps):
        step(args.warmup + s, True)
    torch.cuda.synchronize()

    if args.eager_only:
        t0 = time.perf_counter()
        for s in range(args.steps):
            step(args.warmup + args.steps + s, False)
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
        launch = "eager"
    else:
        # whole-step time: each step replayed from a HIP graph (one graph per replica pattern)
        n_pat = n_rep // math.gcd(n_rep, n_loops)
        graphs = []
        for p_ in range(n_pat):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(p_, False)
            graphs.append(g)
        torch.cuda.synchronize()
        for s in range(args.warmup):
            graphs[s % n_pat].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            graphs[s % n_pat].replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_step = (t1 - t0) * 1e3 / args.steps
        launch = "hip graph replay"
    stream = torch.cuda.current_stream()

    def avg_ms(key):
        v = [a.elapsed_time(b) for a, b in ev[key]]
        return sum(v) / len(v)

    per_loop = {l: avg_ms(("dec", l)) for l in range(L)}
    pack_ms = avg_ms(("pack",))
    step_bytes = sum(algorithmic_bytes(wl, l % L, wl.chained) for l in range(n_loops))
    res_loops = [l for l in range(L - 1)]
    res_ms = sum(per_loop[l] for l in res_loops) / len(res_loops)
    res_bytes = sum(algorithmic_bytes(wl, l, False) for l in res_loops) // len(res_loops)
    anchor_bytes = algorithmic_bytes(wl, L - 1, False)
    res_gbps = res_bytes / (res_ms * 1e-3) / 1e9

    # warm: single replica, residual loop 0 repeated
    for _ in range(3):
        B.rq_decode_attention(cfg, cache, 0, q[0], k_cur[0], v_cur[0], None, ctx_len, T, inp.rot, sc, out, ws, Bt,
                              n_splits=args.splits, stream=stream)
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(10):
        B.rq_decode_attention(cfg, cache, 0, q[0], k_cur[0], v_cur[0], None, ctx_len, T, inp.rot, sc, out, ws, Bt,
                              n_splits=args.splits, stream=stream)
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / 10

    # BF16 baseline on the same K/V: every loop of one anchor group (own K/V per loop)
    bcfg = B.bf16_config_for(wl)
    bws = torch.zeros(B.rq_bf16_workspace_bytes(bcfg), dtype=torch.uint8, device=dev)
    Ks = [inp.kv[0, l, 0] for l in range(L)]
    Vs = [inp.kv[0, l, 1] for l in range(L)]
    for l in range(L):
        B.rq_bf16_decode_attention(bcfg, Ks[l], Vs[l], q[l], k_cur[l], v_cur[l], False, ctx_len, T, sc, out, bws,
                                   Bt, n_splits=args.splits, stream=stream)
    bev = []
    for s in range(max(3, args.steps // 2)):
        for l in range(L):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            B.rq_bf16_decode_attention(bcfg, Ks[l], Vs[l], q[l], k_cur[l], v_cur[l], False, ctx_len, T, sc, out,
                                       bws, Bt, n_splits=args.splits, stream=stream)
            e1.record(stream)
            bev.append((e0, e1))
    torch.cuda.synchronize()
    bf16_ms = sum(a.elapsed_time(b) for a, b in bev) / len(bev)
    bf16_gbps = bf16_bytes(wl) / (bf16_ms * 1e-3) / 1e9

    # With grouped queries the BF16 kernel above reads every KV tile once per query head. The
    # same kernel with one query per KV head reads the same bytes once: a floor for any BF16
    # kernel that shares the tile across the group (it reads as much and computes more).
    bf16_once = None
    if wl.n_q_heads > wl.n_kv_heads:
        G = wl.n_q_heads // wl.n_kv_heads
        bcfg1 = B.rq_bf16_config(d, wl.n_kv_heads, wl.n_kv_heads, Bt, T + 1)
        bws1 = torch.zeros(B.rq_bf16_workspace_bytes(bcfg1), dtype=torch.uint8, device=dev)
        q1 = [q[l][:, ::G].contiguous() for l in range(L)]
        out1 = torch.empty(Bt, wl.n_kv_heads, d, dtype=torch.float32, device=dev)
        for l in range(L):
            B.rq_bf16_decode_attention(bcfg1, Ks[l], Vs[l], q1[l], k_cur[l], v_cur[l], False, ctx_len, T, sc, out1,
                                       bws1, Bt, n_splits=args.splits, stream=stream)
        b0_, b1_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(3, args.steps // 2) * L
        b0_.record(stream)
        for i in range(reps):
            l = i % L
            B.rq_bf16_decode_attention(bcfg1, Ks[l], Vs[l], q1[l], k_cur[l], v_cur[l], False, ctx_len, T, sc, out1,
                                       bws1, Bt, n_splits=args.splits, stream=stream)
        b1_.record(stream)
        torch.cuda.synchronize()
        bf16_once = b0_.elapsed_time(b1_) / reps

    # plain streaming read of the same replicas: the rate a simple load loop reaches here
    sink = torch.empty(B.STREAM_SINK_WORDS, dtype=torch.int32, device=dev)
    probe_bytes = res_bytes // 16 * 16

    def stream_gbps(nbytes, reps):
        for i in range(2):
            B.rq_stream_read(caches[i % n_rep], nbytes, sink, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            B.rq_stream_read(caches[(i + 2) % n_rep], nbytes, sink, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9

    stream_res = stream_gbps(min(probe_bytes, cache_bytes // 16 * 16), 4 * n_rep)
    stream_full = stream_gbps(cache_bytes // 16 * 16, 2 * n_rep)

    # the same residual loop-steps through block tables: every replica's tiles scattered
    # over one pool of 64-token blocks in a random order (rows and replicas interleaved)
    n_tiles = (cfg.max_ctx + 63) // 64
    blk_bytes = B.rq_paged_block_bytes(cfg)
    n_blocks = n_rep * Bt * n_tiles
    perm = torch.randperm(n_blocks, generator=torch.Generator().manual_seed(7)).to(torch.int32)
    tables = [perm[r * Bt * n_tiles:(r + 1) * Bt * n_tiles].reshape(Bt, n_tiles).contiguous().to(dev)
              for r in range(n_rep)]
    pool = torch.zeros(n_blocks * blk_bytes, dtype=torch.uint8, device=dev)
    for r in range(n_rep):
        for grp in range(wl.n_groups):
            st = inp.kv[grp].stride()
            B.rq_quantize_token_paged(cfg, pool, n_blocks, tables[r], inp.kv[grp], grp, pos0, inp.rot, Bt, T,
                                      pending_strides=(st[4], st[2], st[0], st[1], st[3]), stream=stream)
    for i in range(2 * (L - 1)):
        loop = i % (L - 1)
        B.rq_decode_attention_paged(cfg, pool, n_blocks, tables[i % n_rep], loop, q[loop], k_cur[loop], v_cur[loop],
                                    None, ctx_len, T, inp.rot, sc, out, ws, Bt, n_splits=args.splits, stream=stream)
    p0_, p1_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0_.record(stream)
    for i in range(6 * n_rep):
        loop = i % (L - 1)
        B.rq_decode_attention_paged(cfg, pool, n_blocks, tables[i % n_rep], loop, q[loop], k_cur[loop], v_cur[loop],
                                    None, ctx_len, T, inp.rot, sc, out, ws, Bt, n_splits=args.splits, stream=stream)
    p1_.record(stream)
    torch.cuda.synchronize()
    paged_ms = p0_.elapsed_time(p1_) / (6 * n_rep)
    del pool

    # K/V projection of the current token (the step before the pending buffer): back-to-back
    # calls over cold copies of the layer's weights (a model's other layers evict them between
    # two loops of this one), and warm on one copy (a looped layer re-reads its own weights)
    pin_ = synth.projection_inputs(wl, seed=20261203, device=dev)
    H = pin_.x.shape[-1]
    w_bytes = pin_.w.numel() * 2
    n_wrep = max(2, math.ceil(6.4e8 / w_bytes))
    wreps = [pin_.w] + [pin_.w.clone() for _ in range(n_wrep - 1)]
    pk = torch.empty(Bt, wl.n_kv_heads, d, dtype=torch.bfloat16, device=dev)
    pv = torch.empty_like(pk)
    ppend = torch.zeros_like(pending)

    def graph_ms(call, reps):
        """GPU time per call of `reps` calls captured in one HIP graph (no host launch cost)."""
        for i in range(2):
            call(i)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                call(i + 2)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    reps = 4 * n_wrep
    proj_cold = graph_ms(lambda i: B.rq_kv_project(cfg, pin_.x[i % n_loops], wreps[i % n_wrep], i % n_loops, pk, pv,
                                                   ppend, Bt), reps)
    proj_warm = graph_ms(lambda i: B.rq_kv_project(cfg, pin_.x[i % n_loops], wreps[0], i % n_loops, pk, pv, ppend,
                                                   Bt), reps)
    # references: a plain load loop over the same weight bytes (cold copies), and the same
    # launch with hidden = 32 (the grid, products and epilogue without the weight stream)
    proj_stream = graph_ms(lambda i: B.rq_stream_read(wreps[i % n_wrep], w_bytes, sink), reps)
    x32 = pin_.x[0][:, :32].contiguous()
    w32 = pin_.w[..., :32].contiguous()
    proj_floor = graph_ms(lambda i: B.rq_kv_project(cfg, x32, w32, 0, pk, pv, ppend, Bt), reps)
    proj_bytes = w_bytes + Bt * H * 2 + 2 * (Bt * 2 * wl.n_kv_heads * d * 2)

    # The decode step with the projection in front of every loop: rq_kv_project writes the loop's
    # current-token K/V and its pending slot, then attention runs.  The pack of the finished token
    # needs only the pending buffer, so it can run on a second stream beside the anchor loop's
    # attention (which reads token slots below ctx_len only; the pack writes slot ctx_len).
    side = torch.cuda.Stream()

    def step_proj(s_, overlap):
        main = torch.cuda.current_stream()
        for loop in range(n_loops):
            c = caches[(s_ * n_loops + loop) % n_rep]
            B.rq_kv_project(cfg, pin_.x[loop], wreps[(s_ * n_loops + loop) % n_wrep], loop, pk, pv, ppend, Bt)
            anchor = loop % L == L - 1
            if anchor and overlap:
                fork = torch.cuda.Event()
                fork.record(main)
                side.wait_event(fork)
                B.rq_quantize_token(cfg, c, ppend, loop // L, ctx_len, inp.rot, Bt, 1, stream=side)
            B.rq_decode_attention(cfg, c, loop, q[loop], pk, pv, None, ctx_len, T, inp.rot, sc, out, ws, Bt,
                                  n_splits=args.splits)
            if anchor and overlap:
                join = torch.cuda.Event()
                join.record(side)
                main.wait_event(join)
            elif anchor:
                B.rq_quantize_token(cfg, c, ppend, loop // L, ctx_len, inp.rot, Bt, 1)

    def step_graph_ms(overlap):
        for s_ in range(2):
            step_proj(s_, overlap)
        n_pat = n_rep // math.gcd(n_rep, n_loops)
        gs = []
        for p_ in range(n_pat):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_proj(p_, overlap)
            gs.append(g)
        for s_ in range(2):
            gs[s_ % n_pat].replay()
        torch.cuda.synchronize()
        t0_ = time.perf_counter()
        for s_ in range(args.steps):
            gs[s_ % n_pat].replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0_) * 1e3 / args.steps

    proj_step_seq = step_graph_ms(False)
    proj_step_ovl = step_graph_ms(True)
    del wreps

    # the batch-4 case beside the default batch-16 workload (before the roofline timing, so
    # that the roofline's dispatches stay the last decode dispatches of the run)
    batch4 = None
    if args.workload == DEFAULT_WORKLOAD and not variant and not args.chained and not args.no_batch4:
        print("[bench] batch-4 loop-steps", file=sys.stderr, flush=True)
        batch4 = measure_loop_steps(B, dev, "ouro_b4_t8192", args.splits)
        torch.cuda.empty_cache()

    # roofline timing: back-to-back residual loop-steps over the cold replicas, one event
    # pair around all of them (launches overlap the previous kernel, as in a decode step)
    roof_calls = 6 * n_rep
    roof_reps = []
    for _ in range(3):
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r0.record(stream)
        for i in range(roof_calls):
            loop = i % (L - 1)
            B.rq_decode_attention(cfg, caches[i % n_rep], loop, q[loop], k_cur[loop], v_cur[loop], None, ctx_len,
                                  T, inp.rot, sc, out, ws, Bt, n_splits=args.splits, stream=stream)
        r1.record(stream)
        torch.cuda.synchronize()
        roof_reps.append(r0.elapsed_time(r1) / roof_calls)
    roof_ms = sum(roof_reps) / len(roof_reps)
    roof_bytes = sum(algorithmic_bytes(wl, i % (L - 1), wl.chained) for i in range(roof_calls)) / roof_calls
    roof_gbps = roof_bytes / (roof_ms * 1e-3) / 1e9


    value = step_bytes / (ms_step * 1e-3) / 1e9
    traffic = measured_traffic(wl.name) if not wl.chained and args.splits == 0 else None
    result = {
        "metric": "RQ decode-attn HBM GB/s (% of peak) & KV-tokens/s read, vs BF16 decode",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4/u2 codes; i32 key dots (v_dot8 on fixed-point q and R_K q digits); f32 softmax, value sums and output",
        "data": "synthetic (seeded stand-in for Ouro/Huginn K/V: anchor N(0,1) with x8 key outliers, "
                "loops a_l*anchor + 0.15 N(0,1) + drift), random orthogonal rotations",
        "config": {"workload": wl.name, "batch": Bt, "ctx": T, "n_q_heads": wl.n_q_heads,
                   "n_kv_heads": wl.n_kv_heads, "head_dim": d, "loops": wl.n_loops,
                   "loops_per_group": L, "group": wl.group, "anchor_bits": wl.anchor_bits,
                   "resid_bits": wl.resid_bits, "chained": wl.chained, "scale_rule": wl.scale_rule,
                   "resid_bits_loop": list(wl.resid_bits_loop),
                   "cache_replicas": n_rep},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "kv_tokens_per_s": round(Bt * T / (res_ms * 1e-3), 1),
        "step": {"bytes": step_bytes, "ms_wall": round(ms_step, 4), "launch": launch,
                 "ms_per_loop_step": {str(l): round(v, 4) for l, v in per_loop.items()},
                 "ms_pack": round(pack_ms, 4), "pack_tokens_per_s": round(Bt / (pack_ms * 1e-3), 1)},
        "residual_loop_step": {"bytes": res_bytes, "ms": round(res_ms, 4), "gbps": round(res_gbps, 1),
                               "warm_single_replica_ms": round(warm_ms, 4)},
        "anchor_loop_step": {"bytes": anchor_bytes, "ms": round(per_loop[L - 1], 4),
                             "gbps": round(anchor_bytes / (per_loop[L - 1] * 1e-3) / 1e9, 1)},
        "bf16": {"bytes": bf16_bytes(wl), "ms_per_loop_step": round(bf16_ms, 4), "gbps": round(bf16_gbps, 1),
                 "speedup_rq_residual_vs_bf16": round(bf16_ms / res_ms, 3),
                 "speedup_rq_step_vs_bf16_step": round(bf16_ms * n_loops / ms_step, 3),
                 **({"one_query_per_kv_head_ms": round(bf16_once, 4),
                     "speedup_rq_residual_vs_bf16_one_query_per_kv_head": round(bf16_once / res_ms, 3)}
                    if bf16_once is not None else {})},
        "bulk_pack": {"tokens": Bt * T, "ms": round(bulk_ms, 3),
                      "tokens_per_s": round(Bt * T / (bulk_ms * 1e-3), 1),
                      "bf16_in_bytes": bulk_in_bytes(wl), "gbps_in": round(bulk_in_bytes(wl) / (bulk_ms * 1e-3) / 1e9, 1),
                      "rotation_fma": rotation_fma(wl),
                      "f64_tflops": round(2 * rotation_fma(wl) / (bulk_ms * 1e-3) / 1e12, 2)},
        "stream_read": {"kernel": "rq_stream_read (plain 16-byte load loop over the same cache replicas)",
                        "gbps_at_residual_step_bytes": round(stream_res, 1),
                        "gbps_at_full_replica": round(stream_full, 1),
                        "residual_step_frac_of_stream": round(roof_gbps / stream_res, 4)},
        "paged": {"block_tokens": 64, "n_blocks": n_blocks, "block_bytes": blk_bytes,
                  "residual_loop_step_ms": round(paged_ms, 4),
                  "gbps": round(roof_bytes / (paged_ms * 1e-3) / 1e9, 1),
                  "vs_contiguous": round(roof_ms / paged_ms, 4),
                  "timing": "HIP events around back-to-back residual loop-steps through shuffled block tables "
                            "(one per replica, blocks of all replicas interleaved in one pool)"},
        "kv_project": {"hidden": H, "outputs": 2 * wl.n_kv_heads * d, "weight_bytes": w_bytes,
                       "bytes": proj_bytes, "ms": round(proj_cold, 4),
                       "gbps": round(proj_bytes / (proj_cold * 1e-3) / 1e9, 1),
                       "frac_of_hbm_peak": round(proj_bytes / (proj_cold * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                       "warm_ms": round(proj_warm, 4), "weight_replicas": n_wrep,
                       "step_with_projection_ms": round(proj_step_seq, 4),
                       "step_with_projection_pack_beside_anchor_ms": round(proj_step_ovl, 4),
                       "stream_read_same_bytes_ms": round(proj_stream, 4),
                       "launch_hidden32_ms": round(proj_floor, 4),
                       "timing": "HIP graph of back-to-back rq_kv_project calls (BF16 K/V of the current "
                                 "token into k_cur/v_cur and the pending slot) over cold weight copies, one "
                                 "event pair around its replay; warm_ms on one copy"},
        "roofline": {"bound": "hbm", "achieved": round(roof_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(roof_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "ms_per_launch": round(roof_ms, 4), "launches": 3 * roof_calls,
                     "repeats_ms_per_launch": [round(v, 4) for v in roof_reps],
                     "min_frac": round(roof_bytes / (min(roof_reps) * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "timing": "HIP events around back-to-back residual loop-steps (loops 0..L-2, cold replicas), "
                               "on the library's stream, the last decode dispatches of the run; mean of 3 "
                               "repeats (min_frac: the fastest repeat)",
                     "kernel": ("rq_decode_gqa_kernel" if grouped_kernel(wl) else "rq_decode_kernel")
                     + ", residual loop-step (split-K with the merge in its last workgroup)",
                     "algorithmic_bytes": round(roof_bytes), "source_digest": decode_source_digest(wl)},
    }
    if batch4 is not None:
        result["ouro_b4_t8192"] = batch4
    if not args.no_w4a4:
        result["w4a4"] = measure_w4a4(B, dev, sink, eager=args.eager_only)
        result["w4a4_huginn"] = measure_w4a4(B, dev, sink, eager=args.eager_only, name="huginn_up_b8")
    if cpu_base is not None:
        result["cpu_baseline"] = cpu_base
    print(json.dumps(result))


if __name__ == "__main__":
    main()
