"""Seeded synthetic inputs for the ResidualQuant decode path.

This module only draws random numbers and lays them out; it contains none of
the quantization or attention arithmetic, so both the GPU path and the CPU
oracle can take their inputs from it.

The pages ("ResidualQuant ..." explainer, section on the looped Transformer and
the worked example; the arXiv digest, Figure 1 caption and section 5.3) measure
on Ouro-1.4B (4 loops) and Huginn-3.5B (32 loops, 8 groups of 4) with real
benchmark prompts.  Those weights and datasets are not available, so every
workload here is a seeded stand-in with the same shapes:

* anchor-loop K/V ~ N(0, 1); for keys a few fixed "outlier" channels per KV head
  are scaled by 8 (the explainer notes that raw keys carry large outliers);
* every earlier loop l is ``a_l * anchor + 0.15 * N(0, 1) (+ drift_l)``, i.e.
  close to the last loop, which is the cross-loop similarity the method relies on;
* the drift term is one N(0, 1) * drift vector per (loop, KV head, K|V), shared
  by all tokens;
* rotations are Haar-random orthogonal matrices (QR of a Gaussian with the
  signs of diag(R) folded in), one per (KV head, K|V), made in float64 and stored
  as float32.

All K/V values are rounded to bfloat16, which is what a BF16 model writes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple, Union

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    ctx: int                 # context tokens already in the cache (the current token is extra)
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    loops_per_group: int     # L: loops that share one anchor (the last of them is the anchor)
    n_groups: int            # anchor groups; total loops = L * n_groups
    group: int               # channels per quantization group
    anchor_bits: int
    resid_bits: int
    n_outliers: int          # outlier key channels per KV head (scaled x8)
    drift: float             # std of the per-loop drift vector shared across tokens
    loop_scale: Union[Tuple[float, ...], str]   # a_l for loops 0..L-2, or "uniform(0.8,1.0)"
    q_dtype: str             # "fp32" | "bf16"
    chained: bool = False
    scale_rule: int = 0      # 0: least-squares c; 1: norm-ratio c
    resid_bits_loop: Tuple[int, ...] = ()   # residual width per local loop 0..L-2 (empty: resid_bits)

    @property
    def n_loops(self) -> int:
        return self.loops_per_group * self.n_groups

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_A = (0.85, 0.90, 0.95)

#: The five seeded workloads.  Names state what they are and their sizes.
WORKLOADS = {
    # one sequence, head_dim 64, 256 context tokens: small enough for brute force
    "tiny_d64_t256": Workload("tiny_d64_t256", 1, 256, 2, 2, 64, 4, 1, 32, 4, 2,
                              2, 0.0, _A, "fp32"),
    # Ouro-1.4B-sized looped layer, 8k context, batch 4
    "ouro_b4_t8192": Workload("ouro_b4_t8192", 4, 8192, 16, 16, 128, 4, 1, 32, 4, 2,
                              4, 0.05, _A, "bf16"),
    # capacity case: batch 16 at 8k context
    "ouro_b16_t8192": Workload("ouro_b16_t8192", 16, 8192, 16, 16, 128, 4, 1, 32, 4, 2,
                               4, 0.05, _A, "bf16"),
    # long context, uniform INT2 with 16-channel groups (also run chained)
    "int2g16_b4_t16384": Workload("int2g16_b4_t16384", 4, 16384, 16, 16, 128, 4, 1, 16, 2, 2,
                                  4, 0.05, _A, "bf16"),
    # Huginn-3.5B-sized deep loop: 32 loops = 8 anchor groups of 4, GQA 32 q / 8 kv heads
    "huginn_gqa4_b8_t8192": Workload("huginn_gqa4_b8_t8192", 8, 8192, 32, 8, 128, 4, 8, 32, 4, 2,
                                     4, 0.05, "uniform(0.8,1.0)", "bf16"),
}


@dataclasses.dataclass
class Inputs:
    wl: Workload
    kv: torch.Tensor        # [n_groups][L][2][B][Hkv][ctx+1][d] bf16; token index ctx is the current token
    q: torch.Tensor         # [n_loops][B][Hq][d] fp32 or bf16
    rot: torch.Tensor       # [Hkv][2][d][d] fp32, orthogonal
    loop_scale: torch.Tensor  # [n_groups][L-1] fp32, the a_l used
    outliers: torch.Tensor  # [Hkv][n_outliers] int64 key channels scaled x8


def haar_rotations(n_kv_heads: int, head_dim: int, seed: int) -> torch.Tensor:
    """[Hkv][2][d][d] float32 orthogonal matrices (QR of a float64 Gaussian, sign-fixed)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    out = torch.empty(n_kv_heads, 2, head_dim, head_dim, dtype=torch.float64)
    for h in range(n_kv_heads):
        for x in range(2):
            a = torch.randn(head_dim, head_dim, generator=g, dtype=torch.float64)
            qm, rm = torch.linalg.qr(a)
            qm = qm * torch.sign(torch.diagonal(rm)).unsqueeze(0)
            out[h, x] = qm
    return out.to(torch.float32)


def generate(wl: Workload, seed: int = 20261202, device: Union[str, torch.device] = "cpu",
             batch: Optional[int] = None, ctx: Optional[int] = None) -> Inputs:
    """Draw one workload.  ``batch``/``ctx`` override the workload's sizes (for small tests)."""
    if batch is not None or ctx is not None:
        wl = wl.with_(batch=batch if batch is not None else wl.batch,
                      ctx=ctx if ctx is not None else wl.ctx)
    dev = torch.device(device)
    B, T, Hq, Hkv, d, L, G = (wl.batch, wl.ctx, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                              wl.loops_per_group, wl.n_groups)
    cpu = torch.Generator(device="cpu")
    cpu.manual_seed(seed)
    # per-head outlier channels and per-loop scales come from the CPU generator (cheap, device independent)
    outliers = torch.stack([torch.randperm(d, generator=cpu)[: wl.n_outliers] for _ in range(Hkv)])
    if isinstance(wl.loop_scale, str):
        lo, hi = (float(v) for v in wl.loop_scale[len("uniform("):-1].split(","))
        scale = lo + (hi - lo) * torch.rand(G, L - 1, generator=cpu)
    else:
        scale = torch.tensor(wl.loop_scale, dtype=torch.float32).expand(G, L - 1).clone()
    drift = wl.drift * torch.randn(G, L - 1, 2, Hkv, d, generator=cpu)
    rot = haar_rotations(Hkv, d, seed + 7)

    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 1)
    kv = torch.empty(G, L, 2, B, Hkv, T + 1, d, dtype=torch.bfloat16, device=dev)
    out_mask = torch.ones(Hkv, d, dtype=torch.float32)
    for h in range(Hkv):
        out_mask[h, outliers[h]] = 8.0
    out_mask = out_mask.to(dev).view(1, Hkv, 1, d)
    for k in range(G):
        for x in range(2):
            anchor = torch.randn(B, Hkv, T + 1, d, generator=gen, device=dev, dtype=torch.float32)
            if x == 0 and wl.n_outliers:
                anchor.mul_(out_mask)
            kv[k, L - 1, x] = anchor.to(torch.bfloat16)
            for l in range(L - 1):
                noise = torch.randn(B, Hkv, T + 1, d, generator=gen, device=dev, dtype=torch.float32)
                val = float(scale[k, l]) * anchor + 0.15 * noise
                val += drift[k, l, x].to(dev).view(1, Hkv, 1, d)
                kv[k, l, x] = val.to(torch.bfloat16)
            del anchor
    qdt = torch.float32 if wl.q_dtype == "fp32" else torch.bfloat16
    q = torch.randn(wl.n_loops, B, Hq, d, generator=gen, device=dev, dtype=torch.float32).to(qdt)
    return Inputs(wl, kv, q, rot.to(dev), scale, outliers)


def sm_scale(head_dim: int) -> float:
    """Softmax temperature 1/sqrt(d) (the pages give none; standard scaled dot-product attention)."""
    return 1.0 / math.sqrt(head_dim)


@dataclasses.dataclass
class ProjectionInputs:
    x: torch.Tensor         # [n_loops][B][hidden] bf16: the hidden state each loop projects
    w: torch.Tensor         # [2][Hkv][d][hidden] bf16: the layer's K and V weight rows


def model_width(wl: Workload) -> int:
    """Hidden size of the stand-in model: n_q_heads * head_dim (2048 for the Ouro-1.4B-sized
    layer, 4096 for the 32-query-head one)."""
    return wl.n_q_heads * wl.head_dim


def projection_inputs(wl: Workload, seed: int = 20261203, device: Union[str, torch.device] = "cpu",
                      batch: Optional[int] = None, hidden: Optional[int] = None) -> ProjectionInputs:
    """Hidden states ~ N(0, 1) (the output of a normalisation layer) and weights ~ N(0, 1/hidden),
    so that K and V come out of unit scale like the cache generator's; all rounded to BF16."""
    B = batch if batch is not None else wl.batch
    H = hidden if hidden is not None else model_width(wl)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    x = torch.randn(wl.n_loops, B, H, generator=gen, dtype=torch.float32)
    w = torch.randn(2, wl.n_kv_heads, wl.head_dim, H, generator=gen, dtype=torch.float32) / math.sqrt(H)
    return ProjectionInputs(x.to(torch.bfloat16).to(device), w.to(torch.bfloat16).to(device))


# ---- W4A4 linear layer of a looped block (cross-loop residual activations)

@dataclasses.dataclass(frozen=True)
class W4A4Workload:
    name: str
    in_features: int         # K
    out_features: int        # N
    tokens: int              # decode batch
    loops: int               # loops of one group (loop 0 is the anchor)


#: Linear layers of an Ouro-1.4B-sized looped block (model width 2048) at decode.
W4A4_WORKLOADS = {
    # the MLP's up projection (4x width) for a decode batch of 16, one group of 4 loops
    "ouro_up_b16": W4A4Workload("ouro_up_b16", 2048, 8192, 16, 4),
    # the same for a Huginn-sized block (model width 4096) at its decode batch of 8
    "huginn_up_b8": W4A4Workload("huginn_up_b8", 4096, 16384, 8, 4),
    # a small case the float64 oracle checks in full
    "tiny_w4a4": W4A4Workload("tiny_w4a4", 1024, 64, 3, 3),
}


@dataclasses.dataclass
class W4A4Inputs:
    w: torch.Tensor          # [N][K] bf16
    rot: torch.Tensor        # [128][128] fp32, orthogonal
    x: torch.Tensor          # [L][M][K] bf16 activations of loops 0..L-1


def w4a4_inputs(wl: W4A4Workload, seed: int = 20261204, device: Union[str, torch.device] = "cpu",
                tokens: Optional[int] = None) -> W4A4Inputs:
    """Weights ~ N(0, 1/K); the anchor loop's activations ~ N(0, 1) with 8 outlier channels
    per token (x8, shared by every token and loop, as in normalised hidden states of LLMs);
    loop l >= 1: a_l * x0 + 0.15 N(0, 1) with a_l ~ U(0.8, 1.0) per token.  All BF16."""
    M = tokens if tokens is not None else wl.tokens
    K, N, L = wl.in_features, wl.out_features, wl.loops
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    w = torch.randn(N, K, generator=gen, dtype=torch.float64) / math.sqrt(K)
    x0 = torch.randn(M, K, generator=gen, dtype=torch.float64)
    out_ch = torch.randperm(K, generator=gen)[:8]
    x0[:, out_ch] *= 8.0
    xs = [x0]
    for _ in range(1, L):
        a = 0.8 + 0.2 * torch.rand(M, 1, generator=gen, dtype=torch.float64)
        xs.append(a * x0 + 0.15 * torch.randn(M, K, generator=gen, dtype=torch.float64))
    q, r = torch.linalg.qr(torch.randn(128, 128, generator=gen, dtype=torch.float64))
    rot = (q * torch.sign(torch.diagonal(r))).to(torch.float32).contiguous()
    return W4A4Inputs(w.to(torch.bfloat16).to(device), rot.to(device),
                      torch.stack(xs).to(torch.bfloat16).to(device))
