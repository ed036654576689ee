"""GPU parity of rq_kv_project (the K/V projection whose epilogue writes the decode step's
current-token inputs and the pending buffer) against the float64 oracle, through the C ABI.

Parity rule (BF16 outputs of float32 sums of exact products):
* every output equals the oracle's exactly rounded BF16 value, except outputs whose exact
  value lies within E = 6 * sqrt(hidden) * 2^-24 * sum_c |x_c w_c| of the rounding midpoint
  between the oracle's value and the GPU's; there the GPU may return the other neighbour.
  E is the probabilistic bound (lambda = 6) on the error of a float32 sum of `hidden`
  products, in any order;
* such midpoint cases are counted and must stay below 1% of the outputs;
* the pending slot of the loop is written, every other slot keeps its bytes.
"""
import math

import numpy as np
import pytest
import torch

from looped_transformer_decode_amd import synth
from oracle import formats as F
from oracle import projection as P

from _support import say

pytestmark = pytest.mark.gpu

LAMBDA = 6.0


@pytest.fixture(scope="module")
def B():
    from looped_transformer_decode_amd import binding
    return binding


W = synth.WORKLOADS
CASES = {
    # name: (workload, batch, hidden, loop, n_kv_heads override, x row padding)
    "ouro_b4_t8192": (W["ouro_b4_t8192"], 4, None, 3, None, 0),
    "ouro_b16_t8192": (W["ouro_b16_t8192"], 16, None, 1, None, 0),
    "huginn_gqa4_b8_t8192": (W["huginn_gqa4_b8_t8192"], 8, None, 13, None, 0),
    "tiny_d64": (W["tiny_d64_t256"], 1, None, 2, None, 0),
    "ragged_hidden96_strided": (W["ouro_b4_t8192"], 3, 96, 0, 2, 40),
    "rows20_two_tiles": (W["tiny_d64_t256"].with_(batch=24), 20, 1024, 1, None, 0),
    "rows40_four_tiles": (W["tiny_d64_t256"].with_(batch=64), 40, 512, 3, None, 8),
    "hidden8192_two_rounds": (W["ouro_b4_t8192"], 2, 8192, 2, 2, 0),
    # x too large to stage in LDS (16 rows x 8192): A operands loaded per wave
    "rows16_hidden8192_unstaged": (W["ouro_b16_t8192"], 16, 8192, 0, 2, 0),
    # 64 rows (four full row tiles) and the largest hidden (16 k-steps per wave per round, two rounds)
    "rows64_four_full_tiles": (W["tiny_d64_t256"].with_(batch=64), 64, 256, 1, None, 0),
    "max_hidden65536": (W["tiny_d64_t256"], 1, 65536, 3, None, 0),
}


def check_bf16(got_bits: np.ndarray, exact: np.ndarray, mags: np.ndarray, hidden: int, what: str) -> int:
    want = F.bf16_round(exact)
    got = F.bf16_from_bits(got_bits)
    bad = got != want
    n_bad = int(bad.sum())
    if n_bad:
        wb = F.bf16_bits(want[bad]).astype(np.int64)
        gb = got_bits[bad].astype(np.int64)
        same_sign = (wb & 0x8000) == (gb & 0x8000)
        neighbour = same_sign & (np.abs((wb & 0x7FFF) - (gb & 0x7FFF)) == 1)
        mid = (got[bad] + want[bad]) / 2
        e_bound = LAMBDA * math.sqrt(hidden) * 2.0 ** -24 * mags[bad]
        near = np.abs(exact[bad] - mid) <= e_bound
        ok = neighbour & near
        assert ok.all(), (f"{what}: {int((~ok).sum())} outputs differ from the oracle beyond the "
                          f"midpoint rule, e.g. got {got[bad][~ok][:4]} want {want[bad][~ok][:4]} "
                          f"exact {exact[bad][~ok][:4]}")
    assert n_bad <= 0.01 * exact.size, f"{what}: {n_bad} midpoint cases of {exact.size}"
    return n_bad


def _run(B, name, with_cur=True, with_pending=True):
    wl, batch, hidden, loop, hkv, pad = CASES[name]
    if hkv:
        wl = wl.with_(n_kv_heads=hkv, n_q_heads=hkv)
    say(f"[kv_project] case={name} batch={batch} hidden={hidden or synth.model_width(wl)} loop={loop} "
        f"cur={with_cur} pending={with_pending}")
    dev = torch.device("cuda:0")
    inp = synth.projection_inputs(wl, seed=77, batch=batch, hidden=hidden)
    H = inp.x.shape[-1]
    x_host = inp.x[loop]
    if pad:
        xs = torch.zeros(batch, H + pad, dtype=torch.bfloat16)
        xs[:, :H] = x_host
        x_dev = xs.to(dev)[:, :H]
        assert x_dev.stride(0) == H + pad
    else:
        x_dev = x_host.to(dev)
    w_dev = inp.w.to(dev)
    cfg = B.config_for(wl, max_batch=max(batch, wl.batch))
    L, hkv_, d = wl.loops_per_group, wl.n_kv_heads, wl.head_dim
    k_cur = torch.empty(batch, hkv_, d, dtype=torch.bfloat16, device=dev) if with_cur else None
    v_cur = torch.empty(batch, hkv_, d, dtype=torch.bfloat16, device=dev) if with_cur else None
    g = torch.Generator().manual_seed(5)
    pend0 = torch.randn(batch, L, 2, hkv_, d, generator=g).to(torch.bfloat16)
    pending = pend0.to(dev) if with_pending else None
    B.rq_kv_project(cfg, x_dev, w_dev, loop, k_cur, v_cur, pending, batch)
    torch.cuda.synchronize()

    x64 = x_host.double().numpy()
    w64 = inp.w.double().numpy()
    exact, _ = P.kv_projection(x64, w64)
    mags = P.magnitude_sums(x64, w64)
    n_mid = 0
    if with_cur:
        for xx, t in ((0, k_cur), (1, v_cur)):
            bits = t.cpu().view(torch.int16).numpy().astype(np.uint16)
            n_mid += check_bf16(bits, exact[xx], mags[xx], H, f"{name} {'KV'[xx]}")
    if with_pending:
        got = pending.cpu()
        lloc = loop % L
        keep = [l for l in range(L) if l != lloc]
        assert torch.equal(got[:, keep].view(torch.int16), pend0[:, keep].view(torch.int16)), "other slots changed"
        for xx in range(2):
            bits = got[:, lloc, xx].view(torch.int16).numpy().astype(np.uint16)
            n_mid += check_bf16(bits, exact[xx], mags[xx], H, f"{name} pending {'KV'[xx]}")
    say(f"[kv_project] case={name}: ok, {n_mid} midpoint cases of {2 * exact.size * (int(with_cur) + int(with_pending))}")


@pytest.mark.parametrize("name", sorted(CASES))
def test_kv_project_parity(B, name):
    _run(B, name)


def test_kv_project_pending_only(B):
    _run(B, "huginn_gqa4_b8_t8192", with_cur=False, with_pending=True)


def test_kv_project_current_only(B):
    _run(B, "ragged_hidden96_strided", with_cur=True, with_pending=False)


def test_kv_project_matches_k_cur_of_decode_inputs(B):
    """The BF16 K/V the projection writes are bit-identical in k_cur/v_cur and the pending slot."""
    wl = W["ouro_b4_t8192"]
    dev = torch.device("cuda:0")
    inp = synth.projection_inputs(wl, seed=3)
    cfg = B.config_for(wl)
    k = torch.empty(wl.batch, wl.n_kv_heads, wl.head_dim, dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    pending = torch.zeros(wl.batch, wl.loops_per_group, 2, wl.n_kv_heads, wl.head_dim, dtype=torch.bfloat16,
                          device=dev)
    for loop in range(wl.loops_per_group):
        B.rq_kv_project(cfg, inp.x[loop].to(dev), inp.w.to(dev), loop, k, v, pending, wl.batch)
        torch.cuda.synchronize()
        assert torch.equal(pending[:, loop, 0].view(torch.int16), k.view(torch.int16))
        assert torch.equal(pending[:, loop, 1].view(torch.int16), v.view(torch.int16))
