"""GPU check of rq_unpack_debug against the oracle's own unpacker: the float32 vectors
the library rebuilds from a GPU-packed cache must equal the oracle's float64 rebuild of
the same bytes (read_tokens + reconstruct), for every loop of every anchor group, shared
and chained, on a ragged slot range.

Tolerance: the dequantized anchor values z + code * s are exact in float32, so anchor
loops must match exactly.  A residual loop adds R^T r_hat, a float32 sum of d products,
and a chained loop nests up to three of them; each sum is within d * 2^-24 * sum|R_ki r_k|
of the exact value, which the test bounds by 1e-5 * max|x| + 1e-6 per tensor (d <= 128,
|R_ki| <= 1, |r_hat| well below max|x| for these inputs)."""
import numpy as np
import pytest
import torch

from looped_transformer_decode_amd import synth
from oracle import residualquant as RQ

from _support import device_block, gpu_pack, oracle_cfg, say, sub_cache

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
CASES = {
    # name: (workload, chained, batch, ctx, n_kv_heads, n_q_heads, slot range)
    "tiny": (W["tiny_d64_t256"], False, 1, 256, None, None, (5, 203)),
    "tiny_chained": (W["tiny_d64_t256"], True, 1, 256, None, None, (0, 256)),
    "d128g16int2_chained": (W["int2g16_b4_t16384"], True, 2, 190, 2, 2, (63, 190)),
    "gqa4_two_groups": (W["huginn_gqa4_b8_t8192"].with_(n_groups=2), False, 2, 130, 2, 8, (1, 129)),
    "widths_422": (W["ouro_b4_t8192"].with_(resid_bits_loop=(4, 2, 2)), False, 2, 150, 2, 2, (3, 150)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_unpack_matches_oracle_rebuild(name):
    from looped_transformer_decode_amd import binding as B
    wl, chained, batch, T, hkv, hq, (t0, t1) = CASES[name]
    wl = wl.with_(batch=batch, ctx=T, chained=chained, n_kv_heads=hkv or wl.n_kv_heads,
                  n_q_heads=hq or wl.n_q_heads)
    say(f"[unpack] case={name} T={T} slots=[{t0},{t1})")
    inp = synth.generate(wl, seed=77, device="cuda")
    cfg = B.config_for(wl)
    ocfg = oracle_cfg(wl)
    cache = gpu_pack(B, cfg, inp.kv, inp.rot, T)
    rot = inp.rot.double().cpu().numpy()
    L, d = wl.loops_per_group, wl.head_dim
    for loop in range(wl.n_loops):
        out = torch.full((wl.batch, wl.n_kv_heads, 2, t1 - t0, d), float("nan"), device="cuda")
        B.rq_unpack_debug(cfg, cache, loop, inp.rot, t0, t1, wl.batch, out)
        torch.cuda.synchronize()
        got = out.double().cpu().numpy()
        grp, l = divmod(loop, L)
        for b in range(wl.batch):
            for h in range(wl.n_kv_heads):
                block = device_block(cache, ocfg, b, h)
                _, sub = sub_cache(np.zeros(0, np.uint8), ocfg, b, h)
                lay = RQ.Layout(sub)
                for x in range(2):
                    enc = RQ.read_tokens(block, lay, 0, 0, x, grp, t1)
                    ref = RQ.reconstruct(enc, l, rot[h, x], sub)[t0:t1]
                    g = got[b, h, x]
                    if l == L - 1:
                        assert np.array_equal(g, ref), (loop, b, h, x)
                    else:
                        err = np.abs(g - ref).max()
                        assert err <= 1e-5 * np.abs(ref).max() + 1e-6, (loop, b, h, x, err)
