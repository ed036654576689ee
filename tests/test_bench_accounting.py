"""The benchmark's byte accounting (the numerator of every GB/s it reports) against the
oracle's cache layout and closed forms: a loop-step reads, for every
context token and KV head, K and V of the anchor plane and of the residual planes it needs.
Also the benchmark's refusal of multi-GPU launches."""
import pytest

import bench
from looped_transformer_decode_amd import synth
from oracle import residualquant as RQ


def _layout(wl):
    return RQ.Layout(RQ.Config(wl.head_dim, wl.group, wl.anchor_bits, wl.resid_bits, wl.loops_per_group,
                               wl.n_groups, wl.chained, wl.n_kv_heads, wl.n_q_heads, wl.batch, wl.ctx + 1))


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_loop_step_bytes_follow_the_layout(name):
    wl = synth.WORKLOADS[name]
    a, r = _layout(wl).bytes_per_token_head()
    heads_tokens = wl.batch * wl.ctx * wl.n_kv_heads
    L = wl.loops_per_group
    for loop in range(L):
        n_res = 0 if loop == L - 1 else 1
        assert bench.algorithmic_bytes(wl, loop, False) == 2 * (a + n_res * r) * heads_tokens
        n_chain = 0 if loop == L - 1 else L - 1 - loop        # chained: residual planes loop..L-2
        assert bench.algorithmic_bytes(wl, loop, True) == 2 * (a + n_chain * r) * heads_tokens
    assert bench.bf16_bytes(wl) == 2 * 2 * wl.head_dim * heads_tokens


def test_ouro_b4_figures():
    # 72 B anchor and 42 B residual per token, head and K|V at head_dim 128, g = 32, INT4/INT2
    wl = synth.WORKLOADS["ouro_b4_t8192"]
    assert _layout(wl).bytes_per_token_head() == (72, 42)
    assert bench.algorithmic_bytes(wl, 0, False) == 119537664         # 2 * 114 * 4 * 8192 * 16
    assert bench.algorithmic_bytes(wl, 3, False) == 75497472          # 2 * 72 * 4 * 8192 * 16
    assert bench.bf16_bytes(wl) == 268435456                          # 4 * 128 * 4 * 8192 * 16


def test_ouro_b16_figures():
    # the benchmark's default workload: batch 16 at 8k context
    import bench as bn
    assert bn.DEFAULT_WORKLOAD == "ouro_b16_t8192"
    wl = synth.WORKLOADS["ouro_b16_t8192"]
    assert bench.algorithmic_bytes(wl, 0, False) == 478150656         # 2 * 114 * 16 * 8192 * 16
    assert bench.algorithmic_bytes(wl, 3, False) == 301989888         # 2 * 72 * 16 * 8192 * 16
    assert bench.bf16_bytes(wl) == 1073741824                         # 4 * 128 * 16 * 8192 * 16


def test_bulk_pack_and_rotation_counts():
    wl = synth.WORKLOADS["ouro_b4_t8192"]
    # every loop's BF16 K and V of every context token, read once
    assert bench.bulk_in_bytes(wl) == wl.batch * wl.ctx * 4 * 2 * wl.n_kv_heads * wl.head_dim * 2
    # one d x d product per residual vector
    assert bench.rotation_fma(wl) == wl.batch * wl.ctx * wl.n_kv_heads * 2 * 3 * wl.head_dim ** 2
    # chained: loops 2 and 1 also rebuild their reference for loops 1 and 0 (R^T r_hat)
    assert bench.rotation_fma(wl.with_(chained=True)) == wl.batch * wl.ctx * wl.n_kv_heads * 2 * 5 * wl.head_dim ** 2


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus above 1 (or a multi-rank launch) exits with status 2
    and says why, before touching a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *argv], capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=60)
        assert r.returncode == 2
        assert "one GPU" in r.stderr and r.stdout == ""


def test_loop_step_bytes_with_per_loop_widths():
    """Residual widths 4, 2, 2: loop 0 reads its 74-byte residual rows, loops 1 and 2 their
    42-byte ones, beside the 72-byte anchor rows (per token, head and K|V)."""
    wl = synth.WORKLOADS["ouro_b4_t8192"].with_(resid_bits_loop=(4, 2, 2))
    ht = wl.batch * wl.ctx * wl.n_kv_heads
    lay = RQ.Layout(RQ.Config(wl.head_dim, wl.group, wl.anchor_bits, wl.resid_bits, 4, 1, False, wl.n_kv_heads,
                              wl.n_q_heads, wl.batch, wl.ctx + 1, 0, (4, 2, 2)))
    per = lay.bytes_per_token_loop()
    assert per == [74, 42, 42, 72]
    assert [bench.algorithmic_bytes(wl, l, False) for l in range(4)] == \
        [2 * (72 + 74) * ht, 2 * (72 + 42) * ht, 2 * (72 + 42) * ht, 2 * 72 * ht]


def test_w4a4_bytes_match_the_layouts():
    """The W4A4 loop-step byte counts against the oracle's layouts: packed weights, the BF16
    activations, activation rows (written; and the anchor rows read at a residual loop),
    and the float32 output and anchor product."""
    import bench
    from looped_transformer_decode_amd import synth
    from oracle import w4a4 as W4
    wl = synth.W4A4_WORKLOADS["ouro_up_b16"]
    K, N, M = wl.in_features, wl.out_features, wl.tokens
    base = W4.weight_bytes(N, K) + M * K * 2 + W4.act_bytes(M, K) + 2 * M * N * 4
    assert bench.w4a4_bytes(wl, False) == base
    assert bench.w4a4_bytes(wl, True) == base + W4.act_bytes(M, K)
