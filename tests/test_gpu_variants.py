"""GPU parity of the precision, group-length and scale-rule settings on the same kernels:
uniform INT4 (4-bit anchors and 4-bit residuals), the mixed INT2/4 at g = 16, loop groups
of 8 and 16, the norm-ratio coefficient (shared and chained), the grouped-query kernel
with two query heads per KV head, the chained layout with two and four query heads per KV
head (one workgroup per query head) and with two anchor groups, and residual widths per loop (4 bits far from the
anchor, 2 bits near it; with grouped queries the 2-bit loops run on the grouped kernel and
the 4-bit ones on the one-query kernel).  Each case packs a
ragged context (the many-token kernel), decodes every loop (or a spread of loops for the
16-loop group) at several split counts against the oracle, and checks the drained token
of every group whose loops all ran (the one-loop-per-workgroup kernel)."""
import pytest

from looped_transformer_decode_amd import synth

from _support import run_decode_step_parity, run_pack_parity, setup_case

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
U = "uniform(0.8,1.0)"
CASES = {
    # name: (workload, chained, batch, ctx_len per row, n_kv_heads, n_q_heads, loops or None)
    "int4_uniform_d128g32": (W["ouro_b4_t8192"].with_(resid_bits=4), False, 3, [0, 70, 200], 2, 2, None),
    "int4_uniform_d64g16_bf16q": (W["tiny_d64_t256"].with_(group=16, resid_bits=4, q_dtype="bf16"), False, 2,
                                  [129, 63], 2, 2, None),
    "int4_uniform_gqa4": (W["huginn_gqa4_b8_t8192"].with_(resid_bits=4, n_groups=1), False, 2, [150, 90], 2, 8,
                          None),
    "int2_4_g16_d128": (W["ouro_b4_t8192"].with_(group=16), False, 2, [65, 190], 2, 2, None),
    "loops8_d128": (W["ouro_b4_t8192"].with_(loops_per_group=8, loop_scale=U), False, 2, [100, 33], 2, 2, None),
    "loops16_d64": (W["tiny_d64_t256"].with_(loops_per_group=16, loop_scale=U), False, 2, [90, 140], 2, 2,
                    None),
    "gqa2_ragged": (W["huginn_gqa4_b8_t8192"].with_(n_groups=2), False, 3, [130, 0, 64], 2, 4, None),
    "loops16_two_groups_gqa2": (W["ouro_b4_t8192"].with_(loops_per_group=16, n_groups=2, loop_scale=U), False, 1,
                                [80], 2, 4, [0, 7, 14, 15, 16, 30, 31]),
    "norm_ratio_d128g32": (W["ouro_b4_t8192"].with_(scale_rule=1), False, 3, [64, 1, 150], 2, 2, None),
    "norm_ratio_chained_int2g16": (W["int2g16_b4_t16384"].with_(scale_rule=1), True, 2, [65, 130], 2, 2, None),
    # chained with grouped queries (the one-query kernel once per query head) and two anchor groups
    "chained_gqa2_two_groups_d128g32": (W["ouro_b4_t8192"].with_(n_groups=2, loop_scale=U), True, 2, [130, 77], 2, 4,
                                        None),
    "chained_gqa4_int2g16": (W["int2g16_b4_t16384"], True, 2, [100, 190], 2, 8, None),
    "norm_ratio_int4_uniform_d64": (W["tiny_d64_t256"].with_(scale_rule=1, resid_bits=4), False, 1, [200], 2, 2,
                                    None),
    "widths_422_d128g32": (W["ouro_b4_t8192"].with_(resid_bits_loop=(4, 2, 2)), False, 3, [0, 70, 200], 2, 2, None),
    "widths_442_d64g16_bf16q": (W["tiny_d64_t256"].with_(group=16, resid_bits_loop=(4, 4, 2), q_dtype="bf16"), False,
                                2, [129, 63], 2, 2, None),
    "widths_loops8_gqa4": (W["huginn_gqa4_b8_t8192"].with_(loops_per_group=8, n_groups=2, loop_scale=U,
                                                            resid_bits_loop=(4, 4, 4, 2, 2, 2, 2)), False, 2,
                           [150, 90], 2, 8, None),
    "widths_norm_ratio_d128g16": (W["int2g16_b4_t16384"].with_(anchor_bits=4, scale_rule=1, resid_bits_loop=(4, 2, 2)),
                                  False, 2, [65, 130], 2, 2, None),
}


@pytest.fixture(scope="module")
def B():
    from looped_transformer_decode_amd import binding
    return binding


@pytest.mark.parametrize("name", sorted(CASES))
def test_variant_pack_parity(B, name):
    wl, chained, batch, ctx, hkv, hq, _ = CASES[name]
    wl, inp, cfg, ocfg, ctx, T = setup_case(B, wl, chained, batch, ctx, hkv, hq, seed=4321)
    run_pack_parity(B, name, wl, inp, cfg, ocfg, T)


@pytest.mark.parametrize("name", sorted(CASES))
def test_variant_decode_step_parity(B, name):
    wl, chained, batch, ctx, hkv, hq, loops = CASES[name]
    wl, inp, cfg, ocfg, ctx, T = setup_case(B, wl, chained, batch, ctx, hkv, hq, seed=77)
    run_decode_step_parity(B, name, wl, inp, cfg, ocfg, ctx, T, loops=loops)
