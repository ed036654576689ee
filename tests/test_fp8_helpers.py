"""The pack kernels' FP8 E4M3FN and BF16 helpers (csrc/rq_fp8.hpp), compiled for the host
and checked against the oracle's format definitions: every finite byte's value, the floor
and ceiling bytes of values across the whole E4M3 range (grid points, midpoints, the
subnormal range, signed zeros), the saturation outside it, and BF16 round-half-even."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import formats as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("fp8") / "chk")
    r = subprocess.run([HIPCC, "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I",
                        os.path.join(ROOT, "looped_transformer_decode_amd", "csrc"),
                        os.path.join(ROOT, "tests", "fp8_host_check.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr

    def run(values):
        v = np.asarray(values, dtype=np.float64)
        inp = "\n".join(f"{int(b):016x}" for b in v.view(np.uint64)) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.splitlines()
        rows = [l.split() for l in out if not l.startswith("byte")]
        table = {int(l.split()[1], 16): np.array([int(l.split()[2], 16)], np.uint64).view(np.float64)[0]
                 for l in out if l.startswith("byte")}
        fl = np.array([int(r[0], 16) for r in rows])
        dn = np.array([int(r[1], 16) for r in rows])
        up = np.array([int(r[2], 16) for r in rows])
        bf = np.array([int(r[3], 16) for r in rows], np.uint64).view(np.float64)
        return fl, dn, up, bf, table
    return run


def _probe_values():
    g = F.E4M3_GRID
    mids = (g[1:] + g[:-1]) / 2
    rng = np.random.default_rng(50)
    rand = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-2 ** -5, 2 ** -5, 2000),
                           np.exp(rng.uniform(np.log(2 ** -12), np.log(448), 2000))])
    return np.concatenate([g, mids, np.nextafter(g, np.inf), np.nextafter(g, -np.inf), rand, [0.0, -0.0]])


def test_byte_values_match_the_format(checker):
    *_, table = checker([1.0])
    assert len(table) == 254
    for b, v in table.items():
        assert v == F.E4M3_TABLE[b], hex(b)


def test_floor_and_ceiling_bytes_inside_the_range(checker):
    v = _probe_values()
    v = v[(v >= -448) & (v <= 448)]
    fl, dn, up, _, _ = checker(v)
    assert not np.any((fl & 0x7F) == 0x7F)
    assert np.array_equal(F.e4m3_decode(fl), F.e4m3_floor(v))
    a = np.abs(v)
    assert np.array_equal(F.e4m3_decode(dn), F.e4m3_floor(a))
    assert np.array_equal(F.e4m3_decode(up), F.e4m3_ceil(a))


def test_outside_the_range_saturates_at_448(checker):
    v = np.array([-448.5, -450.0, -480.0, -500.0, -512.0, -1e4, 449.0, 1e6])
    fl, dn, up, _, _ = checker(v)
    assert list(fl[:6]) == [0xFE] * 6                   # offset -448: finite, never a NaN byte
    assert F.e4m3_decode(fl[:6]).tolist() == [-448.0] * 6
    assert list(dn[6:]) == [0x7E, 0x7E] and list(up[6:]) == [0x7E, 0x7E]


def test_bf16_rounding_matches_the_oracle(checker):
    rng = np.random.default_rng(51)
    v = np.concatenate([rng.normal(0, 1, 3000), rng.normal(0, 1e-3, 500), rng.uniform(0.5, 2.0, 500)])
    # exact ties: BF16 values plus half their ulp, both parities of the last kept bit
    base = F.bf16_round(rng.uniform(0.5, 4.0, 200))
    ulp = 2.0 ** (np.floor(np.log2(np.abs(base))) - 7)
    v = np.concatenate([v, base + ulp / 2, -(base + ulp / 2), [0.0]])
    _, _, _, bf, _ = checker(v)
    assert np.array_equal(bf, F.bf16_round(v))
