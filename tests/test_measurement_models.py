"""The FLOP and HBM-byte models that bench.py reports reproduce the worked
numbers the pages print (tests/golden/pages_worked_numbers.json):

- "FlashAttention 与显存", plate 04: one head of N = 4096, d = 128 in 16-bit
  has a 33.6 MB score matrix, 32 times Q; writing and reading S and P once
  each moves 134 MB, about 40 us at 3.35 TB/s; the two products take about
  8.7 us at 989 TFLOP/s.
- Same page, plate 03: the H100 ridge is about 295 flop/B and standard
  attention at d = 128 does about 62 flop/B.
- "FlashAttention算子优化", section 3: the tiled forward in FP32 with K and V
  read once reaches about 500 flop/B at sequence length 2048.

Plate 14's no-cache model (every query block reads all of K and V) is checked
against its definition and against the cached model at one query block.
CPU only.
"""
import json
import os

import pytest

import bench
from exact_attention_95_amd.inputs import Workload

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pages_worked_numbers.json")
DT = {1: "fp8_e4m3", 2: "bf16", 4: "f32"}


def entries():
    with open(GOLDEN) as f:
        return json.load(f)["entries"]


def head(n, d, e, causal=False):
    return Workload("golden", 0, 1, 1, n, n, d, DT[e], causal)


def test_plate_04_standard_method_one_head():
    g = entries()[0]
    w = head(g["N"], g["d"], g["element_bytes"])
    s_bytes = g["N"] * g["N"] * g["element_bytes"]
    assert round(s_bytes / 1e6, 1) == g["S_megabytes"]
    assert s_bytes // (g["N"] * g["d"] * g["element_bytes"]) == g["S_over_Q"]
    qkvo = 4 * g["N"] * g["d"] * g["element_bytes"]
    sp = bench.materialised_bytes(w) - qkvo
    assert round(sp / 1e6) == g["S_and_P_written_and_read_megabytes"]
    assert round(sp / (g["hbm_terabytes_per_s"] * 1e12) * 1e6) == g["S_and_P_round_trip_microseconds_about"]
    us = w.flops / (g["matmul_peak_teraflops"] * 1e12) * 1e6
    assert round(us, 1) == g["two_matmuls_microseconds_about"]


def test_plate_03_ridge_and_standard_intensity():
    g = entries()[1]
    assert round(g["peak_teraflops"] / g["hbm_terabytes_per_s"]) == g["ridge_flop_per_byte_about"]
    s = g["standard_attention"]
    w = head(s["N"], s["d"], s["element_bytes"])
    assert round(w.flops / bench.materialised_bytes(w)) == s["flop_per_byte_about"]


@pytest.mark.parametrize("d", [64, 128])
def test_section_3_tiled_fp32_intensity(d):
    g = entries()[2]
    w = head(g["N"], d, g["element_bytes"])
    # Q, K, V read once and O (and the per-row LSE) written once; the page
    # says "about 500" for N / 4 = 512 flop/B before the LSE term
    x = w.flops / bench.algorithmic_bytes(w)
    assert abs(x - g["flop_per_byte_about"]) / g["flop_per_byte_about"] < 0.05
    assert w.flops / (bench.algorithmic_bytes(w) - 4 * g["N"]) == g["N"] / 4


def test_plate_14_model_without_cache():
    w = Workload("t", 0, 2, 3, 1000, 700, 64, "bf16")
    e = 2
    for br in (64, 128, 256, 1000, 4096):
        passes = -(-1000 // br)
        want = 2 * 3 * e * (2 * 1000 * 64 + passes * 2 * 700 * 64)
        assert bench.fa_bytes_without_l2(w, br) == want
    # one query block: every tensor moves once, as in the cached model (without the LSE)
    assert bench.fa_bytes_without_l2(w, 1000) == bench.algorithmic_bytes(w) - 2 * 3 * 1000 * 4
    # doubling N: the standard method's bytes grow about 4x, the tiled method's
    # (fixed block) too, its cached bytes 2x (plate 14's question)
    a, b = head(4096, 128, 2), head(8192, 128, 2)
    assert 3.9 < bench.materialised_bytes(b) / bench.materialised_bytes(a) < 4.0
    assert bench.fa_bytes_without_l2(b, 128) / bench.fa_bytes_without_l2(a, 128) == pytest.approx(4, rel=0.02)
    assert bench.algorithmic_bytes(b) / bench.algorithmic_bytes(a) == 2


def test_variant_rows():
    assert bench.variant_rows("br8x32_bc64") == 256
    assert bench.variant_rows("split_br4x32_bc64") == 128
    with pytest.raises(ValueError):
        bench.variant_rows("bc64")
