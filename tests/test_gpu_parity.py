"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

Whole tensors at sizes the oracle finishes in seconds (several tiles, ragged
tails, N_q != N_kv, every head dim, both masks, every dtype); sampled rows at
the full workload sizes in the launch configuration the benchmark times; and
properties that hold at any size.
"""
import dataclasses

import numpy as np
import pytest
import torch

from conftest import gpu_available
from exact_attention_95_amd import fa
from exact_attention_95_amd.inputs import WORKLOADS, make_inputs, random_problem
from parity import LSE_TOL, TOL, assert_within, full_parity, run_gpu, sampled_parity, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DT_CODE = {"f32": fa.FA_F32, "f16": fa.FA_F16, "bf16": fa.FA_BF16, "fp8_e4m3": fa.FA_FP8_E4M3}

# (B, H, N_q, N_kv, d, dtype, causal)
SMALL = [
    (1, 1, 256, 256, 64, "bf16", False),
    (1, 2, 300, 300, 64, "bf16", True),
    (2, 1, 257, 129, 64, "f16", False),
    (1, 1, 33, 500, 64, "f16", True),
    (1, 2, 512, 512, 128, "bf16", False),
    (2, 1, 450, 450, 128, "bf16", True),
    (1, 1, 200, 700, 128, "f16", True),
    (1, 1, 700, 200, 128, "f16", True),
    (1, 1, 1, 1, 128, "bf16", False),
    (1, 1, 5, 3, 64, "bf16", True),
    (1, 1, 300, 333, 256, "bf16", False),
    (1, 2, 260, 260, 256, "f16", True),
    (1, 1, 256, 256, 64, "f32", False),
    (2, 1, 130, 77, 64, "f32", True),
    (1, 1, 100, 300, 128, "f32", False),
    (1, 1, 97, 97, 256, "f32", True),
    (1, 2, 512, 512, 128, "fp8_e4m3", False),
    (2, 1, 333, 200, 128, "fp8_e4m3", True),
    (1, 1, 70, 900, 128, "fp8_e4m3", False),
]


@pytest.mark.parametrize("idx", range(len(SMALL)), ids=["x".join(str(v) for v in c) for c in SMALL])
def test_small_shapes_match_oracle(idx):
    case = SMALL[idx]
    B, H, nq, nkv, d, dt, causal = case
    w, x = random_problem(100 + idx, B, H, nq, nkv, d, dt, causal)
    say("case", case)
    err = full_parity(w, x=x)
    say(err)
    assert_within(w, err)


def test_single_head_f32_workload():
    """The 1x1x256x64 float32 workload, whole tensor."""
    w = WORKLOADS["single_head_f32_n256_d64"]
    err = full_parity(w)
    say(err)
    assert_within(w, err)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_every_variant_matches_oracle(dt, d, causal):
    n = fa.fa_num_variants(DT_CODE[dt], d, causal)
    assert n >= 1
    # tile counts: even with a ragged tail, odd, and a single tile
    for seed, nq, nkv in ((7, 333, 333), (17, 200, 300), (27, 40, 50)):
        w, x = random_problem(seed, 1, 2, nq, nkv, d, dt, causal)
        for v in range(1, n + 1):
            name = fa.fa_variant_name(DT_CODE[dt], d, causal, v)
            say("variant", name, nq, nkv)
            err = full_parity(w, tile=v, x=x)
            assert_within(w, err, name)


@pytest.mark.parametrize("causal", [False, True])
def test_every_fp8_variant_matches_oracle(causal):
    n = fa.fa_num_variants(fa.FA_FP8_E4M3, 128, causal)
    assert n >= 1
    w, x = random_problem(8, 1, 2, 333, 333, 128, "fp8_e4m3", causal)
    for v in range(1, n + 1):
        err = full_parity(w, tile=v, x=x)
        assert_within(w, err, fa.fa_variant_name(fa.FA_FP8_E4M3, 128, causal, v))


def test_fp8_negative_scale_and_descales():
    w, x = random_problem(9, 1, 2, 260, 300, 128, "fp8_e4m3", False, scale=-0.3)
    err = full_parity(w, x=x)
    say(err)
    assert_within(w, err)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_rows_of_p_sum_to_one(dt):
    """V = 1 everywhere gives O = 1 (each row of P sums to 1)."""
    w, x = random_problem(11, 2, 2, 300, 300, 128, dt, True)
    x["v"] = torch.ones_like(x["v"])
    o, _ = run_gpu(w, x)
    assert torch.allclose(o.float(), torch.ones_like(o, dtype=torch.float32), atol=TOL[dt][0] or 1e-2)


def test_causal_row_zero_is_v0_and_lse_is_s00():
    w, x = random_problem(12, 1, 3, 128, 128, 64, "bf16", True)
    o, lse = run_gpu(w, x)
    assert torch.equal(o[:, :, 0, :].cpu(), x["v"][:, :, 0, :])
    s00 = (x["q"][:, :, 0, :].double() * x["k"][:, :, 0, :].double()).sum(-1) * w.sm_scale
    assert (lse[:, :, 0].double().cpu() - s00).abs().max() <= LSE_TOL


def test_bitwise_repeatable():
    w, x = random_problem(13, 2, 4, 1000, 1000, 128, "bf16", False)
    o1, l1 = run_gpu(w, x)
    o2, l2 = run_gpu(w, x)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("scale", [0.0, -0.2, 2.0])
def test_zero_negative_and_large_scale(scale):
    w, x = random_problem(14, 1, 2, 200, 260, 64, "bf16", True, scale=scale)
    err = full_parity(w, x=x)
    say(scale, err)
    assert_within(w, err)


def test_huge_logits_stay_finite():
    """Scores near 1e4: the running max keeps every exponent <= 2^8."""
    w, x = random_problem(15, 1, 1, 128, 256, 128, "f16", False, scale=8.0)
    err = full_parity(w, x=x)
    say(err)
    assert_within(w, err)


def test_lse_optional_and_no_write_past_end():
    w, x = random_problem(16, 1, 2, 77, 90, 64, "bf16", False)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    guard = torch.full((2 * 77 * 64 + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = guard[:2 * 77 * 64].view(1, 2, 77, 64)
    fa.fwd(q, k, v, scale=w.sm_scale, out=out, with_lse=False)
    torch.cuda.synchronize()
    assert torch.all(guard[2 * 77 * 64:] == 7.0)
    o_ref, _ = run_gpu(w, x)
    assert torch.equal(out, o_ref)


def test_noop_shapes():
    q = torch.zeros(0, 2, 16, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = fa.fwd(q, q, q)
    assert o.shape == (0, 2, 16, 64)
    q = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 2, 5, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = fa.fwd(q, k, k)
    assert o.shape == (1, 2, 0, 64)


def test_validation_errors_reach_python():
    q = torch.zeros(1, 1, 8, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fwd(q, q, q)
    assert e.value.status == fa.FA_ERR_HEAD_DIM
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fwd(q, q, q, out=q)
    assert e.value.status == fa.FA_ERR_ALIAS


# ---- full workload sizes, sampled rows, default launch configuration ----

FULL = [
    ("gpt2_medium_bf16_n1024_d64", 256),
    ("long_f16_causal_n4096_d64", 256),
    ("long_f16_causal_n16384_d64", 256),
    ("long_f16_causal_n65536_d64", 256),
    ("headline_bf16_n8192_d128", 256),
    ("headline_bf16_causal_n8192_d128", 256),
    ("large_head_bf16_n16384_d256", 128),
    ("fp8_e4m3_n16384_d128", 256),
]


@pytest.mark.parametrize("name,br", FULL, ids=[f[0] for f in FULL])
def test_full_size_sampled_rows(name, br):
    w = WORKLOADS[name]
    say("workload", w)
    err = sampled_parity(w, br)
    say(err)
    assert_within(w, err, "sampled")
