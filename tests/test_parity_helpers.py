"""Host-side checks of the parity helpers the GPU tests use (no GPU needed):
the full-size row sampler and the streamed whole-tensor comparison."""
import numpy as np
import torch

import oracle
from exact_attention_95_amd.inputs import WORKLOADS, random_problem
from parity import default_rows, errors, sample_rows, streamed_parity


def test_sampler_covers_block_boundaries_over_the_whole_head():
    w = WORKLOADS["long_f16_causal_n65536_d64"]
    x = {"boost_rows": np.zeros(0, np.int64)}
    local = sample_rows(w, x, 128) % w.n_q
    firsts = local[(local % 128 == 0) & (local > 0)]
    lasts = local[local % 128 == 127]
    assert firsts.size >= 100 and lasts.size >= 100
    assert firsts.max() > 0.9 * w.n_q and lasts.max() > 0.9 * w.n_q
    assert firsts.min() < 0.1 * w.n_q
    assert 0 in local and w.n_q - 1 in local


def test_sampler_keeps_every_boundary_when_few():
    w = WORKLOADS["gpt2_medium_bf16_n1024_d64"]
    x = {"boost_rows": np.array([5, 77], np.int64)}
    rows = sample_rows(w, x, 128)
    local = rows % w.n_q
    for e in range(128, 1024, 128):
        assert e in local and e - 1 in local
    assert 5 in rows and 77 in rows


def test_default_rows_follow_the_variant_table():
    assert default_rows(WORKLOADS["headline_bf16_n8192_d128"]) == 256
    assert default_rows(WORKLOADS["gpt2_medium_bf16_n1024_d64"]) == 128
    assert default_rows(WORKLOADS["large_head_bf16_n16384_d256"]) == 128


def test_streamed_comparison_equals_whole_tensor_errors():
    """The per-head streamed errors equal the errors computed on the whole
    tensor at once, for an output that differs from the oracle's."""
    w, x = random_problem(40, 2, 3, 50, 70, 64, "bf16", True)
    o_ref, lse_ref = oracle.attention(x["q"], x["k"], x["v"], w.sm_scale, w.causal)
    rng = np.random.default_rng(1)
    o_bad = o_ref + 1e-3 * rng.standard_normal(o_ref.shape)
    lse_bad = lse_ref + 1e-4 * rng.standard_normal(lse_ref.shape)
    want = errors(o_bad, lse_bad, o_ref, lse_ref)
    got = streamed_parity(w, x, torch.from_numpy(o_bad), torch.from_numpy(lse_bad))
    for key in ("max_abs", "rel_l2", "lse_max_abs"):
        assert abs(got[key] - want[key]) <= 1e-12 * max(1.0, want[key]), key
    assert got["heads"] == 6 and got["finite"]
