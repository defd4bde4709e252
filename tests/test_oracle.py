"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: arbitrary-precision
brute force, the unshifted textbook softmax, scipy's logsumexp, closed forms,
invariants of the definition, and the equalities the pages state (blockwise
online softmax equals the full-row softmax up to rounding; results do not
depend on the block sizes).  A planted-mistake test checks that these pins
catch plausible slips in the oracle's C source.
"""
import math
import os
import re
import shutil
import subprocess
import tempfile

import mpmath
import numpy as np
import pytest
import scipy.special
import torch

import oracle

mpmath.mp.dps = 50


def _mp_attention(q, k, v, scale, causal):
    """50-digit brute force of O and LSE from the definition (P = softmax(scale*QK^T))."""
    n_q, d = q.shape
    n_kv = k.shape[0]
    o = np.zeros((n_q, d))
    lse = np.zeros(n_q)
    p = np.zeros((n_q, n_kv))
    sc = mpmath.mpf(scale)
    for i in range(n_q):
        vis = range(min(i + 1, n_kv)) if causal else range(n_kv)
        s = [sc * mpmath.fsum(mpmath.mpf(q[i, c]) * mpmath.mpf(k[j, c]) for c in range(d)) for j in vis]
        e = [mpmath.exp(x) for x in s]  # no max shift: plain definition
        z = mpmath.fsum(e)
        for jj, j in enumerate(vis):
            p[i, j] = float(e[jj] / z)
        for c in range(d):
            o[i, c] = float(mpmath.fsum(e[jj] * mpmath.mpf(v[j, c]) for jj, j in enumerate(vis)) / z)
        lse[i] = float(mpmath.log(z))
    return o, lse, p


def _rand(rng, *shape):
    # values with few significant bits keep the brute force exact on input
    return np.round(rng.standard_normal(shape) * 64) / 64


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", range(6))
def test_brute_force_mpmath(seed, causal):
    rng = np.random.default_rng([77, seed, causal])
    n_q, n_kv, d = int(rng.integers(1, 9)), int(rng.integers(1, 9)), int(rng.integers(1, 5))
    q, k, v = _rand(rng, n_q, d), _rand(rng, n_kv, d), _rand(rng, n_kv, d)
    scale = float(rng.uniform(0.1, 2.0))
    o, lse, p = oracle.attention(q, k, v, scale, causal, return_p=True)
    o_ref, lse_ref, p_ref = _mp_attention(q, k, v, scale, causal)
    assert np.abs(o - o_ref).max() <= 1e-13
    assert np.abs(lse - lse_ref).max() <= 1e-13
    assert np.abs(p - p_ref).max() <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_blockwise_brute_force_mpmath(causal):
    rng = np.random.default_rng([78, causal])
    q, k, v = _rand(rng, 7, 3), _rand(rng, 9, 3), _rand(rng, 9, 3)
    o_ref, lse_ref, _ = _mp_attention(q, k, v, 0.7, causal)
    for order in ("v1", "v2"):
        o, lse = oracle.attention_blockwise(q, k, v, 0.7, causal, br=3, bc=2, order=order)
        assert np.abs(o - o_ref).max() <= 1e-13
        assert np.abs(lse - lse_ref).max() <= 1e-13


def test_textbook_unshifted_softmax_and_logsumexp():
    rng = np.random.default_rng(5)
    n_q, n_kv, d = 13, 29, 16
    q, k, v = rng.standard_normal((n_q, d)), rng.standard_normal((n_kv, d)), rng.standard_normal((n_kv, d))
    scale = 0.25
    o, lse, p = oracle.attention(q, k, v, scale, return_p=True)
    s = scale * (q @ k.T)  # library matmul, |s| < 30 so no shift is needed
    assert np.abs(s).max() < 30
    e = np.exp(s)
    p_ref = e / e.sum(axis=1, keepdims=True)
    assert np.abs(p - p_ref).max() <= 1e-14
    assert np.abs(o - p_ref @ v).max() <= 1e-13
    assert np.abs(lse - scipy.special.logsumexp(s, axis=1)).max() <= 1e-13


def test_rows_of_p_sum_to_one_and_causal_zeros():
    rng = np.random.default_rng(6)
    q, k, v = rng.standard_normal((40, 8)) * 3, rng.standard_normal((50, 8)) * 3, rng.standard_normal((50, 8))
    for causal in (False, True):
        _, _, p = oracle.attention(q, k, v, 0.5, causal, return_p=True)
        assert np.abs(p.sum(axis=1) - 1).max() <= 1e-14 * 50
        assert (p >= 0).all()
        if causal:
            assert np.all(np.triu(p, 1)[:, :50] == 0)


def test_closed_forms():
    rng = np.random.default_rng(7)
    d = 6
    q, k, v = rng.standard_normal((5, d)), rng.standard_normal((1, d)), rng.standard_normal((1, d))
    # one key: O = V_0, LSE = s_00
    o, lse = oracle.attention(q, k, v, 0.3)
    assert np.abs(o - v[0]).max() <= 1e-15
    assert np.abs(lse - 0.3 * (q @ k[0])).max() <= 1e-14
    # two keys: weights are logistic sigmoids of the score difference
    k2, v2 = rng.standard_normal((2, d)), rng.standard_normal((2, d))
    o, lse = oracle.attention(q, k2, v2, 0.7)
    s = 0.7 * (q @ k2.T)
    w0 = 1 / (1 + np.exp(s[:, 1] - s[:, 0]))
    assert np.abs(o - (w0[:, None] * v2[0] + (1 - w0)[:, None] * v2[1])).max() <= 1e-14
    # Q = 0 (or scale = 0): O = mean of V, LSE = ln N_kv
    kk, vv = rng.standard_normal((11, d)), rng.standard_normal((11, d))
    for qq, sc in ((np.zeros((3, d)), 1.0), (rng.standard_normal((3, d)), 0.0)):
        o, lse = oracle.attention(qq, kk, vv, sc)
        assert np.abs(o - vv.mean(axis=0)).max() <= 1e-14
        assert np.abs(lse - math.log(11)).max() <= 1e-14
    # equal key rows: uniform weights
    ke = np.repeat(rng.standard_normal((1, d)), 11, axis=0)
    o, _ = oracle.attention(rng.standard_normal((3, d)), ke, vv, 0.9)
    assert np.abs(o - vv.mean(axis=0)).max() <= 1e-14
    # V constant -> O constant; V + c -> O + c
    qq = rng.standard_normal((4, d))
    o, _ = oracle.attention(qq, kk, np.full((11, d), 2.5), 0.4)
    assert np.abs(o - 2.5).max() <= 1e-14
    o1, _ = oracle.attention(qq, kk, vv, 0.4)
    o2, _ = oracle.attention(qq, kk, vv + 3.0, 0.4)
    assert np.abs(o2 - o1 - 3.0).max() <= 1e-14
    # causal row 0 sees only key 0
    o, lse = oracle.attention(qq, kk, vv, 0.4, causal=True)
    assert np.abs(o[0] - vv[0]).max() <= 1e-15
    assert abs(lse[0] - 0.4 * qq[0] @ kk[0]) <= 1e-14


def test_causal_equals_truncated_keys():
    rng = np.random.default_rng(8)
    for n_q, n_kv in ((9, 9), (6, 10), (12, 5)):
        q, k, v = rng.standard_normal((n_q, 4)), rng.standard_normal((n_kv, 4)), rng.standard_normal((n_kv, 4))
        o, lse = oracle.attention(q, k, v, 0.6, causal=True)
        for i in range(n_q):
            nv = min(i + 1, n_kv)
            oi, li = oracle.attention(q[i:i + 1], k[:nv], v[:nv], 0.6)
            assert np.abs(o[i] - oi[0]).max() <= 1e-15
            assert abs(lse[i] - li[0]) <= 1e-15


def test_key_permutation_invariance_and_huge_logits():
    rng = np.random.default_rng(9)
    q, k, v = rng.standard_normal((8, 5)), rng.standard_normal((21, 5)), rng.standard_normal((21, 5))
    perm = rng.permutation(21)
    o1, l1 = oracle.attention(q, k, v, 1.1)
    o2, l2 = oracle.attention(q, k[perm], v[perm], 1.1)
    assert np.abs(o1 - o2).max() <= 1e-14 and np.abs(l1 - l2).max() <= 1e-13
    # logits near 1e4 stay finite and match the shifted-by-constant problem
    o3, l3 = oracle.attention(q * 2000, k, v, 1.1)
    assert np.isfinite(o3).all() and np.isfinite(l3).all()


@pytest.mark.parametrize("causal", [False, True])
def test_blockwise_equals_naive_random_partitions(causal):
    rng = np.random.default_rng([10, causal])
    n_q, n_kv, d = 70, 150, 16
    q = rng.standard_normal((n_q, d)) * 2
    k, v = rng.standard_normal((n_kv, d)), rng.standard_normal((n_kv, d))
    o_ref, l_ref = oracle.attention(q, k, v, 0.25, causal)
    worst = 0.0
    for _ in range(60):
        ncut = int(rng.integers(0, 20))
        kv_cuts = np.unique(np.concatenate([[0, n_kv], rng.integers(1, n_kv, ncut)]))
        q_cuts = np.unique(np.concatenate([[0, n_q], rng.integers(1, n_q, 5)]))
        for order in ("v2", "v1"):
            o, l = oracle.attention_blockwise(q, k, v, 0.25, causal, q_cuts=q_cuts, kv_cuts=kv_cuts, order=order)
            worst = max(worst, np.abs(o - o_ref).max(), np.abs(l - l_ref).max())
    assert worst <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_block_size_invariance(causal):
    rng = np.random.default_rng([11, causal])
    n, d = 256, 64
    q, k, v = (rng.standard_normal((n, d)).astype(np.float32) for _ in range(3))
    o_ref, l_ref = oracle.attention(q, k, v, 0.125, causal)
    for bc in (1, 2, 7, 32, 64, 128, n):
        o, l = oracle.attention_blockwise(q, k, v, 0.125, causal, br=64, bc=bc)
        assert np.abs(o - o_ref).max() <= 1e-12 and np.abs(l - l_ref).max() <= 1e-12
    for br, bc in ((16, 16), (32, 32), (64, 128), (128, 64), (37, 53), (n, n)):
        for order in ("v2", "v1"):
            o, l = oracle.attention_blockwise(q, k, v, 0.125, causal, br=br, bc=bc, order=order)
            assert np.abs(o - o_ref).max() <= 1e-12 and np.abs(l - l_ref).max() <= 1e-12


def test_eight_scores_two_at_a_time():
    """Plate 08's example shape: one row of 8 scores merged 2 at a time equals
    the direct result to ~1e-15 (the page's own score values are not printed,
    so only this property is used)."""
    rng = np.random.default_rng(12)
    for _ in range(20):
        scores = rng.uniform(-4, 4, 8)
        q = np.zeros((1, 8)); q[0, 0] = 1.0
        k = np.zeros((8, 8)); k[:, 0] = scores
        v = np.eye(8)                     # O is then the probability row itself
        o_dir, l_dir = oracle.attention(q, k, v, 1.0)
        o_on, l_on = oracle.attention_blockwise(q, k, v, 1.0, kv_cuts=[0, 2, 4, 6, 8])
        assert np.abs(o_on - o_dir).max() < 1e-15 * 4
        assert abs(l_on[0] - l_dir[0]) < 1e-15 * 8
        assert abs(l_dir[0] - (scores.max() + math.log(np.exp(scores - scores.max()).sum()))) < 1e-14


def test_row_subset_matches_full():
    rng = np.random.default_rng(13)
    q, k, v = (rng.standard_normal((2, 3, 33, 8)) for _ in range(3))
    o, l = oracle.attention(q, k, v, 0.35, True)
    rows = np.array([0, 32, 33, 99, 150, 197])
    o2, l2 = oracle.attention(q, k, v, 0.35, True, rows=rows)
    assert np.array_equal(o2, o.reshape(-1, 8)[rows]) and np.array_equal(l2, l.reshape(-1)[rows])


def test_e4m3_decoder_against_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_to_double(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.nanmax(got) == 448.0 and np.nanmin(got) == -448.0
    assert oracle.e4m3_to_double(0x01) == 2.0 ** -9       # smallest subnormal
    d = float(np.float32(1 / 300.0))
    deq = oracle.dequant_e4m3(codes[:127].numpy(), d)
    assert np.array_equal(deq, ref[:127] * d)


def test_merge_of_key_chunks_equals_full_row():
    """Attention over each chunk of a key partition, merged, equals attention
    over all keys (Flash-Decoding's split and merge)."""
    rng = np.random.default_rng(14)
    n_q, n_kv, d = 9, 300, 16
    q = rng.standard_normal((n_q, d)) * 2
    k, v = rng.standard_normal((n_kv, d)), rng.standard_normal((n_kv, d))
    o_ref, l_ref = oracle.attention(q, k, v, 0.4)
    for _ in range(20):
        cuts = np.unique(np.concatenate([[0, n_kv], rng.integers(1, n_kv, int(rng.integers(0, 12)))]))
        parts = [oracle.attention(q, k[a:b], v[a:b], 0.4) for a, b in zip(cuts[:-1], cuts[1:])]
        o, l = oracle.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        assert np.abs(o - o_ref).max() <= 1e-12 and np.abs(l - l_ref).max() <= 1e-12


def test_merge_ignores_empty_chunks_and_single_chunk_is_identity():
    rng = np.random.default_rng(15)
    o1, l1 = rng.standard_normal((1, 4, 8)), rng.standard_normal((1, 4))
    o, l = oracle.merge(o1, l1)
    assert np.array_equal(o, o1[0]) and np.abs(l - l1[0]).max() <= 1e-15
    o2 = np.concatenate([o1, rng.standard_normal((1, 4, 8))])
    l2 = np.concatenate([l1, np.full((1, 4), -np.inf)])
    o, l = oracle.merge(o2, l2)
    assert np.array_equal(o, o1[0]) and np.abs(l - l1[0]).max() <= 1e-15
    # two equal chunks: same output, LSE + ln 2
    o, l = oracle.merge(np.concatenate([o1, o1]), np.concatenate([l1, l1]))
    assert np.abs(o - o1[0]).max() <= 1e-15 and np.abs(l - l1[0] - math.log(2)).max() <= 1e-14


# ---- planted mistakes: each variant of the C source must fail a pin ----

MUTATIONS = [
    ("exp shift sign", "l += exp(s[j] - m);", "l += exp(s[j] + m);"),
    ("dropped scale", "return scale * acc;", "return acc;"),
    ("key row index", "s[j] = score(qi, k + j * d, d, scale);\n                if (s[j] > m) m = s[j];",
     "s[j] = score(qi, k + j, d, scale);\n                if (s[j] > m) m = s[j];"),
    ("causal off by one", "return (i + 1 < n_kv) ? i + 1 : n_kv;", "return (i < n_kv) ? i : n_kv;"),
    ("lse dropped max", "lse[r] = m + log(l);", "lse[r] = log(l);"),
    ("wrong operand in PV", "const double *vj = v + j * d;\n                for (int64_t c = 0; c < d; ++c) oi[c]",
     "const double *vj = k + j * d;\n                for (int64_t c = 0; c < d; ++c) oi[c]"),
    ("missing l rescale", "l = alpha * l + beta * lt;", "l = l + beta * lt;"),
    ("missing O rescale", "acc[c] = alpha * acc[c] + beta * pv[c];", "acc[c] = acc[c] + beta * pv[c];"),
    ("v1 stale weight", "double old_w = (mi == -INFINITY) ? 0.0 : li * exp(mi - m_new);",
     "double old_w = (mi == -INFINITY) ? 0.0 : exp(mi - m_new);"),
    ("e4m3 bias", "else mag = ldexp(1.0 + mant / 8.0, e - 7);", "else mag = ldexp(1.0 + mant / 8.0, e - 8);"),
    ("merge lse without max", "lse[r] = m + log(den);", "lse[r] = log(den);"),
    ("merge unnormalised", "o[r * d + c] /= den;", "o[r * d + c] /= 1.0;"),
]


def _pins_pass(lib) -> bool:
    """A compact subset of the pins above, run against a given library."""
    rng = np.random.default_rng(99)
    try:
        for causal in (False, True):
            q, k, v = _rand(rng, 5, 3), _rand(rng, 7, 3), _rand(rng, 7, 3)
            o_ref, l_ref, _ = _mp_attention(q, k, v, 0.8, causal)
            o, l = oracle.attention(q, k, v, 0.8, causal, lib=lib)
            if np.abs(o - o_ref).max() > 1e-13 or np.abs(l - l_ref).max() > 1e-13:
                return False
            for order in ("v1", "v2"):
                o, l = oracle.attention_blockwise(q, k, v, 0.8, causal, br=2, bc=3, order=order, lib=lib)
                if np.abs(o - o_ref).max() > 1e-13 or np.abs(l - l_ref).max() > 1e-13:
                    return False
        ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
        got = np.array([oracle.e4m3_to_double(c, lib=lib) for c in range(256)])
        ok = ~np.isnan(ref)
        if not np.array_equal(ref[ok], got[ok]):
            return False
        q, k, v = _rand(rng, 4, 3), _rand(rng, 9, 3), _rand(rng, 9, 3)
        o_ref, l_ref, _ = _mp_attention(q, k, v, 0.8, False)
        parts = [oracle.attention(q, k[a:b], v[a:b], 0.8, lib=lib) for a, b in ((0, 4), (4, 9))]
        o, l = oracle.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]), lib=lib)
        return bool(np.abs(o - o_ref).max() <= 1e-13 and np.abs(l - l_ref).max() <= 1e-13)
    except RuntimeError:
        return False


def test_pins_accept_the_oracle():
    assert _pins_pass(oracle.load())


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, name
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(force=True, src=str(mutated), out=str(tmp_path / "libmut.so")))
    assert not _pins_pass(lib), "pins did not catch: " + name
