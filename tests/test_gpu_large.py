"""Tensors past 4 GiB, at the library's largest sizes.

Every global offset in the kernels is formed in 64-bit arithmetic: per head
(b*H + h)*N*row_bytes, and within a head tile_start*row_bytes.  These tests
put the data that decides the result beyond the 2 GiB and 4 GiB byte offsets,
where a 32-bit offset would wrap.

- Keys past 4 GiB: one head with 2^24 + 37 keys (K and V 4 GiB each).  All
  keys are zero rows with V = 1/4, except five "special" keys at byte offsets
  768, 2 GiB + 1280, 4 GiB - 256, 4 GiB and the last row, whose large scores
  carry the softmax mass (each dominates some rows).  O and LSE then have an
  exact closed form (plain softmax attention evaluated in fp64 over the five
  specials plus n_zero equal keys).  The single-pass entry point refuses rows
  past 2^20 keys (FA_ERR_LONG_KV); split-KV must match both with scores of
  about 39 (zero keys below 1e-8 of the mass) and with scores of about 18
  (zero keys carrying 2-12 % spread over 2^24 keys).
- The same long-tail case at 2^20 keys, the single-pass limit: both entry
  points must match.  Nine heads of 2^20 keys at d = 256 put specials past
  the 4 GiB offset for the single-pass kernel.
- Queries past 4 GiB: two heads of 2^24 + 2^22 + 3 queries (Q and O 5 GiB
  each), with sampled rows around the 2 GiB and 4 GiB offsets checked against
  the fp64 oracle, with and without the causal mask; and the same with E4M3
  inputs at d = 128 (Q 5 GiB, O in bf16 10 GiB).
- Backward past 4 GiB: the same two heads (Q, O, dO and dQ 5 GiB each);
  dQ of sampled rows against the oracle's gradients, dK and dV finite.
"""
import math

import numpy as np
import pytest
import torch

from conftest import gpu_available
from exact_attention_95_amd import fa
import oracle
from parity import BWD_TOL, LSE_TOL, TOL, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

GIB = 1 << 30


def require_device_bytes(n: int):
    torch.cuda.empty_cache()  # blocks cached by earlier tests count as used
    free, _ = torch.cuda.mem_get_info()
    if free < n + 2 * GIB:
        pytest.skip("needs %.1f GiB of free device memory" % (n / GIB))


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str, label: str):
    o = o_gpu.float().cpu().double().numpy().reshape(o_ref.shape)
    lse = lse_gpu.float().cpu().double().numpy().reshape(lse_ref.shape)
    diff = o - o_ref
    err = {"max_abs": float(np.abs(diff).max()),
           "rel_l2": float(np.linalg.norm(diff) / np.linalg.norm(o_ref)),
           "lse_max_abs": float(np.abs(lse - lse_ref).max())}
    say(label, err)
    max_abs, rel = TOL[dtype]
    assert np.isfinite(o).all() and np.isfinite(lse).all(), label
    assert (max_abs is None or err["max_abs"] <= max_abs) and err["rel_l2"] <= rel, (label, err)
    assert err["lse_max_abs"] <= LSE_TOL, (label, err)


def sparse_keys_case(H: int, n_kv: int, d: int, specials, big: float, seed: int = 95, n_q: int = 33):
    """H heads of n_kv keys: zero rows with V = 1/4, except the `specials`
    ((head, row) pairs, at least one per head), whose first component is
    `big` (Q's first component is 1).  Returns the device tensors, the scale,
    and per head O, LSE and the zero keys' share of the softmax mass in
    closed form (fp64): plain softmax attention over the head's specials plus
    n_zero equal keys of score 0."""
    require_device_bytes(2 * H * n_kv * d * 2)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(H, n_q, d, generator=g)
    q[:, :, 0] = 1.0
    q = q.to(torch.bfloat16)
    ks = torch.randn(len(specials), d, generator=g)
    ks[:, 0] = big  # the random part of the score decides which special dominates a row
    ks = ks.to(torch.bfloat16)
    vs = torch.randn(len(specials), d, generator=g).to(torch.bfloat16)
    v_zero = 0.25
    k = torch.zeros(1, H, n_kv, d, dtype=torch.bfloat16, device="cuda")
    v = torch.full((1, H, n_kv, d), v_zero, dtype=torch.bfloat16, device="cuda")
    hs = torch.tensor([h for h, _ in specials], device="cuda")
    rs = torch.tensor([r for _, r in specials], device="cuda")
    k[0, hs, rs] = ks.cuda()
    v[0, hs, rs] = vs.cuda()

    o_ref = np.empty((H, n_q, d))
    lse_ref = np.empty((H, n_q))
    tail = np.empty((H, n_q))
    for h in range(H):
        sel = [i for i, (hh, _) in enumerate(specials) if hh == h]
        assert sel, "every head needs a special key"
        q64 = q[h].double().numpy()
        k64, v64 = ks[sel].double().numpy(), vs[sel].double().numpy()
        s = scale * (q64 @ k64.T)                                   # [n_q, specials of h]
        n_zero = n_kv - len(sel)
        m = np.maximum(s.max(axis=1), 0.0)
        w = np.exp(s - m[:, None])
        w0 = n_zero * np.exp(-m)
        ell = w0 + w.sum(axis=1)
        o_ref[h] = (w0[:, None] * v_zero + w @ v64) / ell[:, None]
        lse_ref[h] = m + np.log(ell)
        tail[h] = w0 / ell
        # each special matters: reading any one of them wrong (here: as a zero
        # row) moves O by far more than the tolerance
        for j in range(len(sel)):
            w_drop = w.copy()
            w_drop[:, j] = 0.0
            w0_drop = w0 + np.exp(-m)
            o_drop = (w0_drop[:, None] * v_zero + w_drop @ v64) / (w0_drop + w_drop.sum(axis=1))[:, None]
            assert np.abs(o_drop - o_ref[h]).max() > 0.5
    return q.cuda()[None], k, v, scale, o_ref, lse_ref, tail


def keys_past_4gib_case(big: float):
    """One head of 2^24 + 37 keys (K and V 4 GiB each); five special keys at
    byte offsets 768, 2 GiB + 1280, 4 GiB - 256, 4 GiB and the last row."""
    n_kv, d = (1 << 24) + 37, 128
    special = [3, (1 << 23) + 5, (1 << 24) - 1, 1 << 24, n_kv - 1]
    say("keys past 4 GiB: n_kv", n_kv, "special rows", special, "big", big)
    return sparse_keys_case(1, n_kv, d, [(0, r) for r in special], big)


def test_keys_past_4gib_closed_form():
    # scores about 39: the 2^24 zero-score keys carry under 1e-8 of the mass,
    # so the result depends on the five specials being read from the right
    # addresses, not on how the long tail is summed.  The single-pass entry
    # point refuses rows past 2^20 keys before any launch.
    q, k, v, scale, o_ref, lse_ref, tail = keys_past_4gib_case(440.0)
    assert tail.max() < 1e-8
    with pytest.raises(fa.FaError) as e:
        fa.fwd(q, k, v, scale=scale)
    assert e.value.status == fa.FA_ERR_LONG_KV
    o, lse = fa.fwd_splitkv(q, k, v, scale=scale)
    torch.cuda.synchronize()
    check(o, lse, o_ref, lse_ref, "bf16", "split-KV")
    o, lse = fa.fwd_splitkv(q, k, v, scale=scale, num_splits=1)  # still cut into <= 2^20-key chunks
    torch.cuda.synchronize()
    check(o, lse, o_ref, lse_ref, "bf16", "split-KV, num_splits=1")


def test_long_tail_over_2_24_keys_split_kv():
    # scores about 18: the zero-score keys carry 2-12 % of the mass, spread
    # over 2^24 keys.  One float32 running sum over all 2^18 key tiles of a
    # row would round away a fixed part of each small addend (here about 2
    # ulps of the sum), an error that grows with the number of tiles; the
    # single-pass entry point therefore refuses the case (FA_ERR_LONG_KV),
    # and split-KV sums chunks of at most 2^20 keys and merges them.
    q, k, v, scale, o_ref, lse_ref, tail = keys_past_4gib_case(200.0)
    assert tail.max() > 1e-2 and tail.min() < 0.5
    with pytest.raises(fa.FaError) as e:
        fa.fwd(q, k, v, scale=scale)
    assert e.value.status == fa.FA_ERR_LONG_KV
    o, lse = fa.fwd_splitkv(q, k, v, scale=scale)
    torch.cuda.synchronize()
    check(o, lse, o_ref, lse_ref, "bf16", "split-KV, long tail")


def test_long_tail_at_the_single_pass_limit():
    # the same worst case (identical small addends, a few % of the mass) at
    # the longest key range the single-pass entry point accepts: 2^20 keys
    n_kv, d = fa.FA_MAX_NKV_SINGLE_PASS, 128
    special = [0, 7, 1 << 19, n_kv - 2, n_kv - 1]
    q, k, v, scale, o_ref, lse_ref, tail = sparse_keys_case(1, n_kv, d, [(0, r) for r in special], 169.0)
    say("long tail at 2^20 keys: tail share %.3g .. %.3g" % (tail.min(), tail.max()))
    assert tail.max() > 1e-2 and tail.min() < 0.5
    o, lse = fa.fwd(q, k, v, scale=scale)
    torch.cuda.synchronize()
    check(o, lse, o_ref, lse_ref, "bf16", "single pass, long tail at the limit")
    o, lse = fa.fwd_splitkv(q, k, v, scale=scale)
    torch.cuda.synchronize()
    check(o, lse, o_ref, lse_ref, "bf16", "split-KV, long tail at the limit")


def test_single_pass_keys_past_4gib_across_heads():
    # nine heads of 2^20 keys at d = 256 (512-byte rows): K and V 4.5 GiB
    # each, head 8 starting at 4 GiB; specials in every head, several at byte
    # offsets past 2 and 4 GiB, scores about 39 (zero keys under 1e-8 of the mass)
    H, n_kv, d = 9, fa.FA_MAX_NKV_SINGLE_PASS, 256
    specials = [(h, r) for h in range(H) for r in ((h * 7919) % n_kv, n_kv - 1 - h)]
    specials += [(8, 3), (7, (1 << 19) + 1)]
    q, k, v, scale, o_ref, lse_ref, tail = sparse_keys_case(H, n_kv, d, specials, 620.0)
    assert tail.max() < 1e-8
    say("heads past 4 GiB: last special at byte offset %.2f GiB"
        % (max((h * n_kv + r) * d * 2 for h, r in specials) / GIB))
    o, lse = fa.fwd(q, k, v, scale=scale)
    torch.cuda.synchronize()
    check(o, lse, o_ref, lse_ref, "bf16", "single pass, heads past 4 GiB")


@pytest.mark.parametrize("causal", [False, True])
def test_queries_past_4gib_sampled_rows(causal):
    B, H, n_q, n_kv, d = 1, 2, (1 << 24) + (1 << 22) + 3, 100, 64
    require_device_bytes(2 * B * H * n_q * d * 2)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    gd = torch.Generator(device="cuda").manual_seed(7 + int(causal))
    q = torch.randn(B, H, n_q, d, generator=gd, device="cuda", dtype=torch.bfloat16)
    g = torch.Generator().manual_seed(11)
    k = torch.randn(B, H, n_kv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, H, n_kv, d, generator=g).to(torch.bfloat16)
    say("queries past 4 GiB: n_q", n_q, "causal", causal)
    o, lse = fa.fwd(q, k.cuda(), v.cuda(), scale=scale, causal=causal)
    torch.cuda.synchronize()

    rng = np.random.default_rng(3)
    fixed = [0, 1, n_kv - 2, n_kv - 1, n_kv, 1 << 23, (1 << 24) - 1, 1 << 24, n_q - 2, n_q - 1]
    for h in range(H):
        local = np.unique(np.concatenate([fixed, rng.integers(0, n_q, 20)]))
        o_rows = o[0, h, torch.from_numpy(local).cuda()]
        lse_rows = lse[0, h, torch.from_numpy(local).cuda()]
        # rows at or past n_kv - 1 see every key under either mask; earlier
        # causal rows are checked against the oracle on the head's first n_kv queries
        late = local >= n_kv - 1 if causal else np.ones(local.size, bool)
        o_ref = np.empty((local.size, d))
        lse_ref = np.empty(local.size)
        if late.any():
            qr = q[0, h, torch.from_numpy(local[late]).cuda()].cpu()
            o_ref[late], lse_ref[late] = oracle.attention(qr, k[0, h], v[0, h], scale, causal=False)
        if (~late).any():
            qh = q[0, h, :n_kv].cpu()
            o_ref[~late], lse_ref[~late] = oracle.attention(
                qh[None, None], k[0, h][None, None], v[0, h][None, None], scale, causal=True,
                rows=local[~late])
        say("head", h, "rows", local.size, "max byte offset of a checked row: %.2f GiB"
            % ((h * n_q + local.max()) * d * 2 / GIB))
        check(o_rows, lse_rows, o_ref, lse_ref, "bf16", "head %d causal %s" % (h, causal))


@pytest.mark.parametrize("causal", [False, True])
def test_e4m3_queries_past_4gib_sampled_rows(causal):
    B, H, n_q, n_kv, d = 1, 2, (1 << 24) + (1 << 22) + 3, 100, 128
    require_device_bytes(B * H * n_q * d * (2 + 1 + 2))  # bf16 draw, E4M3 codes, bf16 O
    scale = float(np.float32(1.0 / math.sqrt(d)))
    mul = 64.0  # N(0,1) * 64 stays inside E4M3's range (|x| <= 448) for these draws
    descale = 1.0 / mul
    gd = torch.Generator(device="cuda").manual_seed(21)
    q = torch.randn(B, H, n_q, d, generator=gd, device="cuda", dtype=torch.bfloat16)
    q = (q * mul).clamp_(-448, 448).to(torch.float8_e4m3fn)
    torch.cuda.empty_cache()
    g = torch.Generator().manual_seed(13)
    k = (torch.randn(B, H, n_kv, d, generator=g) * mul).clamp(-448, 448).to(torch.float8_e4m3fn)
    v = (torch.randn(B, H, n_kv, d, generator=g) * mul).clamp(-448, 448).to(torch.float8_e4m3fn)
    say("E4M3 queries past 4 GiB: n_q", n_q, "causal", causal)
    o, lse = fa.fwd(q, k.cuda(), v.cuda(), scale=scale, causal=causal, descale=(descale, descale, descale))
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    rng = np.random.default_rng(5)
    fixed = [0, 1, n_kv - 2, n_kv - 1, 1 << 23, (1 << 24) - 1, 1 << 24, n_q - 2, n_q - 1]
    for h in range(H):
        local = np.unique(np.concatenate([fixed, rng.integers(0, n_q, 20)]))
        sel = torch.from_numpy(local).cuda()
        kh, vh = oracle.dequant_e4m3(k[0, h], descale), oracle.dequant_e4m3(v[0, h], descale)
        # rows at or past n_kv - 1 see every key under either mask; earlier
        # causal rows against the oracle on the head's first n_kv queries
        late = local >= n_kv - 1 if causal else np.ones(local.size, bool)
        o_ref, lse_ref = np.empty((local.size, d)), np.empty(local.size)
        if late.any():
            q_rows = oracle.dequant_e4m3(q[0, h, torch.from_numpy(local[late]).cuda()].cpu(), descale)
            o_ref[late], lse_ref[late] = oracle.attention(q_rows, kh, vh, scale)
        if (~late).any():
            qh = oracle.dequant_e4m3(q[0, h, :n_kv].cpu(), descale)
            o_ref[~late], lse_ref[~late] = oracle.attention(qh[None, None], kh[None, None], vh[None, None],
                                                            scale, causal=True, rows=local[~late])
        say("head", h, "rows", local.size, "max byte offset of a checked O row: %.2f GiB"
            % ((h * n_q + local.max()) * d * 2 / GIB))
        check(o[0, h, sel], lse[0, h, sel], o_ref, lse_ref, "fp8_e4m3", "E4M3 head %d causal %s" % (h, causal))


def test_backward_queries_past_4gib_sampled_rows():
    B, H, n_q, n_kv, d = 1, 2, (1 << 24) + (1 << 22) + 3, 100, 64
    require_device_bytes(4 * B * H * n_q * d * 2)  # Q, O, dO, dQ
    scale = float(np.float32(1.0 / math.sqrt(d)))
    gd = torch.Generator(device="cuda").manual_seed(31)
    q = torch.randn(B, H, n_q, d, generator=gd, device="cuda", dtype=torch.bfloat16)
    do = torch.randn(B, H, n_q, d, generator=gd, device="cuda", dtype=torch.bfloat16)
    g = torch.Generator().manual_seed(17)
    k = torch.randn(B, H, n_kv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, H, n_kv, d, generator=g).to(torch.bfloat16)
    kd, vd = k.cuda(), v.cuda()
    say("backward past 4 GiB: n_q", n_q)
    o, lse = fa.fwd(q, kd, vd, scale=scale)
    dq, dk, dv = fa.bwd(q, kd, vd, o, lse, do, scale=scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(dk.float()).all()) and bool(torch.isfinite(dv.float()).all())
    rng = np.random.default_rng(9)
    fixed = [0, 1, 1 << 23, (1 << 24) - 1, 1 << 24, n_q - 2, n_q - 1]
    for h in range(H):
        local = np.unique(np.concatenate([fixed, rng.integers(0, n_q, 20)]))
        sel = torch.from_numpy(local).cuda()
        # rows are independent without the mask: the selected rows form a problem of their own
        q_rows, do_rows = q[0, h, sel].cpu(), do[0, h, sel].cpu()
        dq_ref, _, _ = oracle.backward(q_rows, k[0, h], v[0, h], do_rows, scale,
                                       rows=np.arange(local.size), keys=np.zeros(0, np.int64))
        got = dq[0, h, sel].float().cpu().double().numpy()
        err_max = float(np.abs(got - dq_ref).max() / np.abs(dq_ref).max())
        err_l2 = float(np.linalg.norm(got - dq_ref) / np.linalg.norm(dq_ref))
        say("head", h, "rows", local.size, "dQ max err / max |ref| %.2e, rel L2 %.2e, last row at %.2f GiB"
            % (err_max, err_l2, (h * n_q + local.max()) * d * 2 / GIB))
        assert np.isfinite(got).all()
        assert err_max <= BWD_TOL[0] and err_l2 <= BWD_TOL[1], (h, err_max, err_l2)
