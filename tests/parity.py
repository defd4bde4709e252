"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and measure the disagreement."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
from exact_attention_95_amd import fa
from exact_attention_95_amd.inputs import Workload, make_inputs

# Tolerances on O (max abs, relative L2 over the whole tensor) and on LSE (max abs).
TOL = {"f32": (1e-5, 1e-6), "f16": (2e-2, 5e-3), "bf16": (2e-2, 5e-3), "fp8_e4m3": (None, 5e-2)}
LSE_TOL = 1e-3
# Tolerances on each backward gradient (max abs error / max |reference|, relative L2
# over the whole tensor or all sampled rows), 16-bit inputs.  Each gradient
# carries the rounding of its 16-bit MFMA operand (P or dS, 2^-9 relative for
# bf16) and of its 16-bit output (2^-9), about 1.6e-3 RMS together; dS =
# P (dP - D) also carries D = rowsum(dO o O) computed from the forward's 16-bit
# O, and dP - D cancels in rows dominated by one key, which can double the
# error there.  The bar is 1e-2, about 3x the largest error seen.
BWD_TOL = (2e-2, 1e-2)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_operands(w: Workload, x: dict):
    """Exact values the kernel sees, as the oracle's inputs (E4M3: code * descale)."""
    if w.dtype == "fp8_e4m3":
        dq, dk, dv = x["descale"]
        return (oracle.dequant_e4m3(x["q"], dq), oracle.dequant_e4m3(x["k"], dk),
                oracle.dequant_e4m3(x["v"], dv))
    return x["q"], x["k"], x["v"]


def run_gpu(w: Workload, x: dict, tile: int = 0, device="cuda:0"):
    q, k, v = (x[n].to(device) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, scale=w.sm_scale, causal=w.causal, descale=x["descale"], tile=tile)
    torch.cuda.synchronize()
    return o, lse


def errors(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray) -> dict:
    diff = o_gpu - o_ref
    return {
        "max_abs": float(np.abs(diff).max()) if diff.size else 0.0,
        "rel_l2": float(np.linalg.norm(diff) / max(np.linalg.norm(o_ref), 1e-300)) if diff.size else 0.0,
        "lse_max_abs": float(np.abs(lse_gpu - lse_ref).max()) if lse_ref.size else 0.0,
        "finite": bool(np.isfinite(o_gpu).all() and np.isfinite(lse_gpu).all()),
    }


def assert_within(w: Workload, err: dict, label: str = ""):
    max_abs, rel = TOL[w.dtype]
    msg = "%s %s %s" % (w.name, label, err)
    assert err["finite"], msg
    if max_abs is not None:
        assert err["max_abs"] <= max_abs, msg
    assert err["rel_l2"] <= rel, msg
    assert err["lse_max_abs"] <= LSE_TOL, msg


def full_parity(w: Workload, tile: int = 0, x: dict | None = None) -> dict:
    """Whole-tensor comparison (sizes the oracle finishes in seconds)."""
    x = x or make_inputs(w)
    o, lse = run_gpu(w, x, tile)
    qo, ko, vo = oracle_operands(w, x)
    o_ref, lse_ref = oracle.attention(qo, ko, vo, w.sm_scale, w.causal)
    return errors(o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, lse_ref)


def default_rows(w: Workload) -> int:
    """Query rows per workgroup of the default variant for w (its name reads
    br<waves>x<rows per wave>_...)."""
    import re
    name = fa.fa_variant_name(fa_dtype_code(w.dtype), w.d, w.causal, 1)
    m = re.search(r"br(\d+)x(\d+)", name)
    assert m, name
    return int(m.group(1)) * int(m.group(2))


def fa_dtype_code(dt: str) -> int:
    return {"f32": fa.FA_F32, "f16": fa.FA_F16, "bf16": fa.FA_BF16, "fp8_e4m3": fa.FA_FP8_E4M3}[dt]


def sample_rows(w: Workload, x: dict, br: int, n_random: int = 512, heads: int = 4,
                seed: int = 0, max_edges: int = 128) -> np.ndarray:
    """Rows to check at full size: every boosted row, random rows, both rows
    around query-block boundaries (all of them, or max_edges spread evenly
    over the head) and the first/last rows of a few heads."""
    rng = np.random.default_rng([w.seed_id, 99, seed])
    n = w.n_q
    picks = [x["boost_rows"]]
    bh_all = w.B * w.H
    hs = rng.choice(bh_all, size=min(heads, bh_all), replace=False)
    edges = np.arange(br, n, br)
    if edges.size > max_edges:
        edges = edges[np.unique(np.linspace(0, edges.size - 1, max_edges).round().astype(np.int64))]
    for bh in hs:
        base = bh * n
        picks.append(base + rng.integers(0, n, n_random // len(hs)))
        picks.append(base + np.concatenate([[0, n - 1], edges - 1, edges]))
    rows = np.unique(np.concatenate(picks).astype(np.int64))
    return rows


def streamed_parity(w: Workload, x: dict, o: torch.Tensor, lse: torch.Tensor) -> dict:
    """Whole-tensor comparison of the GPU's O and LSE with the oracle, one
    (batch, head) at a time so that host memory holds one head: max abs and
    LSE max abs over every element, relative L2 over the whole tensor."""
    qo, ko, vo = oracle_operands(w, x)
    max_abs = lse_max = 0.0
    sq_diff = sq_ref = 0.0
    finite = True
    for b in range(w.B):
        for h in range(w.H):
            o_ref, lse_ref = oracle.attention(qo[b, h], ko[b, h], vo[b, h], w.sm_scale, w.causal)
            og = o[b, h].double().cpu().numpy()
            lg = lse[b, h].double().cpu().numpy()
            finite &= bool(np.isfinite(og).all() and np.isfinite(lg).all())
            diff = og - o_ref
            max_abs = max(max_abs, float(np.abs(diff).max()))
            lse_max = max(lse_max, float(np.abs(lg - lse_ref).max()))
            sq_diff += float(np.square(diff).sum())
            sq_ref += float(np.square(o_ref).sum())
    return {"max_abs": max_abs, "rel_l2": math.sqrt(sq_diff / max(sq_ref, 1e-300)),
            "lse_max_abs": lse_max, "finite": finite, "heads": w.B * w.H}


def whole_parity(w: Workload, tile: int = 0) -> dict:
    """The workload's seeded inputs through the GPU path (default launch
    configuration), compared with the oracle over the whole tensor."""
    x = make_inputs(w)
    o, lse = run_gpu(w, x, tile)
    return streamed_parity(w, x, o, lse)


def sampled_parity(w: Workload, br: int, tile: int = 0, **kw) -> dict:
    x = make_inputs(w)
    o, lse = run_gpu(w, x, tile)
    rows = sample_rows(w, x, br, **kw)
    o_s = o.reshape(-1, w.d)[torch.from_numpy(rows).to(o.device)].double().cpu().numpy()
    l_s = lse.reshape(-1)[torch.from_numpy(rows).to(o.device)].double().cpu().numpy()
    del o, lse
    qo, ko, vo = oracle_operands(w, x)
    o_ref, lse_ref = oracle.attention(qo, ko, vo, w.sm_scale, w.causal, rows=rows)
    err = errors(o_s, l_s, o_ref, lse_ref)
    err["rows"] = int(rows.size)
    return err


# A gradient that is exactly zero in the definition (one key: dQ = dK = 0)
# comes out as rounding noise; it is checked against this absolute bound.
ZERO_GRAD_ATOL = 1e-3


def grad_errors(g_gpu: np.ndarray, g_ref: np.ndarray) -> dict:
    diff = g_gpu - g_ref
    ref_max = float(np.abs(g_ref).max()) if g_ref.size else 0.0
    return {
        "max_abs": float(np.abs(diff).max()) if diff.size else 0.0,
        "ref_max": ref_max,
        "max_rel": float(np.abs(diff).max() / ref_max) if diff.size and ref_max > 0 else 0.0,
        "rel_l2": float(np.linalg.norm(diff) / np.linalg.norm(g_ref)) if diff.size and ref_max > 0 else 0.0,
        "finite": bool(np.isfinite(g_gpu).all()),
    }


def assert_grads_within(errs: dict, label: str = ""):
    max_rel, rel = BWD_TOL
    for name, e in errs.items():
        msg = "%s %s %s" % (label, name, e)
        assert e["finite"], msg
        if e["ref_max"] == 0:
            assert e["max_abs"] <= ZERO_GRAD_ATOL, msg
            continue
        assert e["max_rel"] <= max_rel, msg
        assert e["rel_l2"] <= rel, msg
