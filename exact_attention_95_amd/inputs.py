"""Seeded synthetic inputs for attention workloads.

This module only draws and stores numbers: it holds none of the attention
arithmetic, and both the GPU path's callers and the CPU oracle's callers take
their inputs from here.

Each (batch, head) slice of Q, K and V is drawn independently as i.i.d.
N(0, 1) float32 from ``numpy.random.default_rng([seed_id, tensor_id, b, h])``
(tensor_id 0 = Q, 1 = K, 2 = V; 4 = the upstream gradient dO of the backward
pass), so any single head can be regenerated on its own.  Storage dtypes are produced by torch's round-to-nearest-even casts;
E4M3 uses one scale per tensor that maps the absolute maximum to 448 and
passes the reciprocal (as float32) on as the descale.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

DTYPES = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "fp8_e4m3": torch.float8_e4m3fn,
}

E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention forward problem: shapes, storage dtype, mask, scale."""

    name: str
    seed_id: int
    B: int
    H: int
    n_q: int
    n_kv: int
    d: int
    dtype: str
    causal: bool = False
    scale: float | None = None      # None: float32 nearest to 1/sqrt(d)
    boost_frac: float = 0.0         # fraction of query rows multiplied by boost
    boost: float = 1.0

    @property
    def sm_scale(self) -> float:
        if self.scale is not None:
            return float(np.float32(self.scale))
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def flops(self) -> float:
        """Attention forward FLOPs: 4*B*H*N_q*N_kv*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.n_q * self.n_kv * self.d
        return f / 2 if self.causal else f

    @property
    def bwd_flops(self) -> float:
        """Attention backward FLOPs of its five matrix products (S recomputed,
        dP, dV, dK, dQ): 10*B*H*N_q*N_kv*d, halved when causal."""
        return 2.5 * self.flops


# Workloads shaped like the ones the pages measure (see the design notes for
# which page each stands in for).  seed_id is the first word of every seed.
WORKLOADS = {
    w.name: w for w in [
        Workload("single_head_f32_n256_d64", 1, 1, 1, 256, 256, 64, "f32"),
        Workload("gpt2_medium_bf16_n1024_d64", 2, 64, 16, 1024, 1024, 64, "bf16"),
        Workload("long_f16_causal_n4096_d64", 3, 16, 8, 4096, 4096, 64, "f16", causal=True),
        Workload("long_f16_causal_n16384_d64", 3, 16, 8, 16384, 16384, 64, "f16", causal=True),
        Workload("long_f16_causal_n65536_d64", 3, 16, 8, 65536, 65536, 64, "f16", causal=True),
        Workload("headline_bf16_n8192_d128", 4, 4, 16, 8192, 8192, 128, "bf16",
                 boost_frac=0.01, boost=8.0),
        Workload("headline_bf16_causal_n8192_d128", 4, 4, 16, 8192, 8192, 128, "bf16",
                 causal=True, boost_frac=0.01, boost=8.0),
        Workload("large_head_bf16_n16384_d256", 5, 2, 16, 16384, 16384, 256, "bf16"),
        Workload("fp8_e4m3_n16384_d128", 6, 2, 16, 16384, 16384, 128, "fp8_e4m3"),
        # decode: one new query row per sequence against a long key/value cache
        Workload("decode_bf16_b8_h32_nkv65536_d128", 7, 8, 32, 1, 65536, 128, "bf16"),
        # the same decode with an E4M3 key/value cache (per-tensor descales)
        Workload("decode_e4m3_b8_h32_nkv65536_d128", 8, 8, 32, 1, 65536, 128, "fp8_e4m3"),
    ]
}


def head_normal(seed_id: int, tensor_id: int, b: int, h: int, n: int, d: int) -> np.ndarray:
    """[n, d] float32 i.i.d. N(0,1) for one (batch, head) slice of one tensor."""
    rng = np.random.default_rng([seed_id, tensor_id, b, h])
    return rng.standard_normal((n, d), dtype=np.float32)


def boost_rows(w: Workload) -> np.ndarray:
    """Flat indices (into B*H*N_q) of the query rows that get multiplied by w.boost."""
    total = w.B * w.H * w.n_q
    count = int(math.floor(w.boost_frac * total))
    if count == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng([w.seed_id, 3])
    return np.sort(rng.choice(total, size=count, replace=False)).astype(np.int64)


def _tensor_f32(w: Workload, tensor_id: int, n: int) -> np.ndarray:
    """All heads of one tensor; heads are drawn in parallel threads (each head
    has its own generator, so the result does not depend on the schedule)."""
    import concurrent.futures
    import os
    x = np.empty((w.B, w.H, n, w.d), dtype=np.float32)

    def fill(bh):
        b, h = divmod(bh, w.H)
        rng = np.random.default_rng([w.seed_id, tensor_id, b, h])
        rng.standard_normal((n, w.d), dtype=np.float32, out=x[b, h])

    if w.B * w.H * n * w.d < (1 << 22):
        for bh in range(w.B * w.H):
            fill(bh)
    else:
        workers = min(16, os.cpu_count() or 1)
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(w.B * w.H)))
    return x


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor E4M3 codes: s = fp32(448 / absmax), codes = rne(x * s); returns (codes, descale)."""
    amax = float(x.abs().max())
    s = np.float32(E4M3_MAX / amax) if amax > 0 else np.float32(1.0)
    y = (x.float() * float(s)).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn)
    return codes, float(np.float32(1.0) / s)


def make_inputs(w: Workload) -> dict:
    """CPU torch tensors q [B,H,N_q,d], k, v [B,H,N_kv,d] in w.dtype.

    Also returns 'descale' (per-tensor E4M3 descales for q, k, v, else 1.0)
    and 'boost_rows' (the flat query rows that were multiplied by w.boost
    before the cast; exact, the boost being a power of two).
    """
    q = _tensor_f32(w, 0, w.n_q)
    rows = boost_rows(w)
    if rows.size:
        q.reshape(-1, w.d)[rows] *= np.float32(w.boost)
    k = _tensor_f32(w, 1, w.n_kv)
    v = _tensor_f32(w, 2, w.n_kv)
    out = {"boost_rows": rows}
    if w.dtype == "fp8_e4m3":
        qs, ks, vs = (quantize_e4m3(torch.from_numpy(t)) for t in (q, k, v))
        out.update(q=qs[0], k=ks[0], v=vs[0], descale=(qs[1], ks[1], vs[1]))
    else:
        dt = DTYPES[w.dtype]
        out.update(q=torch.from_numpy(q).to(dt), k=torch.from_numpy(k).to(dt),
                   v=torch.from_numpy(v).to(dt), descale=(1.0, 1.0, 1.0))
    return out


def random_problem(seed: int, B: int, H: int, n_q: int, n_kv: int, d: int,
                   dtype: str, causal: bool = False, scale: float | None = None,
                   boost_frac: float = 0.0, boost: float = 1.0) -> tuple[Workload, dict]:
    """Workload + inputs for an arbitrary shape (tests of ragged and edge shapes)."""
    w = Workload("random_%d" % seed, 1000 + seed, B, H, n_q, n_kv, d, dtype, causal,
                 scale, boost_frac, boost)
    return w, make_inputs(w)


def make_dout(w: Workload) -> torch.Tensor:
    """Upstream gradient dO [B,H,N_q,d] for the backward pass: i.i.d. N(0,1)
    per head (tensor_id 4), cast to w.dtype (bf16 or f16)."""
    return torch.from_numpy(_tensor_f32(w, 4, w.n_q)).to(DTYPES[w.dtype])
