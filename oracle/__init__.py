"""CPU oracle for exact attention forward (fp64) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  It shares no code with the GPU
library (``exact_attention_95_amd``) and never imports it.

The arithmetic lives in ``fa_oracle.c`` (plain C, IEEE double, libm); this
module only builds that file with gcc, converts inputs to float64 one
(batch, head) slice at a time and calls it through ctypes.

Functions and the passages they follow:

* :func:`attention` -- standard attention, three-pass softmax per row
  ("FlashAttention算子优化" section 1; plate 04 of "FlashAttention 与显存";
  section 1.3 of "Flash Attention 原理与实践").
* :func:`attention_blockwise` -- blockwise online softmax in v2 order
  ("FlashAttention算子优化" section 2, merge rule of plate 08) or v1 order
  ("Flash Attention 原理与实践" section 2.3).
* :func:`merge` -- merge of per-chunk results over a key partition
  (Flash-Decoding's last step, "Flash Attention 原理与实践" section 5.1, with
  the merge rule of plate 08).
* :func:`dequant_e4m3` -- OCP E4M3 code times a per-tensor descale.

Pins (tests/test_oracle.py): brute force at 50 digits with mpmath, the
unshifted textbook softmax, scipy's logsumexp, closed forms (one key, two
keys, Q = 0, constant V, shifted V, equal keys, causal row 0), rows of P
summing to 1, blockwise == naive on random partitions and tile shapes,
v1 == v2, planted mistakes caught, and the E4M3 decoder against torch's
float8_e4m3fn.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compiles the oracle's C source into a shared library with gcc."""
    if (not force and os.path.exists(out)
            and os.path.getmtime(out) >= os.path.getmtime(src)):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load(path: str | None = None):
    """Loads (building first if needed) and returns the ctypes library."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            _lib = _declare(ctypes.CDLL(build()))
        return _lib


def _declare(lib):
    lib.fa_oracle_naive.restype = ctypes.c_int
    lib.fa_oracle_naive.argtypes = [
        _dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_double, ctypes.c_int, _i64p, ctypes.c_int64, _dp, _dp, _dp]
    for name in ("fa_oracle_blockwise", "fa_oracle_blockwise_v1"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [
            _dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_double, ctypes.c_int, _i64p, ctypes.c_int64, _i64p,
            ctypes.c_int64, _dp, _dp]
    lib.fa_oracle_backward.restype = ctypes.c_int
    lib.fa_oracle_backward.argtypes = [
        _dp, _dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
        ctypes.c_int, _i64p, ctypes.c_int64, _i64p, ctypes.c_int64, _dp, _dp, _dp]
    _u32p = ctypes.POINTER(ctypes.c_uint32)
    _u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.fa_oracle_philox4x32_10.restype = None
    lib.fa_oracle_philox4x32_10.argtypes = [_u32p, _u32p, _u32p]
    lib.fa_oracle_dropout_p8.restype = ctypes.c_int
    lib.fa_oracle_dropout_p8.argtypes = [ctypes.c_double]
    lib.fa_oracle_dropout_mask.restype = ctypes.c_int
    lib.fa_oracle_dropout_mask.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_int, _u8p]
    lib.fa_oracle_attention_dropout.restype = ctypes.c_int
    lib.fa_oracle_attention_dropout.argtypes = [
        _dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_int,
        _i64p, ctypes.c_int64, _u8p, ctypes.c_double, _dp, _dp]
    lib.fa_oracle_backward_dropout.restype = ctypes.c_int
    lib.fa_oracle_backward_dropout.argtypes = [
        _dp, _dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
        ctypes.c_int, _u8p, ctypes.c_double, _dp, _dp, _dp]
    lib.fa_oracle_merge.restype = ctypes.c_int
    lib.fa_oracle_merge.argtypes = [_dp, _dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _dp, _dp]
    lib.fa_oracle_num_threads.restype = ctypes.c_int
    lib.fa_oracle_num_threads.argtypes = []
    lib.fa_oracle_set_num_threads.restype = ctypes.c_int
    lib.fa_oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.fa_oracle_e4m3_to_double.restype = ctypes.c_double
    lib.fa_oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.fa_oracle_dequant_e4m3.restype = ctypes.c_int
    lib.fa_oracle_dequant_e4m3.argtypes = [
        ctypes.POINTER(ctypes.c_uint8), ctypes.c_int64, ctypes.c_double, _dp]
    return lib


def _ptr(a, typ=_dp):
    return a.ctypes.data_as(typ) if a is not None else None


def _as_f64(x) -> np.ndarray:
    """float64 copy of a numpy array or CPU torch tensor (exact for fp16/bf16/fp32)."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _heads(x):
    """Views [B,H,N,d] (or [N,d]) as a list of per-head 2-D slices."""
    if x.ndim == 2:
        return x[None, None]
    if x.ndim != 4:
        raise ValueError("expected [B,H,N,d] or [N,d]")
    return x


def attention(q, k, v, scale: float, causal: bool = False, rows=None,
              return_p: bool = False, lib=None):
    """Standard attention in fp64 (three-pass softmax per row).

    q: [B,H,N_q,d], k and v: [B,H,N_kv,d] (numpy or CPU torch, any float
    dtype; converted exactly to float64 one head at a time).  ``scale`` is
    applied to the scores before the max; pass the same value the GPU
    library receives (e.g. the float32 nearest to 1/sqrt(d)).
    ``rows``: optional int array of flat row indices into B*H*N_q; then the
    results are [len(rows), d] and [len(rows)].  Otherwise O is
    [B,H,N_q,d] and LSE [B,H,N_q].  ``return_p`` adds P ([..., N_kv]).
    """
    lib = lib or load()
    q4, k4, v4 = (_heads(t) for t in (q, k, v))
    B, H, n_q, d = q4.shape
    n_kv = k4.shape[2]
    if k4.shape != (B, H, n_kv, d) or v4.shape != (B, H, n_kv, d):
        raise ValueError("shape mismatch")
    if rows is None:
        o = np.empty((B, H, n_q, d))
        lse = np.empty((B, H, n_q))
        p = np.empty((B, H, n_q, n_kv)) if return_p else None
        for b in range(B):
            for h in range(H):
                qh, kh, vh = _as_f64(q4[b, h]), _as_f64(k4[b, h]), _as_f64(v4[b, h])
                oh = np.empty((n_q, d))
                lh = np.empty(n_q)
                ph = np.empty((n_q, n_kv)) if return_p else None
                st = lib.fa_oracle_naive(_ptr(qh), _ptr(kh), _ptr(vh), n_q, n_kv, d,
                                         float(scale), int(bool(causal)), None, n_q,
                                         _ptr(oh), _ptr(lh), _ptr(ph))
                if st:
                    raise RuntimeError("fa_oracle_naive failed: %d" % st)
                o[b, h], lse[b, h] = oh, lh
                if return_p:
                    p[b, h] = ph
        if q.ndim == 2:
            o, lse = o[0, 0], lse[0, 0]
            p = p[0, 0] if return_p else None
        return (o, lse, p) if return_p else (o, lse)
    rows = np.asarray(rows, dtype=np.int64).ravel()
    o = np.empty((rows.size, d))
    lse = np.empty(rows.size)
    p = np.empty((rows.size, n_kv)) if return_p else None
    head_of = rows // n_q
    for bh in np.unique(head_of):
        sel = np.nonzero(head_of == bh)[0]
        b, h = divmod(int(bh), H)
        local = np.ascontiguousarray(rows[sel] - bh * n_q)
        qh, kh, vh = _as_f64(q4[b, h]), _as_f64(k4[b, h]), _as_f64(v4[b, h])
        oh = np.empty((sel.size, d))
        lh = np.empty(sel.size)
        ph = np.empty((sel.size, n_kv)) if return_p else None
        st = lib.fa_oracle_naive(_ptr(qh), _ptr(kh), _ptr(vh), n_q, n_kv, d,
                                 float(scale), int(bool(causal)), _ptr(local, _i64p),
                                 sel.size, _ptr(oh), _ptr(lh), _ptr(ph))
        if st:
            raise RuntimeError("fa_oracle_naive failed: %d" % st)
        o[sel], lse[sel] = oh, lh
        if return_p:
            p[sel] = ph
    return (o, lse, p) if return_p else (o, lse)


def num_threads(lib=None) -> int:
    """Threads the oracle's parallel loops use (OpenMP)."""
    return int((lib or load()).fa_oracle_num_threads())


def set_num_threads(n: int, lib=None) -> int:
    """Sets the threads of later parallel loops on this thread; returns the previous count."""
    return int((lib or load()).fa_oracle_set_num_threads(int(n)))


def cuts_from_block(n: int, block: int) -> np.ndarray:
    """Boundaries of consecutive blocks of ``block`` rows, last one ragged."""
    c = list(range(0, n, block)) + [n]
    return np.asarray(c, dtype=np.int64)


def attention_blockwise(q, k, v, scale: float, causal: bool = False,
                        q_cuts=None, kv_cuts=None, br: int | None = None,
                        bc: int | None = None, order: str = "v2", lib=None):
    """Blockwise online-softmax attention for one head ([N,d] inputs).

    Give the partitions as explicit boundaries (``q_cuts``/``kv_cuts``,
    starting at 0 and ending at N) or as block sizes ``br``/``bc``.
    ``order`` is "v2" (query block outside, division after the key loop) or
    "v1" (key block outside, normalised O written back each step).
    """
    lib = lib or load()
    qh, kh, vh = _as_f64(q), _as_f64(k), _as_f64(v)
    n_q, d = qh.shape
    n_kv = kh.shape[0]
    if q_cuts is None:
        q_cuts = cuts_from_block(n_q, br or n_q)
    if kv_cuts is None:
        kv_cuts = cuts_from_block(n_kv, bc or n_kv)
    q_cuts = np.ascontiguousarray(q_cuts, dtype=np.int64)
    kv_cuts = np.ascontiguousarray(kv_cuts, dtype=np.int64)
    o = np.empty((n_q, d))
    lse = np.empty(n_q)
    fn = {"v2": lib.fa_oracle_blockwise, "v1": lib.fa_oracle_blockwise_v1}[order]
    st = fn(_ptr(qh), _ptr(kh), _ptr(vh), n_q, n_kv, d, float(scale), int(bool(causal)),
            _ptr(q_cuts, _i64p), q_cuts.size, _ptr(kv_cuts, _i64p), kv_cuts.size,
            _ptr(o), _ptr(lse))
    if st:
        raise RuntimeError("blockwise oracle failed: %d" % st)
    return o, lse


def merge(o_parts, lse_parts, lib=None):
    """Merges per-chunk (O_s, LSE_s) of a key partition (plate 08's rule on
    whole chunks).  o_parts: [n_parts, n_rows, d]; lse_parts: [n_parts, n_rows]
    (-inf: chunk with no visible key).  Returns (O [n_rows, d], LSE [n_rows])."""
    lib = lib or load()
    op = np.ascontiguousarray(o_parts, dtype=np.float64)
    lp = np.ascontiguousarray(lse_parts, dtype=np.float64)
    n_parts, n_rows, d = op.shape
    o = np.empty((n_rows, d))
    lse = np.empty(n_rows)
    if lib.fa_oracle_merge(_ptr(op), _ptr(lp), n_parts, n_rows, d, _ptr(o), _ptr(lse)):
        raise RuntimeError("merge failed")
    return o, lse


def backward(q, k, v, dout, scale: float, causal: bool = False, rows=None, keys=None, lib=None):
    """Gradients dQ, dK, dV of standard attention in fp64 for upstream dO.

    q, dout: [B,H,N_q,d]; k, v: [B,H,N_kv,d] (or one head [N,d]; numpy or CPU
    torch, converted exactly to float64 one head at a time).  ``rows`` /
    ``keys``: optional flat indices into B*H*N_q rows / B*H*N_kv keys; then
    dQ is [len(rows), d] and dK, dV are [len(keys), d] (either may be an
    empty selection).  Otherwise full [B,H,N,d] arrays are returned.
    """
    lib = lib or load()
    q4, k4, v4, g4 = (_heads(t) for t in (q, k, v, dout))
    B, H, n_q, d = q4.shape
    n_kv = k4.shape[2]
    if k4.shape != (B, H, n_kv, d) or v4.shape != (B, H, n_kv, d) or g4.shape != q4.shape:
        raise ValueError("shape mismatch")
    full = rows is None and keys is None
    rows = np.arange(B * H * n_q, dtype=np.int64) if rows is None else np.asarray(rows, np.int64).ravel()
    keys = np.arange(B * H * n_kv, dtype=np.int64) if keys is None else np.asarray(keys, np.int64).ravel()
    dq = np.empty((rows.size, d))
    dk = np.empty((keys.size, d))
    dv = np.empty((keys.size, d))
    for bh in np.unique(np.concatenate([rows // n_q, keys // n_kv])):
        b, h = divmod(int(bh), H)
        rsel = np.nonzero(rows // n_q == bh)[0]
        ksel = np.nonzero(keys // n_kv == bh)[0]
        lr = np.ascontiguousarray(rows[rsel] - bh * n_q)
        lk = np.ascontiguousarray(keys[ksel] - bh * n_kv)
        qh, kh, vh, gh = (_as_f64(t[b, h]) for t in (q4, k4, v4, g4))
        dqh = np.empty((rsel.size, d))
        dkh = np.empty((ksel.size, d))
        dvh = np.empty((ksel.size, d))
        st = lib.fa_oracle_backward(_ptr(qh), _ptr(kh), _ptr(vh), _ptr(gh), n_q, n_kv, d,
                                    float(scale), int(bool(causal)), _ptr(lr, _i64p), rsel.size,
                                    _ptr(lk, _i64p), ksel.size, _ptr(dqh), _ptr(dkh), _ptr(dvh))
        if st:
            raise RuntimeError("fa_oracle_backward failed: %d" % st)
        dq[rsel], dk[ksel], dv[ksel] = dqh, dkh, dvh
    if not full:
        return dq, dk, dv
    dq = dq.reshape(B, H, n_q, d)
    dk = dk.reshape(B, H, n_kv, d)
    dv = dv.reshape(B, H, n_kv, d)
    if q.ndim == 2:
        return dq[0, 0], dk[0, 0], dv[0, 0]
    return dq, dk, dv


def philox4x32_10(ctr, key, lib=None):
    """Philox4x32-10 of a 4-word counter and 2-word key; returns 4 words."""
    lib = lib or load()
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    o = (ctypes.c_uint32 * 4)()
    lib.fa_oracle_philox4x32_10(c, k, o)
    return [int(x) for x in o]


def dropout_p8(p: float, lib=None) -> int:
    """The dropout probability quantised to p8 / 256."""
    return int((lib or load()).fa_oracle_dropout_p8(float(p)))


def dropout_rescale(p8: int) -> float:
    return 256.0 / (256.0 - p8)


def dropout_mask(seed: int, offset: int, bh: int, n_q: int, n_kv: int, p8: int, lib=None) -> np.ndarray:
    """[n_q, n_kv] uint8 keep mask (1 = kept) of slice bh."""
    lib = lib or load()
    m = np.empty((n_q, n_kv), dtype=np.uint8)
    st = lib.fa_oracle_dropout_mask(int(seed) & (2**64 - 1), int(offset) & (2**64 - 1), int(bh), n_q, n_kv,
                                    int(p8), m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
    if st:
        raise RuntimeError("fa_oracle_dropout_mask failed: %d" % st)
    return m


def attention_dropout(q, k, v, scale: float, causal: bool, p: float, seed: int, offset: int,
                      rows=None, lib=None):
    """Attention with dropout in fp64 ([B,H,N,d] or [N,d]); returns (O, LSE).

    ``rows``: optional flat row indices into B*H*N_q, as in ``attention``; then
    the results are [len(rows), d] and [len(rows)]."""
    lib = lib or load()
    q4, k4, v4 = (_heads(t) for t in (q, k, v))
    B, H, n_q, d = q4.shape
    n_kv = k4.shape[2]
    p8 = dropout_p8(p, lib)

    def head(b, h, local):
        keep = dropout_mask(seed, offset, b * H + h, n_q, n_kv, p8, lib)
        qh, kh, vh = _as_f64(q4[b, h]), _as_f64(k4[b, h]), _as_f64(v4[b, h])
        n_rows = n_q if local is None else local.size
        oh, lh = np.empty((n_rows, d)), np.empty(n_rows)
        st = lib.fa_oracle_attention_dropout(
            _ptr(qh), _ptr(kh), _ptr(vh), n_q, n_kv, d, float(scale), int(bool(causal)),
            None if local is None else _ptr(local, _i64p), n_rows,
            keep.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), dropout_rescale(p8), _ptr(oh), _ptr(lh))
        if st:
            raise RuntimeError("fa_oracle_attention_dropout failed: %d" % st)
        return oh, lh

    if rows is None:
        o = np.empty((B, H, n_q, d))
        lse = np.empty((B, H, n_q))
        for b in range(B):
            for h in range(H):
                o[b, h], lse[b, h] = head(b, h, None)
        if q.ndim == 2:
            return o[0, 0], lse[0, 0]
        return o, lse
    rows = np.asarray(rows, dtype=np.int64).ravel()
    o = np.empty((rows.size, d))
    lse = np.empty(rows.size)
    head_of = rows // n_q
    for bh in np.unique(head_of):
        sel = np.nonzero(head_of == bh)[0]
        b, h = divmod(int(bh), H)
        o[sel], lse[sel] = head(b, h, np.ascontiguousarray(rows[sel] - bh * n_q))
    return o, lse


def backward_dropout(q, k, v, dout, scale: float, causal: bool, p: float, seed: int, offset: int,
                     heads=None, lib=None):
    """Gradients of attention_dropout in fp64; returns (dQ, dK, dV).

    ``heads``: optional flat (batch, head) indices; then the results are
    [len(heads), N, d] for those heads only."""
    lib = lib or load()
    q4, k4, v4, g4 = (_heads(t) for t in (q, k, v, dout))
    B, H, n_q, d = q4.shape
    n_kv = k4.shape[2]
    p8 = dropout_p8(p, lib)
    sel = list(range(B * H)) if heads is None else [int(x) for x in heads]
    dq, dk, dv = np.empty((len(sel), n_q, d)), np.empty((len(sel), n_kv, d)), np.empty((len(sel), n_kv, d))
    for n, bh in enumerate(sel):
        b, h = divmod(bh, H)
        keep = dropout_mask(seed, offset, bh, n_q, n_kv, p8, lib)
        qh, kh, vh, gh = (_as_f64(t[b, h]) for t in (q4, k4, v4, g4))
        st = lib.fa_oracle_backward_dropout(
            _ptr(qh), _ptr(kh), _ptr(vh), _ptr(gh), n_q, n_kv, d, float(scale), int(bool(causal)),
            keep.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), dropout_rescale(p8),
            _ptr(dq[n]), _ptr(dk[n]), _ptr(dv[n]))
        if st:
            raise RuntimeError("fa_oracle_backward_dropout failed: %d" % st)
    if heads is not None:
        return dq, dk, dv
    dq, dk, dv = dq.reshape(B, H, n_q, d), dk.reshape(B, H, n_kv, d), dv.reshape(B, H, n_kv, d)
    if q.ndim == 2:
        return dq[0, 0], dk[0, 0], dv[0, 0]
    return dq, dk, dv


def e4m3_to_double(code: int, lib=None) -> float:
    """Value of one OCP E4M3 (fn) code."""
    return (lib or load()).fa_oracle_e4m3_to_double(int(code) & 0xFF)


def dequant_e4m3(codes, descale: float, lib=None) -> np.ndarray:
    """E4M3 codes (uint8 array or torch float8_e4m3fn tensor) times descale, in fp64."""
    lib = lib or load()
    if hasattr(codes, "detach"):
        import torch
        codes = codes.detach().to("cpu").contiguous().view(torch.uint8).numpy()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    st = lib.fa_oracle_dequant_e4m3(c.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                    c.size, float(descale), _ptr(out))
    if st:
        raise RuntimeError("dequant failed")
    return out
