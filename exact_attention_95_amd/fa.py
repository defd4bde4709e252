"""ctypes binding of the C ABI in include/fa.h (argument marshalling only).

The functions ``fa_fwd``, ``fa_fwd_ex``, ``fa_validate``, ``fa_strerror``,
``fa_num_variants``, ``fa_variant_name``, ``fa_fwd_splitkv``,
``fa_splitkv_workspace_bytes``, ``fa_bwd``, ``fa_bwd_validate``,
``fa_bwd_workspace_bytes``, ``fa_dropout_mask``, ``fa_fwd_splitkv_noalloc`` and the measurement probes
``fa_probe``, ``fa_probe_hbm_read``, ``fa_probe_work_per_iter`` and ``fa_probe_wall_clock_khz``
(include/fa_probe.h) mirror the C entry points of the same names.  ``fwd``
is the torch convenience form: it allocates O and LSE with torch on the
inputs' device and calls ``fa_fwd_ex`` on torch's current stream.  All attention arithmetic runs in the HIP kernels; there is no CPU
path, and the library must have been built (``exact_attention_95_amd.build``).
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_F32, FA_F16, FA_BF16, FA_FP8_E4M3 = 0, 1, 2, 3
(FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_HEAD_DIM, FA_ERR_DTYPE, FA_ERR_ALIGN, FA_ERR_SCALE,
 FA_ERR_ALIAS, FA_ERR_DEVICE, FA_ERR_LAUNCH, FA_ERR_VARIANT, FA_ERR_WORKSPACE, FA_ERR_DROPOUT,
 FA_ERR_LONG_KV, FA_ERR_SCRATCH) = range(15)
FA_MAX_NKV_SINGLE_PASS = 1 << 20     # include/fa.h
FA_NOALLOC_SCRATCH_BYTES = 64 << 20  # include/fa.h

EXPORTED = ("fa_fwd", "fa_fwd_ex", "fa_validate", "fa_strerror", "fa_num_variants",
            "fa_variant_name", "fa_fwd_splitkv", "fa_splitkv_workspace_bytes", "fa_bwd",
            "fa_bwd_validate", "fa_bwd_workspace_bytes", "fa_dropout_mask", "fa_fwd_splitkv_noalloc")
# measurement probes (include/fa_probe.h)
PROBE_EXPORTED = ("fa_probe", "fa_probe_hbm_read", "fa_probe_work_per_iter", "fa_probe_wall_clock_khz")
(FA_PROBE_MFMA_BF16, FA_PROBE_MFMA_F16, FA_PROBE_MFMA_FP8, FA_PROBE_MFMA_F32, FA_PROBE_EXP,
 FA_PROBE_FMA) = range(6)


class FaFwdArgs(ctypes.Structure):
    """Mirror of ``fa_fwd_args``."""

    _fields_ = [
        ("Q", ctypes.c_void_p), ("K", ctypes.c_void_p), ("V", ctypes.c_void_p),
        ("O", ctypes.c_void_p), ("LSE", ctypes.c_void_p),
        ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N_q", ctypes.c_int64),
        ("N_kv", ctypes.c_int64), ("d", ctypes.c_int64),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int), ("dtype", ctypes.c_int),
        ("descale_q", ctypes.c_float), ("descale_k", ctypes.c_float),
        ("descale_v", ctypes.c_float),
        ("stream", ctypes.c_void_p), ("tile_override", ctypes.c_int),
        ("dropout_p", ctypes.c_float), ("dropout_seed", ctypes.c_uint64),
        ("dropout_offset", ctypes.c_uint64),
    ]


class FaBwdArgs(ctypes.Structure):
    """Mirror of ``fa_bwd_args``."""

    _fields_ = [
        ("Q", ctypes.c_void_p), ("K", ctypes.c_void_p), ("V", ctypes.c_void_p),
        ("O", ctypes.c_void_p), ("dO", ctypes.c_void_p), ("LSE", ctypes.c_void_p),
        ("dQ", ctypes.c_void_p), ("dK", ctypes.c_void_p), ("dV", ctypes.c_void_p),
        ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N_q", ctypes.c_int64),
        ("N_kv", ctypes.c_int64), ("d", ctypes.c_int64),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int), ("dtype", ctypes.c_int),
        ("stream", ctypes.c_void_p),
        ("dropout_p", ctypes.c_float), ("dropout_seed", ctypes.c_uint64),
        ("dropout_offset", ctypes.c_uint64),
    ]


class FaError(RuntimeError):
    def __init__(self, status: int):
        super().__init__("fa status %d: %s" % (status, fa_strerror(status)))
        self.status = status


_lock = threading.Lock()
_lib = None


def load(path: str = LIB_PATH):
    """Loads libfa.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError("HIP library %s is not built; run exact_attention_95_amd.build"
                                   % path)
            lib = ctypes.CDLL(path)
            i64, vp = ctypes.c_int64, ctypes.c_void_p
            lib.fa_fwd.restype = ctypes.c_int
            lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                                   ctypes.c_int, ctypes.c_int]
            lib.fa_fwd_ex.restype = ctypes.c_int
            lib.fa_fwd_ex.argtypes = [ctypes.POINTER(FaFwdArgs)]
            lib.fa_validate.restype = ctypes.c_int
            lib.fa_validate.argtypes = [ctypes.POINTER(FaFwdArgs)]
            lib.fa_strerror.restype = ctypes.c_char_p
            lib.fa_strerror.argtypes = [ctypes.c_int]
            lib.fa_num_variants.restype = ctypes.c_int
            lib.fa_num_variants.argtypes = [ctypes.c_int, i64, ctypes.c_int]
            lib.fa_variant_name.restype = ctypes.c_char_p
            lib.fa_variant_name.argtypes = [ctypes.c_int, i64, ctypes.c_int, ctypes.c_int]
            lib.fa_fwd_splitkv.restype = ctypes.c_int
            lib.fa_fwd_splitkv.argtypes = [ctypes.POINTER(FaFwdArgs), ctypes.c_int, vp, i64]
            lib.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
            lib.fa_fwd_splitkv_noalloc.argtypes = [ctypes.POINTER(FaFwdArgs), ctypes.c_int]
            lib.fa_splitkv_workspace_bytes.restype = i64
            lib.fa_splitkv_workspace_bytes.argtypes = [ctypes.POINTER(FaFwdArgs), ctypes.c_int]
            lib.fa_bwd.restype = ctypes.c_int
            lib.fa_bwd.argtypes = [ctypes.POINTER(FaBwdArgs), vp, i64]
            lib.fa_bwd_validate.restype = ctypes.c_int
            lib.fa_bwd_validate.argtypes = [ctypes.POINTER(FaBwdArgs)]
            lib.fa_bwd_workspace_bytes.restype = i64
            lib.fa_bwd_workspace_bytes.argtypes = [ctypes.POINTER(FaBwdArgs)]
            lib.fa_dropout_mask.restype = ctypes.c_int
            lib.fa_dropout_mask.argtypes = [ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, i64, i64,
                                            i64, vp, vp]
            lib.fa_probe.restype = ctypes.c_int
            lib.fa_probe.argtypes = [ctypes.c_int, i64, i64, vp, vp, vp]
            lib.fa_probe_hbm_read.restype = ctypes.c_int
            lib.fa_probe_hbm_read.argtypes = [vp, i64, i64, vp, vp]
            lib.fa_probe_work_per_iter.restype = ctypes.c_double
            lib.fa_probe_work_per_iter.argtypes = [ctypes.c_int]
            lib.fa_probe_wall_clock_khz.restype = i64
            lib.fa_probe_wall_clock_khz.argtypes = []
            _lib = lib
        return _lib


def fa_fwd(Q, K, V, O, LSE, B, H, N_q, N_kv, d, scale, causal, dtype) -> int:
    """Raw ``fa_fwd``: pointers as ints (device addresses), returns the status."""
    return load().fa_fwd(Q, K, V, O, LSE, B, H, N_q, N_kv, d, scale, int(causal), dtype)


def fa_fwd_ex(args: FaFwdArgs) -> int:
    return load().fa_fwd_ex(ctypes.byref(args))


def fa_validate(args: FaFwdArgs) -> int:
    return load().fa_validate(ctypes.byref(args))


def fa_strerror(status: int) -> str:
    return load().fa_strerror(status).decode()


def fa_num_variants(dtype: int, d: int, causal: bool) -> int:
    return load().fa_num_variants(dtype, d, int(bool(causal)))


def fa_variant_name(dtype: int, d: int, causal: bool, v: int) -> str:
    return load().fa_variant_name(dtype, d, int(bool(causal)), v).decode()


def fa_fwd_splitkv(args: FaFwdArgs, num_splits: int, workspace, workspace_bytes: int) -> int:
    return load().fa_fwd_splitkv(ctypes.byref(args), num_splits, workspace, workspace_bytes)


def fa_fwd_splitkv_noalloc(args: FaFwdArgs, num_splits: int) -> int:
    return load().fa_fwd_splitkv_noalloc(ctypes.byref(args), num_splits)


def fa_splitkv_workspace_bytes(args: FaFwdArgs, num_splits: int) -> int:
    return load().fa_splitkv_workspace_bytes(ctypes.byref(args), num_splits)


def fa_bwd(args: FaBwdArgs, workspace, workspace_bytes: int) -> int:
    return load().fa_bwd(ctypes.byref(args), workspace, workspace_bytes)


def fa_bwd_validate(args: FaBwdArgs) -> int:
    return load().fa_bwd_validate(ctypes.byref(args))


def fa_bwd_workspace_bytes(args: FaBwdArgs) -> int:
    return load().fa_bwd_workspace_bytes(ctypes.byref(args))


def fa_dropout_mask(dropout_p, seed, offset, BH, N_q, N_kv, mask, stream=None) -> int:
    return load().fa_dropout_mask(float(dropout_p), int(seed) & (2**64 - 1), int(offset) & (2**64 - 1),
                                  BH, N_q, N_kv, mask, stream)


def fa_probe(kind, n_wg, iters, sink, clocks=None, stream=None) -> int:
    return load().fa_probe(kind, n_wg, iters, sink, clocks, stream)


def fa_probe_hbm_read(buf, nbytes, n_wg, sink, stream=None) -> int:
    return load().fa_probe_hbm_read(buf, nbytes, n_wg, sink, stream)


def fa_probe_work_per_iter(kind) -> float:
    return load().fa_probe_work_per_iter(kind)


def fa_probe_wall_clock_khz() -> int:
    return load().fa_probe_wall_clock_khz()


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16,
             torch.float8_e4m3fn: FA_FP8_E4M3}
    if t.dtype not in codes:
        raise TypeError("unsupported dtype %s" % t.dtype)
    return codes[t.dtype]


def make_args(q, k, v, o, lse, scale: float, causal: bool, descale=(1.0, 1.0, 1.0),
              stream=None, tile: int = 0, dropout=(0.0, 0, 0)) -> FaFwdArgs:
    """fa_fwd_args for torch tensors q [B,H,N_q,d], k/v [B,H,N_kv,d], o, lse."""
    B, H, N_q, d = q.shape
    a = FaFwdArgs()
    a.Q, a.K, a.V, a.O = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()
    a.LSE = lse.data_ptr() if lse is not None else None
    a.B, a.H, a.N_q, a.N_kv, a.d = B, H, N_q, k.shape[2], d
    a.scale = scale
    a.causal = int(bool(causal))
    a.dtype = _dtype_code(q)
    a.descale_q, a.descale_k, a.descale_v = (float(x) for x in descale)
    a.stream = stream
    a.tile_override = tile
    a.dropout_p = float(dropout[0])
    a.dropout_seed = int(dropout[1]) & (2**64 - 1)
    a.dropout_offset = int(dropout[2]) & (2**64 - 1)
    return a


def check_tensors(q, k, v, out=None, lse=None, extra=(), workspace=None, need_cuda: bool = True,
                  dtypes=None, out_dtype=None):
    """Host-side checks of the torch tensors handed to the library, before any
    launch: q [B,H,N_q,d] and k, v [B,H,N_kv,d] of one dtype (``dtypes``: the
    allowed ones); ``out`` [B,H,N_q,d] of ``out_dtype``; ``lse`` float32
    [B,H,N_q]; ``extra``: (name, tensor, shape, dtype) tuples; ``workspace``
    uint8.  Every tensor must be contiguous and on q's device (a GPU device
    unless ``need_cuda`` is False).  Raises TypeError (dtype) or ValueError
    (anything else); the C library checks sizes, alignment and overlap again
    from the raw arguments."""
    import torch
    named = [("q", q), ("k", k), ("v", v)]
    if need_cuda and not all(t.is_cuda for _, t in named):
        raise RuntimeError("the attention library needs GPU tensors; there is no CPU path")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected [B,H,N,d] tensors: q %s k %s v %s"
                         % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k, v must share a dtype (got %s, %s, %s)" % (q.dtype, k.dtype, v.dtype))
    if dtypes is not None and q.dtype not in dtypes:
        raise TypeError("unsupported dtype %s here" % q.dtype)
    if k.shape != v.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape),
                                                              tuple(v.shape)))
    B, H, N_q, d = q.shape
    if out is not None:
        named.append(("out", out))
        if tuple(out.shape) != (B, H, N_q, d):
            raise ValueError("out must be [B,H,N_q,d] = %s, got %s" % ((B, H, N_q, d), tuple(out.shape)))
        if out_dtype is not None and out.dtype != out_dtype:
            raise TypeError("out must be %s, got %s" % (out_dtype, out.dtype))
    if lse is not None:
        named.append(("lse", lse))
        if tuple(lse.shape) != (B, H, N_q):
            raise ValueError("lse must be [B,H,N_q] = %s, got %s" % ((B, H, N_q), tuple(lse.shape)))
        if lse.dtype != torch.float32:
            raise TypeError("lse must be float32, got %s" % lse.dtype)
    for name, t, shape, dt in extra:
        named.append((name, t))
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s must be %s, got %s" % (name, tuple(shape), tuple(t.shape)))
        if t.dtype != dt:
            raise TypeError("%s must be %s, got %s" % (name, dt, t.dtype))
    if workspace is not None:
        named.append(("workspace", workspace))
        if workspace.dtype != torch.uint8:
            raise TypeError("workspace must be uint8, got %s" % workspace.dtype)
    for name, t in named:
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if t.device != q.device:
            raise ValueError("%s is on %s, q on %s" % (name, t.device, q.device))


def _stream_handle(stream, device):
    import torch
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def fwd(q, k, v, scale: float | None = None, causal: bool = False, descale=None, out=None,
        lse=None, with_lse: bool = True, stream=None, tile: int = 0, dropout_p: float = 0.0,
        seed: int = 0, offset: int = 0):
    """Attention forward of torch device tensors; returns (O, LSE).

    q: [B,H,N_q,d]; k, v: [B,H,N_kv,d]; all contiguous, same dtype, on one
    gfx950 device.  scale defaults to 1/sqrt(d) (as float32).  For
    float8_e4m3fn inputs, descale = (descale_q, descale_k, descale_v) and O is
    bfloat16.  ``out`` / ``lse``: optional preallocated outputs (checked).
    ``stream``: a torch stream or raw hipStream_t (default: torch's
    current stream).  ``dropout_p``, ``seed``, ``offset``: dropout of P with
    the library's Philox mask (see include/fa.h).
    """
    import torch
    out_dtype = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    check_tensors(q, k, v, out, lse, out_dtype=out_dtype)
    B, H, N_q, d = q.shape
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    if out is None:
        out = torch.empty((B, H, N_q, d), dtype=out_dtype, device=q.device)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N_q), dtype=torch.float32, device=q.device)
    stream = _stream_handle(stream, q.device)
    args = make_args(q, k, v, out, lse, scale, causal, descale or (1.0, 1.0, 1.0), stream, tile,
                     (dropout_p, seed, offset))
    with torch.cuda.device(q.device):
        st = fa_fwd_ex(args)
    if st != FA_OK:
        raise FaError(st)
    return out, lse


def fwd_splitkv(q, k, v, scale: float | None = None, causal: bool = False, num_splits: int = 0,
                out=None, lse=None, with_lse: bool = True, stream=None, tile: int = 0,
                workspace=None, noalloc: bool = False, descale=None):
    """Split-KV attention forward (bf16/fp16 with d in {64, 128, 256}, or
    float8_e4m3fn with d = 128 and bf16 O); returns (O, LSE).

    Same contract as ``fwd`` (``descale`` as there); the key range is processed in ``num_splits``
    chunks (0: library choice) whose partials are merged on the GPU.  The
    float32 workspace is allocated with torch unless ``workspace`` (a uint8
    device tensor) is given, or unless ``noalloc``: then the partials go to
    the library's static scratch buffer (``fa_fwd_splitkv_noalloc``).
    """
    import torch
    # an unsupported (but consistent) dtype is the C library's to report
    out_dtype = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    check_tensors(q, k, v, out, lse, workspace=workspace, out_dtype=out_dtype)
    B, H, N_q, d = q.shape
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    if out is None:
        out = torch.empty((B, H, N_q, d), dtype=out_dtype, device=q.device)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N_q), dtype=torch.float32, device=q.device)
    stream = _stream_handle(stream, q.device)
    args = make_args(q, k, v, out, lse, scale, causal, descale or (1.0, 1.0, 1.0), stream, tile)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace")
        with torch.cuda.device(q.device):
            st = fa_fwd_splitkv_noalloc(args, num_splits)
        if st != FA_OK:
            raise FaError(st)
        return out, lse
    need = fa_splitkv_workspace_bytes(args, num_splits)
    if need < 0:
        raise FaError(fa_validate(args) or FA_ERR_VARIANT)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        st = fa_fwd_splitkv(args, num_splits, workspace.data_ptr(), workspace.numel())
    if st != FA_OK:
        raise FaError(st)
    return out, lse


def make_bwd_args(q, k, v, o, lse, do, dq, dk, dv, scale: float, causal: bool,
                  stream=None, dropout=(0.0, 0, 0)) -> FaBwdArgs:
    """fa_bwd_args for torch tensors (shapes as in ``bwd``)."""
    B, H, N_q, d = q.shape
    a = FaBwdArgs()
    ptr = lambda t: t.data_ptr() if t is not None else None
    a.Q, a.K, a.V, a.O, a.dO = ptr(q), ptr(k), ptr(v), ptr(o), ptr(do)
    a.LSE = ptr(lse)
    a.dQ, a.dK, a.dV = ptr(dq), ptr(dk), ptr(dv)
    a.B, a.H, a.N_q, a.N_kv, a.d = B, H, N_q, k.shape[2], d
    a.scale = scale
    a.causal = int(bool(causal))
    a.dtype = _dtype_code(q)
    a.stream = stream
    a.dropout_p = float(dropout[0])
    a.dropout_seed = int(dropout[1]) & (2**64 - 1)
    a.dropout_offset = int(dropout[2]) & (2**64 - 1)
    return a


def bwd(q, k, v, o, lse, do, scale: float | None = None, causal: bool = False, stream=None,
        workspace=None, dropout_p: float = 0.0, seed: int = 0, offset: int = 0):
    """Attention backward of torch device tensors; returns (dQ, dK, dV).

    q, o, do: [B,H,N_q,d]; k, v: [B,H,N_kv,d] (bf16 or fp16, d in {64, 128,
    256}, contiguous, one gfx950 device); lse: [B,H,N_q] float32.  o and lse must be the forward's
    outputs for these inputs, scale and causal.  The float32 workspace (D per
    query row) is allocated with torch unless ``workspace`` (a uint8 device
    tensor) is given.
    """
    import torch
    B, H, N_q, d = q.shape if q.dim() == 4 else (0, 0, 0, 0)
    check_tensors(q, k, v, workspace=workspace,
                  extra=(("o", o, (B, H, N_q, d), q.dtype), ("do", do, (B, H, N_q, d), q.dtype),
                         ("lse", lse, (B, H, N_q), torch.float32)))
    B, H, N_q, d = q.shape
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = _stream_handle(stream, q.device)
    args = make_bwd_args(q, k, v, o, lse, do, dq, dk, dv, scale, causal, stream,
                         (dropout_p, seed, offset))
    need = fa_bwd_workspace_bytes(args)
    if need < 0:
        raise FaError(fa_bwd_validate(args))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        st = fa_bwd(args, workspace.data_ptr(), workspace.numel())
    if st != FA_OK:
        raise FaError(st)
    return dq, dk, dv


def dropout_mask(dropout_p: float, seed: int, offset: int, B: int, H: int, N_q: int, N_kv: int,
                 device="cuda", stream=None):
    """The dropout keep mask ([B,H,N_q,N_kv] uint8 on the GPU) the kernels use."""
    import torch
    m = torch.empty((B, H, N_q, N_kv), dtype=torch.uint8, device=device)
    stream = _stream_handle(stream, m.device)
    with torch.cuda.device(m.device):
        st = fa_dropout_mask(dropout_p, seed, offset, B * H, N_q, N_kv, m.data_ptr() if m.numel() else None,
                             stream)
    if st != FA_OK:
        raise FaError(st)
    return m
