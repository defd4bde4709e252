"""C-ABI tests that need no GPU: the library loads, exports every function
include/fa.h and include/fa_probe.h declare, and fa_validate reaches every
pre-launch status."""
import ctypes
import math
import os
import re

import pytest

from exact_attention_95_amd import fa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fa.h")
PROBE_HEADER = os.path.join(os.path.dirname(HEADER), "fa_probe.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    probes = declared_functions(PROBE_HEADER)
    assert set(names) == set(fa.EXPORTED)
    assert set(probes) == set(fa.PROBE_EXPORTED)
    lib = fa.load()
    for n in names + probes:
        assert hasattr(lib, n), n
    # and nothing but these fa_ symbols is exported as a C function
    out = os.popen("nm -D --defined-only %s" % fa.LIB_PATH).read()
    exported = {m for m in re.findall(r" T (fa_\w+)$", out, flags=re.M)}
    assert exported == set(names) | set(probes)


def test_probe_host_side():
    """Work per loop iteration of each probe, and the argument checks that run
    before any HIP call."""
    mfma = {fa.FA_PROBE_MFMA_BF16: 32 * 32 * 16, fa.FA_PROBE_MFMA_F16: 32 * 32 * 16,
            fa.FA_PROBE_MFMA_FP8: 32 * 32 * 64, fa.FA_PROBE_MFMA_F32: 32 * 32 * 2}
    for kind, macs in mfma.items():
        assert fa.fa_probe_work_per_iter(kind) == 8 * 2 * macs  # 8 MFMAs per iteration
    assert fa.fa_probe_work_per_iter(fa.FA_PROBE_EXP) == 16 * 64
    assert fa.fa_probe_work_per_iter(fa.FA_PROBE_FMA) == 16 * 64
    assert fa.fa_probe_work_per_iter(6) == 0.0
    assert fa.fa_probe(6, 1, 1, 0x1000) == fa.FA_ERR_DTYPE
    assert fa.fa_probe(-1, 1, 1, 0x1000) == fa.FA_ERR_DTYPE
    assert fa.fa_probe(fa.FA_PROBE_EXP, 0, 1, 0x1000) == fa.FA_ERR_SHAPE
    assert fa.fa_probe(fa.FA_PROBE_EXP, (1 << 20) + 1, 1, 0x1000) == fa.FA_ERR_SHAPE
    assert fa.fa_probe(fa.FA_PROBE_EXP, 1, 0, 0x1000) == fa.FA_ERR_SHAPE
    assert fa.fa_probe(fa.FA_PROBE_EXP, 1, (1 << 30) + 1, 0x1000) == fa.FA_ERR_SHAPE
    assert fa.fa_probe(fa.FA_PROBE_EXP, 1, 1, None) == fa.FA_ERR_NULL
    assert fa.fa_probe(fa.FA_PROBE_EXP, 1, 1, 0x1002) == fa.FA_ERR_ALIGN
    assert fa.fa_probe(fa.FA_PROBE_EXP, 1, 1, 0x1000, 0x2004) == fa.FA_ERR_ALIGN
    # the HBM read probe: byte count, grid, pointers and alignment
    assert fa.fa_probe_hbm_read(0x10000, 0, 1, 0x1000) == fa.FA_ERR_SHAPE
    assert fa.fa_probe_hbm_read(0x10000, 24, 1, 0x1000) == fa.FA_ERR_SHAPE
    assert fa.fa_probe_hbm_read(0x10000, 16, 0, 0x1000) == fa.FA_ERR_SHAPE
    assert fa.fa_probe_hbm_read(0x10000, 16, (1 << 20) + 1, 0x1000) == fa.FA_ERR_SHAPE
    assert fa.fa_probe_hbm_read(None, 16, 1, 0x1000) == fa.FA_ERR_NULL
    assert fa.fa_probe_hbm_read(0x10000, 16, 1, None) == fa.FA_ERR_NULL
    assert fa.fa_probe_hbm_read(0x10008, 16, 1, 0x1000) == fa.FA_ERR_ALIGN
    assert fa.fa_probe_hbm_read(0x10000, 16, 1, 0x1002) == fa.FA_ERR_ALIGN


def test_args_struct_layout(tmp_path):
    """The ctypes mirror matches the C compiler's layout of fa_fwd_args."""
    fields = [f[0] for f in fa.FaFwdArgs._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "fa.h"\nint main(void){\n'
                   + "".join('printf("%%zu\\n", offsetof(fa_fwd_args, %s));\n' % f for f in fields)
                   + 'printf("%zu\\n", sizeof(fa_fwd_args)); return 0; }\n')
    exe = tmp_path / "layout"
    assert os.system("gcc -I%s -o %s %s" % (os.path.dirname(HEADER), exe, src)) == 0
    got = [int(x) for x in os.popen(str(exe)).read().split()]
    want = [getattr(fa.FaFwdArgs, f).offset for f in fields] + [ctypes.sizeof(fa.FaFwdArgs)]
    assert got == want



def test_headers_are_plain_c_and_the_library_links_from_c(tmp_path):
    """Both public headers compile as strict C99 with no warnings, and a C
    program links against libfa.so and calls its host-side entry points (no
    GPU call: fa_validate and fa_strerror only)."""
    src = tmp_path / "caller.c"
    src.write_text(
        '#include <stdio.h>\n#include <string.h>\n#include "fa.h"\n#include "fa_probe.h"\n'
        "int main(void) {\n"
        "    fa_fwd_args a;\n"
        "    memset(&a, 0, sizeof a);\n"
        "    a.B = 1; a.H = 1; a.N_q = 4; a.N_kv = 4; a.d = 64; a.scale = 0.125f; a.dtype = FA_BF16;\n"
        '    printf("%d\\n", fa_validate(&a));\n'
        "    a.d = 96;\n"
        '    printf("%d\\n", fa_validate(&a));\n'
        '    printf("%s\\n", fa_strerror(FA_ERR_NULL));\n'
        "    return 0;\n}\n")
    exe = tmp_path / "caller"
    lib_dir = os.path.dirname(fa.LIB_PATH)
    cmd = ("gcc -std=c99 -Wall -Wextra -pedantic -Werror -I%s -o %s %s -L%s -lfa -Wl,-rpath,%s"
           % (os.path.dirname(HEADER), exe, src, lib_dir, lib_dir))
    assert os.system(cmd) == 0, cmd
    out = os.popen(str(exe)).read().split("\n")
    assert int(out[0]) == fa.FA_ERR_NULL      # required pointers missing
    assert int(out[1]) == fa.FA_ERR_HEAD_DIM  # d = 96 is not compiled
    assert out[2] == fa.fa_strerror(fa.FA_ERR_NULL)

def good_args(**kw):
    a = fa.FaFwdArgs()
    a.Q, a.K, a.V, a.O, a.LSE = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
    a.B, a.H, a.N_q, a.N_kv, a.d = 2, 3, 100, 90, 64
    a.scale = 0.125
    a.causal = 0
    a.dtype = fa.FA_BF16
    a.descale_q = a.descale_k = a.descale_v = 1.0
    a.tile_override = 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_validate_accepts_good_args():
    assert fa.fa_validate(good_args()) == fa.FA_OK
    for dt in (fa.FA_F32, fa.FA_F16, fa.FA_BF16):
        for d in (64, 128, 256):
            for causal in (0, 1):
                assert fa.fa_validate(good_args(dtype=dt, d=d, causal=causal)) == fa.FA_OK
    assert fa.fa_validate(good_args(LSE=None)) == fa.FA_OK
    assert fa.fa_validate(good_args(scale=0.0)) == fa.FA_OK
    assert fa.fa_validate(good_args(scale=-3.0)) == fa.FA_OK


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), fa.FA_ERR_NULL),
    (dict(K=None), fa.FA_ERR_NULL),
    (dict(V=None), fa.FA_ERR_NULL),
    (dict(O=None), fa.FA_ERR_NULL),
    (dict(B=-1), fa.FA_ERR_SHAPE),
    (dict(H=-2), fa.FA_ERR_SHAPE),
    (dict(N_q=-1), fa.FA_ERR_SHAPE),
    (dict(N_kv=0), fa.FA_ERR_SHAPE),
    (dict(N_q=1 << 40), fa.FA_ERR_SHAPE),
    (dict(B=1 << 20, H=1 << 20), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_HEAD_DIM),
    (dict(d=0), fa.FA_ERR_HEAD_DIM),
    (dict(dtype=7), fa.FA_ERR_DTYPE),
    (dict(dtype=-1), fa.FA_ERR_DTYPE),
    (dict(Q=0x100008), fa.FA_ERR_ALIGN),
    (dict(O=0x400004), fa.FA_ERR_ALIGN),
    (dict(LSE=0x500002), fa.FA_ERR_ALIGN),
    (dict(scale=math.inf), fa.FA_ERR_SCALE),
    (dict(scale=math.nan), fa.FA_ERR_SCALE),
    (dict(scale=3e38), fa.FA_ERR_SCALE),
    (dict(O=0x100000 + 4096), fa.FA_ERR_ALIAS),
    (dict(O=0x300000), fa.FA_ERR_ALIAS),
    (dict(LSE=0x400000 + 64), fa.FA_ERR_ALIAS),
    (dict(LSE=0x200000), fa.FA_ERR_ALIAS),
    (dict(tile_override=99), fa.FA_ERR_VARIANT),
    (dict(tile_override=-1), fa.FA_ERR_VARIANT),
])
def test_validate_reports_each_status(kw, status):
    assert fa.fa_validate(good_args(**kw)) == status


def test_empty_problems_are_valid_noops_even_with_null_pointers():
    for kw in (dict(B=0), dict(H=0), dict(N_q=0)):
        a = good_args(Q=None, K=None, V=None, O=None, LSE=None, **kw)
        assert fa.fa_validate(a) == fa.FA_OK
        assert fa.fa_fwd_ex(a) == fa.FA_OK     # returns before touching HIP


def test_validate_null_args_pointer():
    lib = fa.load()
    assert lib.fa_validate(None) == fa.FA_ERR_NULL
    assert lib.fa_fwd_ex(None) == fa.FA_ERR_NULL


def declared_statuses(header=HEADER):
    """(name, value) of every fa_status enumerator the header declares."""
    text = open(header).read()
    body = text[text.index("FA_OK = 0"):text.index("} fa_status;")]
    return [(n, int(v)) for n, v in re.findall(r"(FA_\w+)\s*=\s*(\d+)", body)]


def test_strerror_names_every_status():
    statuses = declared_statuses()
    assert [v for _, v in statuses] == list(range(len(statuses)))  # dense, from 0
    assert len(statuses) == 15
    for name, value in statuses:
        assert getattr(fa, name) == value, name  # the binding mirrors the header
    msgs = {fa.fa_strerror(v) for _, v in statuses}
    assert len(msgs) == len(statuses) and "unknown status" not in msgs
    assert fa.fa_strerror(len(statuses)) == "unknown status"
    assert fa.fa_strerror(12345) == "unknown status"
    assert fa.fa_strerror(-1) == "unknown status"


def test_single_pass_key_range_limit():
    """fa_fwd / fa_fwd_ex accept at most FA_MAX_NKV_SINGLE_PASS keys per row;
    split-KV takes longer rows (chunks of at most that many keys)."""
    text = open(HEADER).read()
    assert re.search(r"#define FA_MAX_NKV_SINGLE_PASS \(1 << 20\)", text)
    assert fa.FA_MAX_NKV_SINGLE_PASS == 1 << 20
    big = dict(B=1, H=1, N_q=3, d=128, Q=0x1000, K=1 << 32, V=1 << 34, O=0x2000, LSE=0x3000)
    lim = fa.FA_MAX_NKV_SINGLE_PASS
    assert fa.fa_validate(good_args(N_kv=lim, **big)) == fa.FA_OK
    assert fa.fa_validate(good_args(N_kv=lim + 1, **big)) == fa.FA_ERR_LONG_KV
    for dt in (fa.FA_F32, fa.FA_F16, fa.FA_FP8_E4M3):
        assert fa.fa_validate(good_args(N_kv=lim + 1, dtype=dt, **big)) == fa.FA_ERR_LONG_KV
    a = good_args(N_kv=lim + 1, **big)
    assert fa.fa_fwd_ex(a) == fa.FA_ERR_LONG_KV        # refused before any HIP call
    lib = fa.load()
    assert lib.fa_fwd(a.Q, a.K, a.V, a.O, a.LSE, 1, 1, 3, lim + 1, 128, 0.1, 0, fa.FA_BF16) == \
        fa.FA_ERR_LONG_KV
    # split-KV: any N_kv up to 2^30; even num_splits = 1 is cut into chunks of <= 2^20 keys
    n_kv = (1 << 24) + 37
    a = good_args(N_kv=n_kv, **big)
    chunks = -(-n_kv // lim)
    one = fa.fa_splitkv_workspace_bytes(a, 1)
    want = -(-chunks * 3 * 128 * 4 // 256) * 256 + -(-chunks * 3 * 4 // 256) * 256
    assert one == want
    assert fa.fa_splitkv_workspace_bytes(good_args(N_kv=(1 << 30) + 1, **big), 0) == -1


def test_splitkv_grid_bound():
    """The split-KV grid (chunks x heads x 128-row query blocks) must fit 2^31 - 1."""
    # 2^22 heads of 1024 rows: 8 query blocks each, 2^25 blocks; 64 chunks would be 2^31
    a = good_args(B=1 << 11, H=1 << 11, N_q=1024, N_kv=64 * 64, d=64, K=1 << 44, V=1 << 45,
                  O=1 << 46, LSE=1 << 47, Q=1 << 43)
    assert fa.fa_splitkv_workspace_bytes(a, 63) > 0
    assert fa.fa_splitkv_workspace_bytes(a, 64) == -1
    assert fa.fa_fwd_splitkv(a, 64, 1 << 48, 1 << 50) == fa.FA_ERR_SHAPE


def test_variant_table():
    for dt in (fa.FA_F32, fa.FA_F16, fa.FA_BF16):
        for d in (64, 128, 256):
            for c in (0, 1):
                n = fa.fa_num_variants(dt, d, c)
                assert n >= 1
                names = [fa.fa_variant_name(dt, d, c, v) for v in range(1, n + 1)]
                assert all(names) and len(set(names)) == n
                assert fa.fa_variant_name(dt, d, c, n + 1) == ""
                assert fa.fa_variant_name(dt, d, c, 0) == ""
    assert fa.fa_num_variants(fa.FA_BF16, 96, 0) == 0
    for c in (0, 1):
        assert fa.fa_num_variants(fa.FA_FP8_E4M3, 128, c) >= 1
        assert fa.fa_num_variants(fa.FA_FP8_E4M3, 64, c) == 0


def test_fp8_validation():
    assert fa.fa_validate(good_args(dtype=fa.FA_FP8_E4M3, d=128)) == fa.FA_OK
    assert fa.fa_validate(good_args(dtype=fa.FA_FP8_E4M3, d=64)) == fa.FA_ERR_HEAD_DIM
    assert fa.fa_validate(good_args(dtype=fa.FA_FP8_E4M3, d=128, descale_k=math.inf)) == fa.FA_ERR_SCALE
    assert fa.fa_validate(good_args(dtype=fa.FA_FP8_E4M3, d=128, descale_q=1e30, descale_k=1e30)) == fa.FA_ERR_SCALE


def test_fwd_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="GPU"):
        fa.fwd(q, q, q)


def test_splitkv_workspace_bytes():
    a = good_args(B=2, H=3, N_q=5, N_kv=1000, d=128, K=0x1000000, V=0x2000000, O=0x3000000,
                  LSE=0x4000000)
    # 1000 keys = 16 tiles of 64; 2 chunks of 8 tiles
    n, rows = 2, 2 * 3 * 5
    want = -(-n * rows * 128 * 4 // 256) * 256 + -(-n * rows * 4 // 256) * 256
    assert fa.fa_splitkv_workspace_bytes(a, 2) == want
    assert fa.fa_splitkv_workspace_bytes(a, 1000) > 0           # capped at one chunk per tile
    assert fa.fa_splitkv_workspace_bytes(a, 0) > 0
    assert fa.fa_splitkv_workspace_bytes(a, -1) == -1
    # d = 256: 90 keys make 2 tiles, one chunk; 600 rows of 256 floats and their LSE
    assert fa.fa_splitkv_workspace_bytes(good_args(d=256), 0) == 600 * 256 * 4 + -(-600 * 4 // 256) * 256
    assert fa.fa_splitkv_workspace_bytes(good_args(dtype=fa.FA_F32), 0) == -1
    assert fa.fa_splitkv_workspace_bytes(good_args(B=0), 0) == 0
    assert fa.fa_fwd_splitkv(good_args(B=0), 0, None, 0) == fa.FA_OK


def test_bwd_args_struct_layout(tmp_path):
    """The ctypes mirror matches the C compiler's layout of fa_bwd_args."""
    fields = [f[0] for f in fa.FaBwdArgs._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "fa.h"\nint main(void){\n'
                   + "".join('printf("%%zu\\n", offsetof(fa_bwd_args, %s));\n' % f for f in fields)
                   + 'printf("%zu\\n", sizeof(fa_bwd_args)); return 0; }\n')
    exe = tmp_path / "layout"
    assert os.system("gcc -I%s -o %s %s" % (os.path.dirname(HEADER), exe, src)) == 0
    got = [int(x) for x in os.popen(str(exe)).read().split()]
    want = [getattr(fa.FaBwdArgs, f).offset for f in fields] + [ctypes.sizeof(fa.FaBwdArgs)]
    assert got == want


def good_bwd_args(**kw):
    a = fa.FaBwdArgs()
    # B*H*N*d*2 bytes = 2*3*100*64*2 = 76800 (Q-like), 2*3*90*64*2 = 69120 (K-like)
    a.Q, a.K, a.V, a.O, a.dO, a.LSE = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000
    a.dQ, a.dK, a.dV = 0x700000, 0x800000, 0x900000
    a.B, a.H, a.N_q, a.N_kv, a.d = 2, 3, 100, 90, 64
    a.scale = 0.125
    a.causal = 0
    a.dtype = fa.FA_BF16
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_bwd_validate_accepts_good_args():
    for dt in (fa.FA_BF16, fa.FA_F16):
        for d in (64, 128):
            for causal in (0, 1):
                assert fa.fa_bwd_validate(good_bwd_args(dtype=dt, d=d, causal=causal)) == fa.FA_OK
    assert fa.fa_bwd_validate(good_bwd_args(scale=-3.0)) == fa.FA_OK
    assert fa.fa_bwd_validate(good_bwd_args(scale=0.0)) == fa.FA_OK


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=fa.FA_F32), fa.FA_ERR_DTYPE),
    (dict(dtype=fa.FA_FP8_E4M3), fa.FA_ERR_DTYPE),
    (dict(dtype=9), fa.FA_ERR_DTYPE),
    (dict(d=96), fa.FA_ERR_HEAD_DIM),
    (dict(d=512), fa.FA_ERR_HEAD_DIM),
    (dict(d=96), fa.FA_ERR_HEAD_DIM),
    (dict(N_kv=0), fa.FA_ERR_SHAPE),
    (dict(B=-1), fa.FA_ERR_SHAPE),
    (dict(N_q=(1 << 30) + 1), fa.FA_ERR_SHAPE),
    (dict(scale=math.nan), fa.FA_ERR_SCALE),
    (dict(scale=math.inf), fa.FA_ERR_SCALE),
    (dict(scale=3.0e38), fa.FA_ERR_SCALE),
    (dict(dO=None), fa.FA_ERR_NULL),
    (dict(LSE=None), fa.FA_ERR_NULL),
    (dict(dQ=None), fa.FA_ERR_NULL),
    (dict(dK=None), fa.FA_ERR_NULL),
    (dict(O=0x400008), fa.FA_ERR_ALIGN),
    (dict(dV=0x900004), fa.FA_ERR_ALIGN),
    (dict(LSE=0x600002), fa.FA_ERR_ALIGN),
    (dict(dQ=0x100000), fa.FA_ERR_ALIAS),                  # dQ on Q
    (dict(dK=0x700000 + 64), fa.FA_ERR_ALIAS),             # dK inside dQ
    (dict(dV=0x800000), fa.FA_ERR_ALIAS),                  # dV on dK
    (dict(dQ=0x600000), fa.FA_ERR_ALIAS),                  # dQ over LSE
])
def test_bwd_validate_reports_each_status(kw, status):
    assert fa.fa_bwd_validate(good_bwd_args(**kw)) == status


def test_bwd_validate_null_args_and_empty_problems():
    assert fa.load().fa_bwd_validate(None) == fa.FA_ERR_NULL
    empty = good_bwd_args(B=0, Q=None, K=None, V=None, O=None, dO=None, LSE=None, dQ=None, dK=None, dV=None)
    assert fa.fa_bwd_validate(empty) == fa.FA_OK
    assert fa.fa_bwd_workspace_bytes(empty) == 0
    assert fa.fa_bwd(empty, None, 0) == fa.FA_OK
    # N_q = 0: only dK, dV (zeros) are written, so only K, V, dK, dV are needed
    no_rows = good_bwd_args(N_q=0, Q=None, O=None, dO=None, LSE=None, dQ=None)
    assert fa.fa_bwd_validate(no_rows) == fa.FA_OK
    assert fa.fa_bwd_workspace_bytes(no_rows) == 0


def test_bwd_workspace_bytes():
    a = good_bwd_args()
    assert fa.fa_bwd_workspace_bytes(a) == 2 * (-(-2 * 3 * 100 * 4 // 256) * 256)  # D, LSE log2(e)
    assert fa.fa_bwd_workspace_bytes(good_bwd_args(d=256)) == 2 * (-(-2 * 3 * 100 * 4 // 256) * 256)
    assert fa.fa_bwd_workspace_bytes(good_bwd_args(d=96)) == -1


def test_bwd_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 4)
    with pytest.raises(RuntimeError, match="GPU"):
        fa.bwd(q, q, q, q, lse, q)


@pytest.mark.parametrize("p", [-0.1, 1.0, 2.0, math.nan, math.inf])
def test_dropout_probability_is_validated(p):
    assert fa.fa_validate(good_args(dropout_p=p)) == fa.FA_ERR_DROPOUT
    assert fa.fa_bwd_validate(good_bwd_args(dropout_p=p)) == fa.FA_ERR_DROPOUT
    assert fa.fa_dropout_mask(p, 1, 2, 1, 4, 4, None) == fa.FA_ERR_DROPOUT


def test_dropout_support_limits():
    assert fa.fa_validate(good_args(dropout_p=0.1)) == fa.FA_OK
    assert fa.fa_validate(good_args(dropout_p=0.1, dtype=fa.FA_F16, d=128, causal=1)) == fa.FA_OK
    assert fa.fa_validate(good_args(dropout_p=0.1, dtype=fa.FA_F32)) == fa.FA_ERR_DROPOUT
    assert fa.fa_validate(good_args(dropout_p=0.1, d=256)) == fa.FA_OK
    assert fa.fa_validate(good_args(dropout_p=0.1, dtype=fa.FA_FP8_E4M3, d=128)) == fa.FA_ERR_DROPOUT
    # p quantised to 0 (p < 1/512) is no dropout, accepted everywhere
    assert fa.fa_validate(good_args(dropout_p=1e-4, dtype=fa.FA_F32)) == fa.FA_OK
    a = good_args(B=2, H=3, N_q=5, N_kv=1000, d=128, K=0x1000000, V=0x2000000, O=0x3000000,
                  LSE=0x4000000, dropout_p=0.2)
    assert fa.fa_splitkv_workspace_bytes(a, 0) == -1
    assert fa.fa_fwd_splitkv(a, 0, None, 0) == fa.FA_ERR_DROPOUT
    assert fa.fa_bwd_validate(good_bwd_args(dropout_p=0.3, dropout_seed=2**64 - 1, dropout_offset=7)) == fa.FA_OK
    assert fa.fa_bwd_validate(good_bwd_args(d=256)) == fa.FA_OK
    assert fa.fa_bwd_validate(good_bwd_args(d=256, dropout_p=0.2)) == fa.FA_OK
    assert fa.fa_bwd_validate(good_bwd_args(d=256, dropout_p=0.2, dtype=fa.FA_F32)) == fa.FA_ERR_DTYPE


def test_dropout_mask_entry_validation():
    assert fa.fa_dropout_mask(0.1, 1, 2, -1, 4, 4, None) == fa.FA_ERR_SHAPE
    assert fa.fa_dropout_mask(0.1, 1, 2, 1, -4, 4, None) == fa.FA_ERR_SHAPE
    assert fa.fa_dropout_mask(0.1, 1, 2, 0, 4, 4, None) == fa.FA_OK
    assert fa.fa_dropout_mask(0.1, 1, 2, 3, 0, 4, None) == fa.FA_OK
    assert fa.fa_dropout_mask(0.1, 1, 2, 1, 4, 4, None) == fa.FA_ERR_NULL


def test_tensor_checks_run_before_any_launch():
    """The Python binding rejects mismatched dtypes, shapes, non-contiguous or
    misplaced tensors (including out, lse and the workspace) on the host; the
    checker runs on CPU tensors here with the device requirement lifted."""
    import torch
    chk = fa.check_tensors
    bf, f16 = torch.bfloat16, torch.float16
    q = torch.zeros(2, 3, 5, 64, dtype=bf)
    k = torch.zeros(2, 3, 7, 64, dtype=bf)
    chk(q, k, k, need_cuda=False)
    chk(q, k, k, torch.zeros(2, 3, 5, 64, dtype=bf), torch.zeros(2, 3, 5), need_cuda=False, out_dtype=bf)
    bad = [
        (TypeError, dict(k=k.to(torch.float8_e4m3fn))),
        (TypeError, dict(v=k.to(f16))),
        (ValueError, dict(k=torch.zeros(2, 3, 7, 128, dtype=bf), v=torch.zeros(2, 3, 7, 128, dtype=bf))),
        (ValueError, dict(v=torch.zeros(2, 3, 8, 64, dtype=bf))),
        (ValueError, dict(k=torch.zeros(2, 3, 64, 7, dtype=bf).transpose(2, 3))),
        (ValueError, dict(q=torch.zeros(3, 5, 64, dtype=bf))),
        (ValueError, dict(out=torch.zeros(2, 3, 4, 64, dtype=bf))),
        (ValueError, dict(out=torch.zeros(2, 3, 64, 5, dtype=bf).transpose(2, 3))),
        (TypeError, dict(out=torch.zeros(2, 3, 5, 64, dtype=f16))),
        (TypeError, dict(lse=torch.zeros(2, 3, 5, dtype=bf))),
        (ValueError, dict(lse=torch.zeros(2, 3, 4))),
        (TypeError, dict(workspace=torch.zeros(64, dtype=torch.float32))),
        (ValueError, dict(workspace=torch.zeros(64, 2, dtype=torch.uint8)[:, 0])),
        (TypeError, dict(dtypes=(f16,))),
    ]
    for exc, kw in bad:
        args = dict(q=q, k=k, v=k, out=None, lse=None, workspace=None, out_dtype=bf)
        args.update(kw)
        with pytest.raises(exc):
            chk(args.pop("q"), args.pop("k"), args.pop("v"), need_cuda=False, **args)
    # backward extras: o, do [B,H,N_q,d] in q's dtype and float32 lse
    ok = (("o", q, (2, 3, 5, 64), bf), ("lse", torch.zeros(2, 3, 5), (2, 3, 5), torch.float32))
    chk(q, k, k, extra=ok, need_cuda=False)
    with pytest.raises(TypeError):
        chk(q, k, k, extra=(("lse", torch.zeros(2, 3, 5, dtype=bf), (2, 3, 5), torch.float32),),
            need_cuda=False)
    with pytest.raises(ValueError):
        chk(q, k, k, extra=(("do", q[:, :, :4], (2, 3, 5, 64), bf),), need_cuda=False)
    # every public entry point refuses CPU tensors before touching the library's kernels
    with pytest.raises(RuntimeError, match="GPU"):
        fa.fwd_splitkv(q, k, k)


def test_noalloc_entry_point_host_checks():
    """fa_fwd_splitkv_noalloc: argument errors and the scratch limit are
    reported before any HIP call; empty problems are no-ops."""
    text = open(HEADER).read()
    assert re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \(64 << 20\)", text)
    assert fa.FA_NOALLOC_SCRATCH_BYTES == 64 << 20
    lib = fa.load()
    assert lib.fa_fwd_splitkv_noalloc(None, 0) == fa.FA_ERR_NULL
    assert fa.fa_fwd_splitkv_noalloc(good_args(B=0), 0) == fa.FA_OK
    assert fa.fa_fwd_splitkv_noalloc(good_args(d=96), 0) == fa.FA_ERR_HEAD_DIM
    assert fa.fa_fwd_splitkv_noalloc(good_args(dtype=fa.FA_F32), 0) == fa.FA_ERR_VARIANT
    assert fa.fa_fwd_splitkv_noalloc(good_args(), -1) == fa.FA_ERR_SHAPE
    assert fa.fa_fwd_splitkv_noalloc(good_args(dropout_p=0.2), 0) == fa.FA_ERR_DROPOUT
    # 64 heads of 4096 rows at d = 128: one chunk, 128 MiB of partials
    big = good_args(B=1, H=64, N_q=4096, N_kv=8192, d=128, Q=1 << 36, K=1 << 37, V=1 << 38,
                    O=1 << 39, LSE=1 << 40)
    assert fa.fa_splitkv_workspace_bytes(big, 0) > fa.FA_NOALLOC_SCRATCH_BYTES
    assert fa.fa_fwd_splitkv_noalloc(big, 0) == fa.FA_ERR_SCRATCH
    # the decode shape of the benchmark fits with room to spare
    dec = good_args(B=8, H=32, N_q=1, N_kv=65536, d=128, Q=1 << 36, K=1 << 37, V=1 << 38,
                    O=1 << 39, LSE=1 << 40)
    assert 0 < fa.fa_splitkv_workspace_bytes(dec, 0) <= fa.FA_NOALLOC_SCRATCH_BYTES // 64
