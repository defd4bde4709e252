"""Pins for the oracle's dropout (no GPU).

The generator is Philox4x32-10 from its published definition; it is pinned
by the known-answer vectors published with that algorithm (Random123).  The
mask's statistics are pinned by binomial bounds; the dropout attention by
the no-dropout oracle (p8 = 0, all kept), by a closed form (V = 1: O_i =
rescale * sum of the kept probabilities) and by its definition recomputed
from the probabilities; the dropout gradients by central differences of the
dropout forward (the mask is fixed, so the function is smooth).  A planted-
mistake test checks that these pins catch plausible slips in the C source.
"""
import shutil

import numpy as np
import pytest

import oracle

# Known-answer vectors of Philox4x32-10 (counter, key, output).
PHILOX_KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,out", PHILOX_KAT)
def test_philox_known_answers(ctr, key, out):
    assert oracle.philox4x32_10(ctr, key) == list(out)


def test_p8_quantisation():
    assert oracle.dropout_p8(0.0) == 0
    assert oracle.dropout_p8(1e-9) == 0
    assert oracle.dropout_p8(0.1) == 26            # floor(25.6 + 0.5)
    assert oracle.dropout_p8(0.5) == 128
    assert oracle.dropout_p8(0.999) == 255         # clamped
    assert oracle.dropout_rescale(128) == 2.0


def test_mask_is_the_defined_byte():
    """Spot-check the mask against Philox outputs picked by hand."""
    seed, offset, bh, p8 = 0x1234_5678_9ABC_DEF0, 0x11_0000_0005, 3, 100
    m = oracle.dropout_mask(seed, offset, bh, 13, 22, p8)
    key = (seed & 0xFFFFFFFF, seed >> 32)
    for i, j in [(0, 0), (5, 7), (12, 21), (9, 16), (3, 3)]:
        out = oracle.philox4x32_10((j // 4, i // 4, bh, offset & 0xFFFFFFFF), key)
        byte = (out[i % 4] >> (8 * (j % 4))) & 0xFF
        assert m[i, j] == (1 if byte >= p8 else 0)


@pytest.mark.parametrize("p8", [26, 128, 230])
def test_mask_keep_rate_is_binomial(p8):
    m = oracle.dropout_mask(99, 1, 0, 256, 512, p8)
    n = m.size
    keep = (256 - p8) / 256
    assert abs(m.mean() - keep) <= 5 * np.sqrt(keep * (1 - keep) / n)
    # rows and columns are not degenerate either
    assert m.mean(axis=1).std() < 0.1 and m.mean(axis=0).std() < 0.1


def test_mask_depends_on_seed_offset_and_head():
    a = oracle.dropout_mask(5, 0, 0, 64, 64, 128)
    for other in (oracle.dropout_mask(6, 0, 0, 64, 64, 128), oracle.dropout_mask(5, 1, 0, 64, 64, 128),
                  oracle.dropout_mask(5, 0, 1, 64, 64, 128)):
        assert 0.4 < (a != other).mean() < 0.6


def test_no_dropout_equals_plain_attention():
    rng = np.random.default_rng(1)
    q, k, v = rng.standard_normal((2, 3, 20, 8)), rng.standard_normal((2, 3, 30, 8)), rng.standard_normal((2, 3, 30, 8))
    for causal in (False, True):
        o0, l0 = oracle.attention(q, k, v, 0.3, causal)
        o1, l1 = oracle.attention_dropout(q, k, v, 0.3, causal, 0.0, 7, 0)
        assert np.abs(o0 - o1).max() <= 1e-15 and np.abs(l0 - l1).max() <= 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_attention_definition(causal):
    """O = rescale * (P o keep) V with P the pinned oracle's probabilities, and
    V = 1 gives O_i = rescale * sum of row i's kept probabilities."""
    rng = np.random.default_rng(2)
    q, k, v = rng.standard_normal((17, 6)), rng.standard_normal((25, 6)), rng.standard_normal((25, 6))
    p, seed, off = 0.3, 77, 9
    p8 = oracle.dropout_p8(p)
    keep = oracle.dropout_mask(seed, off, 0, 17, 25, p8).astype(float)
    _, lse_ref, P = oracle.attention(q, k, v, 0.5, causal, return_p=True)
    o, lse = oracle.attention_dropout(q, k, v, 0.5, causal, p, seed, off)
    assert np.abs(o - oracle.dropout_rescale(p8) * (P * keep) @ v).max() <= 1e-14
    assert np.abs(lse - lse_ref).max() <= 1e-14
    o1, _ = oracle.attention_dropout(q, k, np.ones_like(v), 0.5, causal, p, seed, off)
    assert np.abs(o1[:, 0] - oracle.dropout_rescale(p8) * (P * keep).sum(axis=1)).max() <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_gradients_match_differences(causal):
    rng = np.random.default_rng(3 + causal)
    n_q, n_kv, d, scale, p, seed, off = 6, 9, 4, 0.6, 0.4, 1234, 5
    q, k, v, g = (rng.standard_normal(s) for s in ((n_q, d), (n_kv, d), (n_kv, d), (n_q, d)))

    def loss(q_, k_, v_):
        o, _ = oracle.attention_dropout(q_, k_, v_, scale, causal, p, seed, off)
        return float((o * g).sum())

    got = oracle.backward_dropout(q, k, v, g, scale, causal, p, seed, off)
    eps = 1e-6
    for which, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            a, b = [q, k, v], [q, k, v]
            a[which], b[which] = xp, xm
            num[idx] = (loss(*a) - loss(*b)) / (2 * eps)
        assert np.abs(num - got[which]).max() <= 5e-8


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_selections_equal_the_full_result(causal):
    """Selected rows (attention) and selected heads (gradients) equal the
    corresponding parts of the whole computation, with the mask of the right
    slice and row."""
    rng = np.random.default_rng(7 + causal)
    B, H, n_q, n_kv, d = 2, 3, 23, 31, 5
    q, k, v, g = (rng.standard_normal((B, H, n, d)) for n in (n_q, n_kv, n_kv, n_q))
    args = (0.7, causal, 0.3, 99, 4)
    o, lse = oracle.attention_dropout(q, k, v, *args)
    rows = np.array([0, 5, 22, n_q + 3, 2 * n_q + 11, 5 * n_q + 22, 4 * n_q])
    o_r, lse_r = oracle.attention_dropout(q, k, v, *args, rows=rows)
    assert np.abs(o_r - o.reshape(-1, d)[rows]).max() <= 1e-15
    assert np.abs(lse_r - lse.reshape(-1)[rows]).max() <= 1e-15
    dq, dk, dv = oracle.backward_dropout(q, k, v, g, *args)
    heads = [4, 1]
    sq, sk, sv = oracle.backward_dropout(q, k, v, g, *args, heads=heads)
    for n, bh in enumerate(heads):
        b, h = divmod(bh, H)
        assert np.array_equal(sq[n], dq[b, h]) and np.array_equal(sk[n], dk[b, h]) and np.array_equal(sv[n], dv[b, h])


def test_dropout_gradients_without_dropout_equal_plain():
    rng = np.random.default_rng(5)
    q, k, v, g = (rng.standard_normal(s) for s in ((7, 5), (11, 5), (11, 5), (7, 5)))
    a = oracle.backward(q, k, v, g, 0.4, True)
    b = oracle.backward_dropout(q, k, v, g, 0.4, True, 0.0, 3, 0)
    for x, y in zip(a, b):
        assert np.abs(x - y).max() <= 1e-14


# ---- planted mistakes ----

DROPOUT_MUTATIONS = [
    ("philox multiplier", "(uint64_t)0xD2511F53u * c0", "(uint64_t)0xD2511F57u * c0"),
    ("philox word order", "const uint32_t n1 = (uint32_t)p1;", "const uint32_t n1 = (uint32_t)p0;"),
    ("philox key bump", "k1 += 0xBB67AE85u;", "k1 += 0xBB67AE84u;"),
    ("mask byte index", "(out[i % 4] >> (8 * (j % 4)))", "(out[j % 4] >> (8 * (i % 4)))"),
    ("mask threshold", "byte >= (unsigned)p8 ? 1 : 0", "byte > (unsigned)p8 ? 1 : 0"),
    ("dropout forward rescale", "const double zij = rescale * exp(s[j] - m) / l;", "const double zij = exp(s[j] - m) / l;"),
    ("dropout dP unmasked", "const double dpij = keep[i * n_kv + j] ? rescale * dpt : 0.0;", "const double dpij = rescale * dpt;"),
    ("dropout dV unmasked", "const double zij = keep[i * n_kv + j] ? rescale * P[i * n_kv + j] : 0.0;",
     "const double zij = rescale * P[i * n_kv + j];"),
]


def _dropout_pins_pass(lib) -> bool:
    try:
        for ctr, key, out in PHILOX_KAT:
            if oracle.philox4x32_10(ctr, key, lib=lib) != list(out):
                return False
        # the mask against its definition on a 16 x 24 slice, with p8 equal to
        # one of the slice's bytes so that the boundary case occurs
        seed, off, bh = 0x1234_5678_9ABC_DEF0, 5, 3
        key = (seed & 0xFFFFFFFF, seed >> 32)
        byte = lambda i, j: (oracle.philox4x32_10((j // 4, i // 4, bh, off), key, lib=lib)[i % 4]
                             >> (8 * (j % 4))) & 0xFF
        p8 = max(1, byte(0, 0))
        m = oracle.dropout_mask(seed, off, bh, 16, 24, p8, lib=lib)
        for i in range(16):
            for j in range(24):
                if m[i, j] != (1 if byte(i, j) >= p8 else 0):
                    return False
        rng = np.random.default_rng(3)
        q, k, v, g = (rng.standard_normal(s) for s in ((6, 4), (9, 4), (9, 4), (6, 4)))
        p8 = oracle.dropout_p8(0.4)
        keep = oracle.dropout_mask(1234, 5, 0, 6, 9, p8, lib=lib).astype(float)
        _, _, P = oracle.attention(q, k, v, 0.6, True, return_p=True, lib=lib)
        o, _ = oracle.attention_dropout(q, k, v, 0.6, True, 0.4, 1234, 5, lib=lib)
        if np.abs(o - oracle.dropout_rescale(p8) * (P * keep) @ v).max() > 1e-14:
            return False
        got = oracle.backward_dropout(q, k, v, g, 0.6, True, 0.4, 1234, 5, lib=lib)

        def loss(q_, k_, v_):
            o_, _ = oracle.attention_dropout(q_, k_, v_, 0.6, True, 0.4, 1234, 5, lib=lib)
            return float((o_ * g).sum())
        eps = 1e-6
        for which, x in enumerate((q, k, v)):
            for idx in [(0, 0), (3, 2), (5, 3)]:
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                a, b = [q, k, v], [q, k, v]
                a[which], b[which] = xp, xm
                if abs((loss(*a) - loss(*b)) / (2 * eps) - got[which][idx]) > 5e-8:
                    return False
        return True
    except RuntimeError:
        return False


def test_dropout_pins_accept_the_oracle():
    assert _dropout_pins_pass(oracle.load())


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name,old,new", DROPOUT_MUTATIONS, ids=[m[0] for m in DROPOUT_MUTATIONS])
def test_planted_dropout_mistake_is_caught(name, old, new, tmp_path):
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, name
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(force=True, src=str(mutated), out=str(tmp_path / "libmut.so")))
    assert not _dropout_pins_pass(lib), "pins did not catch: " + name
