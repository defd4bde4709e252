"""Pins for the oracle's attention gradients (no GPU).

The pages give no derivative formulas, so the gradients are tied to things
other than the oracle's own formulas: central differences of the forward
(50-digit arithmetic on tiny inputs, and fp64 on the pinned forward oracle),
closed forms (one key; one visible key; equal keys), invariants of the
definition (softmax is unchanged by adding one vector to every key, so the
key gradients sum to zero; linearity in dO; V + c), and agreement between
selected-row/key and full evaluations.  A planted-mistake test checks that
these pins catch plausible slips in the C source.
"""
import shutil

import mpmath
import numpy as np
import pytest

import oracle

mpmath.mp.dps = 50


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _mp_loss(q, k, v, g, scale, causal):
    """sum_i dO_i . O_i with O from the plain definition, in 50 digits."""
    n_q, d, n_kv = len(q), len(q[0]), len(k)
    total = mpmath.mpf(0)
    for i in range(n_q):
        vis = range(min(i + 1, n_kv)) if causal else range(n_kv)
        s = [scale * mpmath.fsum(q[i][c] * k[j][c] for c in range(d)) for j in vis]
        e = [mpmath.exp(x) for x in s]
        z = mpmath.fsum(e)
        for c in range(d):
            oc = mpmath.fsum(e[t] * v[j][c] for t, j in enumerate(vis)) / z
            total += g[i][c] * oc
    return total


def _mp_grads(q, k, v, g, scale, causal, h=mpmath.mpf("1e-20")):
    """Central differences of the 50-digit loss (error ~h^2, far below fp64)."""
    to_mp = lambda a: [[mpmath.mpf(float(x)) for x in row] for row in a]
    Q, K, V, G = to_mp(q), to_mp(k), to_mp(v), to_mp(g)
    sc = mpmath.mpf(float(scale))
    out = []
    for X in (Q, K, V):
        grad = np.zeros((len(X), len(X[0])))
        for a in range(len(X)):
            for c in range(len(X[0])):
                x0 = X[a][c]
                X[a][c] = x0 + h
                lp = _mp_loss(Q, K, V, G, sc, causal)
                X[a][c] = x0 - h
                lm = _mp_loss(Q, K, V, G, sc, causal)
                X[a][c] = x0
                grad[a, c] = float((lp - lm) / (2 * h))
        out.append(grad)
    return out


@pytest.mark.parametrize("n_q,n_kv,d,causal", [(3, 4, 2, False), (4, 3, 2, True), (2, 5, 3, True),
                                               (1, 1, 2, False)])
def test_gradients_match_50_digit_differences(n_q, n_kv, d, causal):
    rng = np.random.default_rng(100 + n_q * 7 + n_kv)
    q, k, v, g = _rand(rng, n_q, d), _rand(rng, n_kv, d), _rand(rng, n_kv, d), _rand(rng, n_q, d)
    ref = _mp_grads(q, k, v, g, 0.9, causal)
    got = oracle.backward(q, k, v, g, 0.9, causal)
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert np.abs(a - b).max() <= 1e-13, name


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_fp64_differences(causal):
    """Central differences of the (separately pinned) fp64 forward oracle on
    a larger tile, including a ragged causal shape."""
    rng = np.random.default_rng(7 + causal)
    n_q, n_kv, d, scale = 6, 9, 4, 0.6
    q, k, v, g = _rand(rng, n_q, d), _rand(rng, n_kv, d), _rand(rng, n_kv, d), _rand(rng, n_q, d)

    def loss(q_, k_, v_):
        o, _ = oracle.attention(q_, k_, v_, scale, causal)
        return float((o * g).sum())

    got = oracle.backward(q, k, v, g, scale, causal)
    eps = 1e-6
    for which, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.abs(num - got[which]).max() <= 2e-8


def test_single_key_closed_form():
    """One key: O_i = v_0 whatever Q and K are, so dQ = dK = 0, dV_0 = sum_i dO_i."""
    rng = np.random.default_rng(3)
    q, k, v, g = _rand(rng, 5, 4), _rand(rng, 1, 4), _rand(rng, 1, 4), _rand(rng, 5, 4)
    for causal in (False, True):
        dq, dk, dv = oracle.backward(q, k, v, g, 1.3, causal)
        assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0
        assert np.abs(dv[0] - g.sum(axis=0)).max() <= 1e-14


def test_causal_first_row_has_no_query_gradient():
    """Causal row 0 sees only key 0 (P = 1), so dQ_0 = 0 and key 0 gets dV += dO_0."""
    rng = np.random.default_rng(4)
    q, k, v, g = _rand(rng, 1, 3), _rand(rng, 6, 3), _rand(rng, 6, 3), _rand(rng, 1, 3)
    dq, dk, dv = oracle.backward(q, k, v, g, 0.7, True)
    assert np.abs(dq).max() <= 1e-15
    assert np.abs(dv[0] - g[0]).max() <= 1e-15 and np.abs(dv[1:]).max() == 0 and np.abs(dk).max() <= 1e-15


def test_equal_keys_give_zero_query_gradient():
    """Equal key rows make every row's weights uniform whatever q is: dQ = 0."""
    rng = np.random.default_rng(5)
    q, g = _rand(rng, 4, 3), _rand(rng, 4, 3)
    k = np.tile(_rand(rng, 1, 3), (7, 1))
    v = _rand(rng, 7, 3)
    dq, _, dv = oracle.backward(q, k, v, g, 0.8, False)
    assert np.abs(dq).max() <= 1e-14
    # and dV_j = sum_i dO_i / n_kv
    assert np.abs(dv - g.sum(axis=0) / 7).max() <= 1e-14


def test_single_query_dv_is_weighted_dout():
    """N_q = 1: dV_j = P_0j dO_0 with P the (pinned) forward probabilities."""
    rng = np.random.default_rng(6)
    q, k, v, g = _rand(rng, 1, 4), _rand(rng, 9, 4), _rand(rng, 9, 4), _rand(rng, 1, 4)
    _, _, p = oracle.attention(q, k, v, 0.5, False, return_p=True)
    _, _, dv = oracle.backward(q, k, v, g, 0.5, False)
    assert np.abs(dv - p[0][:, None] * g[0][None, :]).max() <= 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero(causal):
    """softmax(q.(k_j + c)) = softmax(q.k_j): the loss is invariant under one
    shift of all keys, so sum_j dK_j = 0."""
    rng = np.random.default_rng(8 + causal)
    q, k, v, g = _rand(rng, 7, 5), _rand(rng, 11, 5), _rand(rng, 11, 5), _rand(rng, 7, 5)
    _, dk, _ = oracle.backward(q, k, v, g, 0.4, causal)
    assert np.abs(dk.sum(axis=0)).max() <= 1e-13


def test_linear_in_dout_and_invariant_to_value_shift():
    rng = np.random.default_rng(10)
    q, k, v = _rand(rng, 5, 3), _rand(rng, 8, 3), _rand(rng, 8, 3)
    g1, g2 = _rand(rng, 5, 3), _rand(rng, 5, 3)
    a = oracle.backward(q, k, v, g1, 0.9, True)
    b = oracle.backward(q, k, v, g2, 0.9, True)
    c = oracle.backward(q, k, v, g1 + 2 * g2, 0.9, True)
    for x, y, z in zip(a, b, c):
        assert np.abs(x + 2 * y - z).max() <= 1e-13
    assert all(np.abs(x).max() == 0 for x in oracle.backward(q, k, v, 0 * g1, 0.9, True))
    # V + c shifts O by c: dQ, dK, dV do not change
    s = oracle.backward(q, k, v + np.array([1.5, -2.0, 0.25]), g1, 0.9, True)
    for x, y in zip(a, s):
        assert np.abs(x - y).max() <= 1e-13


def test_selected_rows_and_keys_match_full():
    rng = np.random.default_rng(11)
    B, H, n_q, n_kv, d = 2, 3, 13, 17, 4
    q, g = _rand(rng, B, H, n_q, d), _rand(rng, B, H, n_q, d)
    k, v = _rand(rng, B, H, n_kv, d), _rand(rng, B, H, n_kv, d)
    dq, dk, dv = oracle.backward(q, k, v, g, 0.5, True)
    rows = np.array([0, 5, 12, 40, 77])
    keys = np.array([3, 16, 50, 101])
    sq, sk, sv = oracle.backward(q, k, v, g, 0.5, True, rows=rows, keys=keys)
    assert np.array_equal(sq, dq.reshape(-1, d)[rows])
    assert np.array_equal(sk, dk.reshape(-1, d)[keys])
    assert np.array_equal(sv, dv.reshape(-1, d)[keys])


# ---- planted mistakes: each variant of the C source must fail a pin ----

BWD_MUTATIONS = [
    ("dS without the D term", "const double dsij = pij * (dpij - D[i]);", "const double dsij = pij * dpij;"),
    ("dS sign", "const double dsij = pij * (dpij - D[i]);", "const double dsij = pij * (D[i] - dpij);"),
    ("D without P", "Di += pij * dpij;", "Di += dpij;"),
    ("dV from dS", "if (dvj) dvj[c] += pij * dout[i * d + c];", "if (dvj) dvj[c] += dsij * dout[i * d + c];"),
    ("dK from k", "if (dkj) dkj[c] += dsij * q[i * d + c];", "if (dkj) dkj[c] += dsij * k[j * d + c];"),
    ("dQ scale dropped", "for (int64_t c = 0; c < d; ++c) dqi[c] *= scale;", ""),
    ("dK causal off by one", "if (j >= visible_keys(i, n_kv, causal)) continue;",
     "if (j > visible_keys(i, n_kv, causal)) continue;"),
    ("dP with k", "for (int64_t c = 0; c < d; ++c) dpij += dout[i * d + c] * v[j * d + c];\n                Di",
     "for (int64_t c = 0; c < d; ++c) dpij += dout[i * d + c] * k[j * d + c];\n                Di"),
]


def _bwd_pins_pass(lib) -> bool:
    """A compact subset of the pins above, run against a given library."""
    rng = np.random.default_rng(123)
    try:
        for causal in (False, True):
            q, k, v, g = _rand(rng, 3, 2), _rand(rng, 4, 2), _rand(rng, 4, 2), _rand(rng, 3, 2)
            ref = _mp_grads(q, k, v, g, 0.9, causal)
            got = oracle.backward(q, k, v, g, 0.9, causal, lib=lib)
            if any(np.abs(a - b).max() > 1e-12 for a, b in zip(got, ref)):
                return False
        return True
    except RuntimeError:
        return False


def test_bwd_pins_accept_the_oracle():
    assert _bwd_pins_pass(oracle.load())


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name,old,new", BWD_MUTATIONS, ids=[m[0] for m in BWD_MUTATIONS])
def test_planted_backward_mistake_is_caught(name, old, new, tmp_path):
    src = open(oracle._SRC).read()
    assert src.count(old) >= 1, name
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(force=True, src=str(mutated), out=str(tmp_path / "libmut.so")))
    assert not _bwd_pins_pass(lib), "pins did not catch: " + name
