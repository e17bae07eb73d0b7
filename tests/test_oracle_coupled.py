"""Pins for the oracle's coupled and scalar gate forms (erase and write gate
one scalar beta per token and value head; with a scalar decay alpha as well):
the gradients of beta and alpha against central differences of the pinned
forward run on the broadcast gates, and the special case in which the coupled
form is the plain delta rule's."""
import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import rand_inputs


def test_expand_scalar_gates_broadcasts():
    rng = np.random.default_rng(31)
    alpha = rng.uniform(0.5, 1, (1, 3, 2)); beta = rng.uniform(0, 1, (1, 3, 2))
    a, b, w = oracle.expand_scalar_gates(alpha, beta, 4, 5, scalar_decay=True)
    assert a.shape == (1, 3, 2, 4) and b.shape == (1, 3, 2, 4) and w.shape == (1, 3, 2, 5)
    for i in range(4):
        np.testing.assert_array_equal(a[..., i], alpha)
        np.testing.assert_array_equal(b[..., i], beta)
    for j in range(5):
        np.testing.assert_array_equal(w[..., j], beta)


@pytest.mark.parametrize("scalar_decay", [False, True])
def test_backward_coupled_finite_differences(scalar_decay):
    """dbeta (and dalpha) against central differences of L = <dO, o> + <dS_T, S_T>
    with the forward run on the broadcast gates; dq, dk, dv, dS0 as well."""
    rng = np.random.default_rng(32 + scalar_decay)
    B, T, Hv, dk, dv = 1, 5, 2, 3, 2
    q, k, v, a, _, _, S0 = rand_inputs(rng, B, T, 1, Hv, dk, dv)
    if scalar_decay:
        a = rng.uniform(0.5, 1.0, (B, T, Hv))
    X = {"a": a, "b": rng.uniform(0.0, 1.0, (B, T, Hv)), "q": q, "v": v, "S0": S0}
    dO = rng.standard_normal((B, T, Hv, dv)); dST = rng.standard_normal((B, Hv, dk, dv))
    g = oracle.backward_coupled(q, k, v, X["a"], X["b"], S0, dO, dST, scalar_decay=scalar_decay)
    assert "dw" not in g

    def loss(**Y):
        if scalar_decay:
            A = np.repeat(Y["a"][..., None], dk, axis=-1)
        else:
            A = Y["a"]
        Bg = np.repeat(Y["b"][..., None], dk, axis=-1)
        W = np.repeat(Y["b"][..., None], dv, axis=-1)
        o, ST = oracle.forward(Y["q"], k, Y["v"], A, Bg, W, Y["S0"], nthreads=1)
        return float((o * dO).sum() + (ST * dST).sum())

    h = 1e-6
    for name, x in X.items():
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            Y = dict(X)
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            Y[name] = xp; lp = loss(**Y)
            Y[name] = xm; lm = loss(**Y)
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - g["d" + name]).max() / np.abs(fd).max()
        assert err < 1e-7, (name, err)


def test_coupled_unit_decay_is_delta_rule_gradient():
    """alpha = 1, beta = 1, one key channel and one value column, k_t = +-1,
    S0 = 0: the erase removes the whole old state, S_t = k_t v_t and
    o_t = q_t k_t v_t, and a state no longer reaches later tokens
    (dS_t/dS_{t-1} = 1 - beta k^2 = 0). So beta_t acts on token t alone:
    dS_t/dbeta_t = k_t v_t - k_t^2 S_{t-1}, giving
    dbeta_t = dO_t q_t (k_t v_t - k_{t-1} v_{t-1}), and
    dS_t/dalpha_t = (1 - beta_t k_t^2) S_{t-1} = 0 gives dalpha = 0."""
    T = 6
    rng = np.random.default_rng(33)
    k = rng.choice([-1.0, 1.0], T); q = rng.standard_normal(T); v = rng.standard_normal(T)
    dO = rng.standard_normal(T)
    r4 = lambda x: x.reshape(1, T, 1, 1)
    g = oracle.backward_coupled(r4(q), r4(k), r4(v), np.ones((1, T, 1)), np.ones((1, T, 1)), None, r4(dO), None,
                                scalar_decay=True)
    prev = np.concatenate([[0.0], (k * v)[:-1]])
    np.testing.assert_allclose(g["db"][0, :, 0], dO * q * (k * v - prev), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["da"][0, :, 0], 0.0, atol=1e-12)
