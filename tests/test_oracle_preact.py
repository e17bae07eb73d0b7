"""Pins for the oracle's gate activations (decay a = exp(-softplus(x)), erase
and write gates b, w = sigmoid(x)), checked against closed-form values,
identities of the two functions and scipy's logistic function."""
import numpy as np
import pytest
from scipy.special import expit

import oracle
from tests.test_oracle_pins import rand_inputs


def test_activation_closed_forms():
    z = np.zeros(3)
    a, b, w = oracle.activate_gates(z, z, z)
    np.testing.assert_array_equal(a, 0.5)
    np.testing.assert_array_equal(b, 0.5)
    x = np.full(2, np.log(3.0))  # e^x = 3: a = 1/4, sigmoid = 3/4
    a, b, w = oracle.activate_gates(x, x, -x)
    np.testing.assert_allclose(a, 0.25, rtol=1e-15)
    np.testing.assert_allclose(b, 0.75, rtol=1e-15)
    np.testing.assert_allclose(w, 0.25, rtol=1e-15)


def test_activation_identities_and_library():
    x = np.linspace(-30, 30, 601)
    a, b, w = oracle.activate_gates(x, x, x)
    np.testing.assert_allclose(a + b, 1.0, rtol=0, atol=2e-16)            # 1/(1+e^x) + 1/(1+e^-x) = 1
    np.testing.assert_allclose(b, expit(x), rtol=4e-15, atol=0)           # sigmoid
    np.testing.assert_allclose(a, expit(-x), rtol=1e-14, atol=0)          # exp(-softplus(x)) = sigmoid(-x)
    np.testing.assert_allclose(np.log(a), -np.log1p(np.exp(x)), rtol=1e-14, atol=1e-16)  # log a = -softplus(x)
    np.testing.assert_array_equal(w, b)
    big = np.array([-800.0, 800.0])
    a, b, _ = oracle.activate_gates(big, big, big)
    np.testing.assert_array_equal(a, [1.0, 0.0])
    np.testing.assert_array_equal(b, [0.0, 1.0])


def test_forward_preact_is_forward_of_activated_gates():
    rng = np.random.default_rng(21)
    q, k, v, _, _, _, S0 = rand_inputs(rng, 1, 9, 1, 2, 4, 3)
    xa = rng.standard_normal((1, 9, 2, 4)); xb = rng.standard_normal((1, 9, 2, 4)); xw = rng.standard_normal((1, 9, 2, 3))
    o1, s1 = oracle.forward_preact(q, k, v, xa, xb, xw, S0)
    o2, s2 = oracle.forward(q, k, v, expit(-xa), expit(xb), expit(xw), S0)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s1, s2, rtol=1e-13, atol=1e-14)


def test_backward_preact_finite_differences():
    """The pre-activation gradients against central differences of
    L = <dO, o> + <dS_T, S_T> through forward_preact."""
    rng = np.random.default_rng(22)
    B, T, Hv, dk, dv = 1, 5, 2, 3, 2
    q, k, v, _, _, _, S0 = rand_inputs(rng, B, T, 1, Hv, dk, dv)
    X = {"a": rng.standard_normal((B, T, Hv, dk)) - 1.0, "b": rng.standard_normal((B, T, Hv, dk)),
         "w": rng.standard_normal((B, T, Hv, dv))}
    dO = rng.standard_normal((B, T, Hv, dv)); dST = rng.standard_normal((B, Hv, dk, dv))
    g = oracle.backward_preact(q, k, v, X["a"], X["b"], X["w"], S0, dO, dST)

    def loss(**Y):
        o, ST = oracle.forward_preact(q, k, v, Y["a"], Y["b"], Y["w"], S0, nthreads=1)
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
