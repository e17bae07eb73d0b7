"""Pins for the oracle's backward pass (gradients of the recurrence).

The pages define no backward pass: it is the derivative of the forward map,
whose oracle is pinned in ``test_oracle_pins.py``. Each pin here checks the
backward against something other than itself: central finite differences of
the pinned forward, closed-form gradients of causal linear attention (and of
its decay and erase gate at a = 1, b = 0), the grouped-head sum, and the
zero-length case. ``test_pins_catch_backward_mutant`` plants one mistake at a
time in a copy of the oracle's backward and shows that a pin catches it.
"""
import functools

import numpy as np
import pytest

import oracle
from tests.mutant_build import build_mutant
from tests.test_oracle_pins import rand_inputs


def _loss_grads(rng, B, T, Hv, dk, dv):
    dO = rng.standard_normal((B, T, Hv, dv))
    dST = rng.standard_normal((B, Hv, dk, dv))
    return dO, dST


# ----------------------------------------------------------------------------- pins

def pin_finite_differences(fwd, bwd):
    """Every gradient against central differences of L = <dO, o> + <dS_T, S_T>
    (fp64, step 1e-6: truncation and rounding error near 1e-9 relative)."""
    rng = np.random.default_rng(11)
    B, T, Hqk, Hv, dk, dv = 2, 5, 1, 2, 3, 2
    q, k, v, a, b, w, S0 = rand_inputs(rng, B, T, Hqk, Hv, dk, dv)
    dO, dST = _loss_grads(rng, B, T, Hv, dk, dv)
    g = bwd(q, k, v, a, b, w, S0, dO, dST)
    X = dict(q=q, k=k, v=v, a=a, b=b, w=w, S0=S0)

    def loss(**Y):
        o, ST = fwd(Y["q"], Y["k"], Y["v"], Y["a"], Y["b"], Y["w"], Y["S0"], nthreads=1)
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
        assert err < 1e-7, f"d{name}: {err:.2e} from finite differences"


def pin_linear_attention_gradients(fwd, bwd):
    """a = 1, b = 0, w = 1, S0 = 0: o_t = sum_{s<=t} (q_t.k_s) v_s, so
    dq_t = sum_{s<=t} (dO_t.v_s) k_s, dk_s = sum_{t>=s} (dO_t.v_s) q_t,
    dv_s = dw_s / v_s = sum_{t>=s} (q_t.k_s) dO_t (no dS_T)."""
    rng = np.random.default_rng(12)
    T, dk, dv = 9, 4, 3
    q = rng.standard_normal((T, dk)); k = rng.standard_normal((T, dk)); v = rng.standard_normal((T, dv))
    dO = rng.standard_normal((T, dv))
    r4 = lambda x: x.reshape(1, T, 1, -1)
    g = bwd(r4(q), r4(k), r4(v), np.ones((1, T, 1, dk)), np.zeros((1, T, 1, dk)), np.ones((1, T, 1, dv)),
            None, r4(dO), None)
    mask = np.tril(np.ones((T, T)))            # [t, s]: s <= t
    P = (dO @ v.T) * mask                      # P[t, s] = dO_t . v_s
    A = (q @ k.T) * mask                       # A[t, s] = q_t . k_s
    np.testing.assert_allclose(g["dq"][0, :, 0], P @ k, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dk"][0, :, 0], P.T @ q, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dv"][0, :, 0], A.T @ dO, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dw"][0, :, 0], (A.T @ dO) * v, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dS0"][0, 0], q.T @ dO, rtol=1e-12, atol=1e-12)


def pin_decay_and_erase_gradients_at_identity(fwd, bwd):
    """At a = 1, b = 0, w = 1, S0 = 0 (linear attention) the decay and erase
    gradients have closed forms: a_r scales every k_s v_s^T with s < r <= t, so
    da_r[i] = sum_{t>=r} sum_{s<r} q_t[i] k_s[i] (dO_t.v_s); the erase at
    token r removes b_r*k_r times the read r_r = sum_{s<r} (k_s.k_r) v_s, so
    db_r[i] = -k_r[i] sum_{t>=r} q_t[i] (dO_t.r_r)."""
    rng = np.random.default_rng(13)
    T, dk, dv = 8, 3, 4
    q = rng.standard_normal((T, dk)); k = rng.standard_normal((T, dk)); v = rng.standard_normal((T, dv))
    dO = rng.standard_normal((T, dv))
    r4 = lambda x: x.reshape(1, T, 1, -1)
    g = bwd(r4(q), r4(k), r4(v), np.ones((1, T, 1, dk)), np.zeros((1, T, 1, dk)), np.ones((1, T, 1, dv)),
            None, r4(dO), None)
    da = np.zeros((T, dk)); db = np.zeros((T, dk))
    for r in range(T):
        rr = sum(((k[s] @ k[r]) * v[s] for s in range(r)), np.zeros(dv))
        for t in range(r, T):
            for s in range(r):
                da[r] += q[t] * k[s] * (dO[t] @ v[s])
            db[r] -= k[r] * q[t] * (dO[t] @ rr)
    np.testing.assert_allclose(g["da"][0, :, 0], da, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["db"][0, :, 0], db, rtol=1e-11, atol=1e-12)


def pin_grouped_heads_sum(fwd, bwd):
    """Two value heads sharing one query/key head: the shared head's dq and dk
    are the sums of the gradients of the two heads run as separate problems."""
    rng = np.random.default_rng(14)
    B, T, dk, dv = 1, 6, 3, 2
    q, k, v, a, b, w, S0 = rand_inputs(rng, B, T, 1, 2, dk, dv)
    dO, dST = _loss_grads(rng, B, T, 2, dk, dv)
    g = bwd(q, k, v, a, b, w, S0, dO, dST)
    dq = np.zeros_like(q); dk_ = np.zeros_like(k)
    for h in range(2):
        sl = slice(h, h + 1)
        gh = bwd(q, k, v[:, :, sl], a[:, :, sl], b[:, :, sl], w[:, :, sl], S0[:, sl], dO[:, :, sl], dST[:, sl])
        dq += gh["dq"]; dk_ += gh["dk"]
        np.testing.assert_allclose(g["dv"][:, :, sl], gh["dv"], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(g["da"][:, :, sl], gh["da"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(g["dq"], dq, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(g["dk"], dk_, rtol=1e-13, atol=1e-14)


BWD_PINS = [pin_finite_differences, pin_linear_attention_gradients, pin_decay_and_erase_gradients_at_identity,
            pin_grouped_heads_sum]


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_backward_pin(pin):
    pin(oracle.forward, oracle.backward)


def test_backward_zero_length():
    """No tokens: the state passes through, so dS0 = dS_T and nothing else exists."""
    rng = np.random.default_rng(15)
    z = lambda *s: np.zeros(s)
    dST = rng.standard_normal((2, 2, 3, 4))
    g = oracle.backward(z(2, 0, 1, 3), z(2, 0, 1, 3), z(2, 0, 2, 4), z(2, 0, 2, 3), z(2, 0, 2, 3), z(2, 0, 2, 4),
                        None, z(2, 0, 2, 4), dST)
    np.testing.assert_array_equal(g["dS0"], dST)
    assert g["dq"].shape == (2, 0, 1, 3) and g["dv"].shape == (2, 0, 2, 4)


def test_backward_null_upstream_state_gradient_is_zero():
    rng = np.random.default_rng(16)
    q, k, v, a, b, w, S0 = rand_inputs(rng, 1, 4, 1, 1, 3, 2)
    dO = rng.standard_normal(v.shape)
    g0 = oracle.backward(q, k, v, a, b, w, S0, dO, None)
    g1 = oracle.backward(q, k, v, a, b, w, S0, dO, np.zeros((1, 1, 3, 2)))
    for key in g0:
        np.testing.assert_array_equal(g0[key], g1[key])


# ----------------------------------------------------------------------------- planted mistakes

BWD_MUTANTS = [
    ("bwd_read_prev_state", "for (int j = 0; j < dv; ++j) s += St[(size_t)i * dv + j] * dOt[j];",
     "for (int j = 0; j < dv; ++j) s += Sp[(size_t)i * dv + j] * dOt[j];"),
    ("bwd_no_query_adjoint", "for (int j = 0; j < dv; ++j) L[(size_t)i * dv + j] += qt[i] * dOt[j];",
     "for (int j = 0; j < dv; ++j) L[(size_t)i * dv + j] += 0.0 * qt[i] * dOt[j];"),
    ("bwd_erase_read_sign", "dr[j] -= L[(size_t)i * dv + j] * eb;", "dr[j] += L[(size_t)i * dv + j] * eb;"),
    ("bwd_dv_ungated", "dvt[j] = du[j] * wt[j];", "dvt[j] = du[j];"),
    ("bwd_db_without_key", "dbt[i] = de * kt[i];", "dbt[i] = de;"),
    ("bwd_dk_no_erase_term", "dkt[i] = kw + de * bt[i];", "dkt[i] = kw;"),
    ("bwd_dk_read_undecayed", "s += at[i] * Sp[(size_t)i * dv + j] * dr[j];", "s += Sp[(size_t)i * dv + j] * dr[j];"),
    ("bwd_no_read_adjoint", "for (int j = 0; j < dv; ++j) L[(size_t)i * dv + j] += kt[i] * dr[j];",
     "for (int j = 0; j < dv; ++j) L[(size_t)i * dv + j] += 0.0 * kt[i] * dr[j];"),
    ("bwd_adjoint_not_decayed", "for (int j = 0; j < dv; ++j) L[(size_t)i * dv + j] *= at[i];",
     "for (int j = 0; j < dv; ++j) L[(size_t)i * dv + j] *= 1.0;"),
    ("bwd_da_current_state", "s += L[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];",
     "s += L[(size_t)i * dv + j] * St[(size_t)i * dv + j];"),
]


@pytest.mark.parametrize("mut", BWD_MUTANTS, ids=lambda m: m[0])
def test_pins_catch_backward_mutant(mut, tmp_path_factory):
    name, old, new = mut
    d = str(tmp_path_factory.mktemp("bwd_mutants"))
    lib = oracle.bind(build_mutant(name, old, new, d))
    fwd = functools.partial(oracle.forward, lib=lib)
    bwd = functools.partial(oracle.backward, lib=lib)
    caught = []
    for pin in BWD_PINS:
        try:
            pin(fwd, bwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every backward pin"
