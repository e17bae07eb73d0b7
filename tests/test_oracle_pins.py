"""Pins for the fp64 oracle: each checks it against something other than itself.

Every pin is a function of a forward callable with the oracle's signature, so
that ``test_oracle_mutants.py`` can run the same pins against deliberately
broken copies of the oracle and show that each planted mistake is caught.
"""
import os
import re

import numpy as np
import pytest

from tests.chunk_algebra import chunked_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "delta_rule_worked_example.txt")


# ----------------------------------------------------------------------------- helpers

def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_inputs(rng, B, T, Hqk, Hv, dk, dv, with_s0=True, a_lo=0.3):
    q = _unit(rng.standard_normal((B, T, Hqk, dk)))
    k = _unit(rng.standard_normal((B, T, Hqk, dk)))
    v = rng.standard_normal((B, T, Hv, dv))
    a = rng.uniform(a_lo, 1.0, (B, T, Hv, dk))
    b = rng.uniform(0.0, 1.0, (B, T, Hv, dk))
    w = rng.uniform(0.0, 1.0, (B, T, Hv, dv))
    S0 = rng.standard_normal((B, Hv, dk, dv)) * 0.5 if with_s0 else None
    return q, k, v, a, b, w, S0


def parse_golden(path=GOLDEN):
    cases, cur = [], None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("case "):
                cur = {"name": line[5:].strip()}
                cases.append(cur)
                continue
            key, val = line.split(":", 1)
            if key == "source":
                cur[key] = val.strip()
                continue
            rows = [r for r in val.split(";")]
            arr = np.array([[float(x) for x in r.split()] for r in rows])
            cur[key] = arr if arr.shape[0] > 1 else arr[0]
    return cases


def one_step(fwd, S0, q, k, v, a, b, w):
    """Run one token through `fwd` on a single head."""
    dk, dv = S0.shape
    r4 = lambda x: np.asarray(x, dtype=np.float64).reshape(1, 1, 1, -1)
    o, ST = fwd(r4(q), r4(k), r4(v), r4(a), r4(b), r4(w), S0.reshape(1, 1, dk, dv))
    return o[0, 0, 0], ST[0, 0]


# ----------------------------------------------------------------------------- pins

def pin_worked_example(fwd):
    """Every value the delta-rule tutorial prints for its 2x2 example."""
    cases = parse_golden()
    assert len(cases) >= 6
    for c in cases:
        S0 = c["S0"]
        if "expect_kread_before" in c:  # the fixture's own arithmetic: k^T S0
            np.testing.assert_array_equal(c["k"] @ S0, c["expect_kread_before"])
        if "expect_qread_before" in c:
            np.testing.assert_array_equal(c["q"] @ S0, c["expect_qread_before"])
        gate = lambda g, n: np.full(n, float(np.atleast_1d(g)[0]))
        o, S1 = one_step(fwd, S0, c["q"], c["k"], c["v"], np.ones(2), gate(c["b"], 2), gate(c["w"], 2))
        if "expect_S1" in c:
            np.testing.assert_allclose(S1, c["expect_S1"], rtol=0, atol=1e-15, err_msg=c["name"])
        if "expect_kread_after" in c:
            np.testing.assert_allclose(c["k"] @ S1, c["expect_kread_after"], rtol=0, atol=1e-15,
                                       err_msg=c["name"])
        np.testing.assert_allclose(o, c["expect_o"], rtol=0, atol=1e-15, err_msg=c["name"])


def pin_linear_attention_closed_form(fwd):
    """a=1, b=0, w=1, S0=0: o_t = sum_{s<=t} (q_t . k_s) v_s and S_T = sum_s k_s v_s^T
    (tutorial introduction: accumulating outer products equals the score-weighted sum)."""
    rng = np.random.default_rng(11)
    B, T, Hqk, Hv, dk, dv = 2, 23, 2, 4, 5, 3
    q, k, v, _, _, _, _ = rand_inputs(rng, B, T, Hqk, Hv, dk, dv, with_s0=False)
    q = rng.standard_normal(q.shape)  # the closed form needs no normalisation
    k = rng.standard_normal(k.shape)
    ones_k = np.ones((B, T, Hv, dk))
    o, ST = fwd(q, k, v, ones_k, np.zeros_like(ones_k), np.ones((B, T, Hv, dv)), None)
    G = Hv // Hqk
    mask = np.tril(np.ones((T, T)))
    for n in range(B):
        for h in range(Hv):
            qh, kh, vh = q[n, :, h // G], k[n, :, h // G], v[n, :, h]
            scores = (qh @ kh.T) * mask
            np.testing.assert_allclose(o[n, :, h], scores @ vh, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(ST[n, h], kh.T @ vh, rtol=1e-12, atol=1e-12)


def pin_zero_difference_invariant(fwd):
    """a=1, b=w=beta uniform, unit key, v equal to what the key already reads:
    the state does not change (tutorial, add-or-correct section)."""
    rng = np.random.default_rng(12)
    dk, dv = 6, 4
    for beta in (1.0, 0.5, 0.2):
        S0 = rng.standard_normal((dk, dv))
        k = _unit(rng.standard_normal(dk))
        v = S0.T @ k
        q = rng.standard_normal(dk)
        o, S1 = one_step(fwd, S0, q, k, v, np.ones(dk), np.full(dk, beta), np.full(dv, beta))
        np.testing.assert_allclose(S1, S0, rtol=0, atol=1e-14)
        np.testing.assert_allclose(o, S0.T @ q, rtol=0, atol=1e-14)


def pin_query_change_identity(fwd):
    """a=1, b=w=beta: a query's read changes by beta (q . k) (v - r) (tutorial,
    effect-on-other-lookups section)."""
    rng = np.random.default_rng(13)
    dk, dv = 7, 5
    for beta in (1.0, 0.5, 0.3):
        S0 = rng.standard_normal((dk, dv))
        k = _unit(rng.standard_normal(dk))
        q = rng.standard_normal(dk)
        v = rng.standard_normal(dv)
        o, _ = one_step(fwd, S0, q, k, v, np.ones(dk), np.full(dk, beta), np.full(dv, beta))
        r = S0.T @ k
        np.testing.assert_allclose(o - S0.T @ q, beta * (q @ k) * (v - r), rtol=1e-12, atol=1e-13)


def pin_key_read_identity_channel_gates(fwd):
    """Unit key, general channel-wise a, b, w: after the step the key reads
    (1 - sum_i b_i k_i^2) r + w * v, with r the key read of the decayed state.
    This fixes where decay, erase gate (key axis) and write gate (value axis) sit;
    with b = w = beta it is the tutorial's beta-section statement."""
    rng = np.random.default_rng(14)
    dk, dv = 8, 5
    for _ in range(5):
        S0 = rng.standard_normal((dk, dv))
        k = _unit(rng.standard_normal(dk))
        a = rng.uniform(0.2, 1.0, dk)
        b = rng.uniform(0.0, 1.0, dk)
        w = rng.uniform(0.0, 1.0, dv)
        v = rng.standard_normal(dv)
        o, S1 = one_step(fwd, S0, k, k, v, a, b, w)  # q = k: the output is the key read
        r = (a[:, None] * S0).T @ k
        expect = (1.0 - np.sum(b * k * k)) * r + w * v
        np.testing.assert_allclose(o, expect, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(k @ S1, expect, rtol=1e-12, atol=1e-13)


def pin_decay_only(fwd):
    """b=0, w=0: the state only decays, S_t = diag(prod_{s<=t} a_s) S0 (key-axis rows)."""
    rng = np.random.default_rng(15)
    B, T, Hqk, Hv, dk, dv = 1, 9, 1, 2, 6, 3
    q, k, v, a, _, _, S0 = rand_inputs(rng, B, T, Hqk, Hv, dk, dv)
    o, ST = fwd(q, k, v, a, np.zeros_like(a), np.zeros_like(v), S0)
    for h in range(Hv):
        cum = np.cumprod(a[0, :, h], axis=0)  # [T, dk]
        np.testing.assert_allclose(ST[0, h], cum[-1][:, None] * S0[0, h], rtol=1e-13, atol=1e-15)
        for t in range(T):
            np.testing.assert_allclose(o[0, t, h], (cum[t][:, None] * S0[0, h]).T @ q[0, t, 0],
                                       rtol=1e-12, atol=1e-14)


def pin_delta_rule_reduction(fwd):
    """a=1 and b=w=beta_t on every channel: the delta rule S + beta k (v - S^T k)^T
    of the tutorial's beta section, stepped token by token with a scalar beta."""
    rng = np.random.default_rng(16)
    T, dk, dv = 12, 5, 4
    q = _unit(rng.standard_normal((T, dk)))
    k = _unit(rng.standard_normal((T, dk)))
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.0, 1.0, T)
    S0 = rng.standard_normal((dk, dv))
    o, ST = fwd(q[None, :, None], k[None, :, None], v[None, :, None], np.ones((1, T, 1, dk)),
                np.repeat(beta[None, :, None, None], dk, axis=3),
                np.repeat(beta[None, :, None, None], dv, axis=3), S0[None, None])
    S = S0.copy()
    for t in range(T):
        e = v[t] - S.T @ k[t]
        S = S + beta[t] * np.outer(k[t], e)
        np.testing.assert_allclose(o[0, t, 0], S.T @ q[t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ST[0, 0], S, rtol=1e-12, atol=1e-13)


def pin_gated_deltanet_reduction(fwd):
    """Scalar decay alpha_t and b=w=beta_t: Gated DeltaNet, written in product form
    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T (the coupled-gate
    predecessor the tilnote post describes)."""
    rng = np.random.default_rng(17)
    T, dk, dv = 10, 4, 6
    q = _unit(rng.standard_normal((T, dk)))
    k = _unit(rng.standard_normal((T, dk)))
    v = rng.standard_normal((T, dv))
    alpha = rng.uniform(0.5, 1.0, T)
    beta = rng.uniform(0.0, 1.0, T)
    o, ST = fwd(q[None, :, None], k[None, :, None], v[None, :, None],
                np.repeat(alpha[None, :, None, None], dk, axis=3),
                np.repeat(beta[None, :, None, None], dk, axis=3),
                np.repeat(beta[None, :, None, None], dv, axis=3), None)
    S = np.zeros((dk, dv))
    for t in range(T):
        S = alpha[t] * (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ S + beta[t] * np.outer(k[t], v[t])
        np.testing.assert_allclose(o[0, t, 0], S.T @ q[t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ST[0, 0], S, rtol=1e-12, atol=1e-13)


def pin_chunked_agreement(fwd):
    """Brute force: the chunk-parallel fp64 form agrees with the stepwise oracle at
    several chunk lengths, including a ragged last chunk."""
    rng = np.random.default_rng(18)
    B, T, Hqk, Hv, dk, dv = 2, 37, 2, 4, 6, 5
    q, k, v, a, b, w, S0 = rand_inputs(rng, B, T, Hqk, Hv, dk, dv)
    o, ST = fwd(q, k, v, a, b, w, S0)
    for C in (1, 4, 8, 16):
        oc, Sc = chunked_forward(q, k, v, a, b, w, S0, C)
        np.testing.assert_allclose(o, oc, rtol=1e-10, atol=1e-12, err_msg=f"C={C}")
        np.testing.assert_allclose(ST, Sc, rtol=1e-10, atol=1e-12, err_msg=f"C={C}")


def pin_gqa_mapping(fwd):
    """V head h uses QK head h // (H_v / H_qk): equals running with q, k repeated per V head."""
    rng = np.random.default_rng(19)
    B, T, Hqk, Hv, dk, dv = 1, 11, 2, 4, 4, 3
    q, k, v, a, b, w, S0 = rand_inputs(rng, B, T, Hqk, Hv, dk, dv)
    o, ST = fwd(q, k, v, a, b, w, S0)
    rep = lambda x: np.repeat(x, Hv // Hqk, axis=2)
    o2, ST2 = fwd(rep(q), rep(k), v, a, b, w, S0)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(ST, ST2)


PINS = [pin_worked_example, pin_linear_attention_closed_form, pin_zero_difference_invariant,
        pin_query_change_identity, pin_key_read_identity_channel_gates, pin_decay_only,
        pin_delta_rule_reduction, pin_gated_deltanet_reduction, pin_chunked_agreement, pin_gqa_mapping]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin, oracle_mod):
    pin(oracle_mod.forward)


# ----------------------------------------------------------------------------- structure

def test_column_separability(oracle_mod):
    """Value columns of S evolve independently: a column subset gives the same columns."""
    rng = np.random.default_rng(20)
    q, k, v, a, b, w, S0 = rand_inputs(rng, 1, 15, 1, 2, 6, 8)
    o, ST = oracle_mod.forward(q, k, v, a, b, w, S0)
    cols = np.array([1, 4, 5, 7])
    o2, ST2 = oracle_mod.forward(q, k, v[..., cols], a, b, w[..., cols], S0[..., cols])
    np.testing.assert_array_equal(o[..., cols], o2)
    np.testing.assert_array_equal(ST[..., cols], ST2)


def test_split_prefill(oracle_mod):
    """[0, T) equals [0, T1) then [T1, T) started from S_T1 (the state is the checkpoint)."""
    rng = np.random.default_rng(21)
    q, k, v, a, b, w, S0 = rand_inputs(rng, 2, 30, 1, 2, 5, 4)
    o, ST = oracle_mod.forward(q, k, v, a, b, w, S0)
    T1 = 13
    cut = lambda x, s: x[:, s]
    o1, S1 = oracle_mod.forward(*(cut(x, slice(0, T1)) for x in (q, k, v, a, b, w)), S0)
    o2, S2 = oracle_mod.forward(*(cut(x, slice(T1, None)) for x in (q, k, v, a, b, w)), S1)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), o)
    np.testing.assert_array_equal(S2, ST)


def test_zero_length(oracle_mod):
    rng = np.random.default_rng(22)
    q, k, v, a, b, w, S0 = rand_inputs(rng, 2, 0, 1, 1, 4, 4)
    o, ST = oracle_mod.forward(q, k, v, a, b, w, S0)
    assert o.shape == (2, 0, 1, 4)
    np.testing.assert_array_equal(ST, S0)


def test_null_state_is_zero_state(oracle_mod):
    rng = np.random.default_rng(23)
    q, k, v, a, b, w, _ = rand_inputs(rng, 1, 9, 1, 1, 4, 4, with_s0=False)
    o1, S1 = oracle_mod.forward(q, k, v, a, b, w, None)
    o2, S2 = oracle_mod.forward(q, k, v, a, b, w, np.zeros((1, 1, 4, 4)))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def test_anchored_chunk_factorisation_matches_exact():
    """The chunk-start anchor factorisation (k_t gamma_t).(k_s / gamma_s) equals the
    exact per-channel ratio when the chunk's decay range is moderate; this is the
    algebra of the HIP prefill's Gram matrices."""
    rng = np.random.default_rng(24)
    q, k, v, a, b, w, S0 = rand_inputs(rng, 1, 64, 1, 2, 16, 8, a_lo=0.1)
    for C in (16, 32, 64):
        o1, S1 = chunked_forward(q, k, v, a, b, w, S0, C, anchored=False)
        o2, S2 = chunked_forward(q, k, v, a, b, w, S0, C, anchored=True)
        np.testing.assert_allclose(o1, o2, rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(S1, S2, rtol=1e-9, atol=1e-11)
