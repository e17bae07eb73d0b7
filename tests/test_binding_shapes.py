"""Host checks of the torch binding's argument validation (no GPU).

Every tensor's full shape must follow from (B, T, H_qk, H_v, d_k, d_v) of q
and v before anything reaches the library: the kernels index all tensors
from those sizes, so e.g. gates given per query/key head instead of per value
head would be read past their end. These tests relax only the binding's
"is a GPU tensor" check so that CPU tensors reach the shape checks, and make
every library entry fail if it were called.
"""
import pytest
import torch

import gated_delta_rule_83_amd as g


@pytest.fixture(autouse=True)
def host_tensors(monkeypatch):
    def check(t, name, dtype=None):
        if t is None:
            return
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")

    monkeypatch.setattr(g, "_check", check)

    def refuse(*a, **k):
        raise AssertionError("a mis-shaped call reached the library")

    for nm in ("gdn2_chunk_forward", "gdn2_chunk_forward_preact", "gdn2_chunk_forward_coupled",
               "gdn2_chunk_forward_scalar", "gdn2_chunk_forward_varlen_gates", "gdn2_decode_step_gates",
               "gdn2_chunk_backward", "gdn2_chunk_backward_varlen", "gdn2_chunk_backward_varlen_gates",
               "gdn2_chunk_backward_preact", "gdn2_chunk_backward_coupled", "gdn2_chunk_backward_scalar"):
        monkeypatch.setattr(g, nm, refuse)


B, T, HQK, HV, DK, DV = 2, 10, 2, 4, 16, 32


def problem(dtype=torch.float32):
    f = lambda *s, dt=torch.float32: torch.zeros(s, dtype=dt)
    return dict(q=f(B, T, HQK, DK, dt=dtype), k=f(B, T, HQK, DK, dt=dtype), v=f(B, T, HV, DV, dt=dtype),
                a=f(B, T, HV, DK), b=f(B, T, HV, DK), w=f(B, T, HV, DV), S0=f(B, HV, DK, DV))


@pytest.mark.parametrize("name,shape", [
    ("a", (B, T, HQK, DK)),        # gates per query/key head instead of per value head
    ("b", (B, T, HV, DV + 16)),
    ("w", (B, T, HV, DK)),
    ("k", (B, T, HQK, DK * 2)),
    ("S0", (B, HQK, DK, DV)),
    ("a", (B, T - 1, HV, DK)),
])
def test_forward_rejects_misshaped(name, shape):
    x = problem()
    x[name] = torch.zeros(shape)
    with pytest.raises(ValueError):
        g.chunk_forward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], x["S0"])


def test_forward_rejects_misshaped_outputs():
    x = problem()
    with pytest.raises(ValueError):
        g.chunk_forward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], None, o=torch.zeros(B, T, HQK, DV))
    with pytest.raises(ValueError):
        g.chunk_forward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], None, S_T=torch.zeros(B, HV, DK, DK))


def test_forward_rejects_bad_grouping_and_batch():
    x = problem()
    with pytest.raises(ValueError):  # H_v not a multiple of H_qk
        g.chunk_forward(x["q"], x["k"], torch.zeros(B, T, 3, DV), x["a"][:, :, :3].contiguous(),
                        x["b"][:, :, :3].contiguous(), torch.zeros(B, T, 3, DV), None)
    with pytest.raises(ValueError):  # v with another T
        g.chunk_forward(x["q"], x["k"], torch.zeros(B, T + 1, HV, DV), x["a"], x["b"], x["w"], None)


def test_preact_rejects_misshaped():
    x = problem()
    with pytest.raises(ValueError):
        g.chunk_forward_preact(x["q"], x["k"], x["v"], x["a"], x["b"], torch.zeros(B, T, HV, DK), None)


def test_scalar_gate_forms_reject_misshaped():
    x = problem()
    beta = torch.zeros(B, T, HV)
    with pytest.raises(ValueError):  # alpha per key channel in the scalar form
        g.chunk_forward_scalar(x["q"], x["k"], x["v"], x["a"], beta)
    with pytest.raises(ValueError):  # beta per query/key head
        g.chunk_forward_coupled(x["q"], x["k"], x["v"], x["a"], torch.zeros(B, T, HQK))
    with pytest.raises(ValueError):  # a scalar where the coupled form wants per-channel decay
        g.chunk_forward_coupled(x["q"], x["k"], x["v"], torch.zeros(B, T, HV), beta)


def test_varlen_rejects_misshaped():
    x = problem()
    sq = lambda t: t[0].contiguous()
    cu = torch.tensor([0, 4, 10], dtype=torch.int32)
    with pytest.raises(ValueError):  # S0 for a different number of sequences
        g.chunk_forward_varlen(sq(x["q"]), sq(x["k"]), sq(x["v"]), sq(x["a"]), sq(x["b"]), sq(x["w"]), cu,
                               torch.zeros(3, HV, DK, DV))
    with pytest.raises(ValueError):  # gates per query/key head
        g.chunk_forward_varlen(sq(x["q"]), sq(x["k"]), sq(x["v"]), torch.zeros(T, HQK, DK), sq(x["b"]),
                               sq(x["w"]), cu)
    with pytest.raises(ValueError):  # a leading dimension other than 1
        g.chunk_forward_varlen(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], cu)
    with pytest.raises(ValueError):  # scalar form with per-channel alpha
        g.chunk_forward_varlen(sq(x["q"]), sq(x["k"]), sq(x["v"]), sq(x["a"]), torch.zeros(T, HV), None, cu,
                               gates="scalar")


def test_decode_rejects_misshaped():
    N = 3
    S = torch.zeros(N, HV, DK, DV)
    one = lambda *s: torch.zeros(N, 1, *s)
    q, k, v = one(HQK, DK), one(HQK, DK), one(HV, DV)
    a, b, w = one(HV, DK), one(HV, DK), one(HV, DV)
    with pytest.raises(ValueError):  # one sequence too many
        g.decode_step(torch.zeros(N + 1, 1, HQK, DK), k, v, a, b, w, S)
    with pytest.raises(ValueError):  # gates per query/key head
        g.decode_step(q, k, v, one(HQK, DK), b, w, S)
    with pytest.raises(ValueError):  # missing write gate
        g.decode_step(q, k, v, a, b, None, S)
    with pytest.raises(ValueError):  # coupled form with per-channel beta
        g.decode_step(q, k, v, a, b, None, S, gates="coupled")


def test_backward_rejects_misshaped():
    x = problem()
    dO = torch.zeros(B, T, HV, DV)
    with pytest.raises(ValueError):  # dO per query/key head
        g.chunk_backward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], x["S0"], torch.zeros(B, T, HQK, DV))
    with pytest.raises(ValueError):  # dS_T with the wrong head count
        g.chunk_backward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], x["S0"], dO, torch.zeros(B, HQK, DK, DV))
    with pytest.raises(ValueError):  # a preallocated gradient of the wrong shape
        g.chunk_backward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], x["S0"], dO,
                         grads={"da": torch.zeros(B, T, HQK, DK)})
    with pytest.raises(ValueError):  # gates per query/key head
        g.chunk_backward(x["q"], x["k"], x["v"], torch.zeros(B, T, HQK, DK), x["b"], x["w"], x["S0"], dO)
