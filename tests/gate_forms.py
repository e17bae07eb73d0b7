"""Inputs and per-form entry points for the packed-sequence tests of every
gate form (per-channel gates, pre-activations, coupled beta, scalar alpha and
beta). Shared by the forward and backward GPU tests; holds no arithmetic of
the method."""
import numpy as np
import torch

import gated_delta_rule_83_amd as g
import oracle
from tests.parity import rand_inputs

FORMS = ("channel", "preact", "coupled", "scalar")


def form_inputs(rng, form, T, Hv, dk, dv, dtype, dev, B=1, Hqk=1):
    """Torch inputs [B, T, ...] of one gate form (grouped heads when Hqk < Hv)."""
    f = np.float32
    d = rand_inputs(rng, B, T, Hqk, Hv, dk, dv, with_s0=False)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = {nm: torch.from_numpy(d[nm]).to(tdt).to(dev) for nm in ("q", "k", "v")}
    if form == "channel":
        for nm in ("a", "b", "w"):
            x[nm] = torch.from_numpy(d[nm]).to(dev)
    elif form == "preact":
        x["a"] = torch.from_numpy((rng.standard_normal((B, T, Hv, dk)) - 2.0).astype(f)).to(tdt).to(dev)
        x["b"] = torch.from_numpy(rng.standard_normal((B, T, Hv, dk)).astype(f)).to(tdt).to(dev)
        x["w"] = torch.from_numpy(rng.standard_normal((B, T, Hv, dv)).astype(f)).to(tdt).to(dev)
    else:
        a = rng.uniform(0.5, 1.0, (B, T, Hv)).astype(f) if form == "scalar" else d["a"]
        x["a"] = torch.from_numpy(a).to(dev)
        x["b"] = torch.from_numpy(rng.uniform(0.0, 1.0, (B, T, Hv)).astype(f)).to(dev)
        x["w"] = None
    return x


def forward_alone(form, x, S0, chunk):
    """The unpacked entry point of the form on [1, T, ...] inputs."""
    if form == "channel":
        return g.chunk_forward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], S0, chunk=chunk)
    if form == "preact":
        return g.chunk_forward_preact(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], S0, chunk=chunk)
    fn = g.chunk_forward_coupled if form == "coupled" else g.chunk_forward_scalar
    return fn(x["q"], x["k"], x["v"], x["a"], x["b"], S0, chunk=chunk)


def backward_alone(form, x, S0, dO, dST):
    if form == "channel":
        return g.chunk_backward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], S0, dO, dST)
    if form == "preact":
        return g.chunk_backward_preact(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], S0, dO, dST)
    fn = g.chunk_backward_coupled if form == "coupled" else g.chunk_backward_scalar
    return fn(x["q"], x["k"], x["v"], x["a"], x["b"], S0, dO, dST)


def oracle_forward(form, x, S0):
    if form == "channel":
        return oracle.forward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], S0)
    if form == "preact":
        return oracle.forward_preact(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], S0)
    a, b, w = oracle.expand_scalar_gates(x["a"], x["b"], x["q"].shape[-1], x["v"].shape[-1], form == "scalar")
    return oracle.forward(x["q"], x["k"], x["v"], a, b, w, S0)


def oracle_backward(form, x, S0, dO, dST):
    if form == "channel":
        return oracle.backward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], S0, dO, dST)
    if form == "preact":
        return oracle.backward_preact(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], S0, dO, dST)
    return oracle.backward_coupled(x["q"], x["k"], x["v"], x["a"], x["b"], S0, dO, dST,
                                   scalar_decay=form == "scalar")


def sl(x, t0, t1):
    """Tokens t0..t1-1 of a [1, T, ...] tensor (or None), contiguous."""
    return None if x is None else x[:, t0:t1].contiguous()
