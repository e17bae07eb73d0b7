"""Seeded synthetic inputs for the Gated DeltaNet-2 forward path.

This module only draws and shapes inputs. It holds none of the recurrence's
arithmetic, so that both the HIP path and the fp64 oracle can be fed from it
without sharing any of the method.

What is drawn follows the method's statement of its inputs (Gated DeltaNet-2
blog post on tilnote.io, section on the GDN-2 design; news.hamidun.com item,
section on the architecture): per token a query and key on the key axis, a
value on the value axis, a channel-wise decay and a channel-wise erase gate on
the key axis, and a channel-wise write gate on the value axis. Keys and
queries are L2-normalised, which the delta-rule tutorial (ai-systems-
engineering.com "Delta rule", section on beta) gives as the condition under
which one correction step lands exactly on the new value.

Gate activations, as the synthetic workloads define them:
  a = exp(-softplus(x)) = 1 / (1 + e^x)      decay, in (0, 1]
  b = sigmoid(x), w = sigmoid(x)             erase / write gates, in (0, 1)

Layouts (row-major, contiguous):
  q, k : [B, T, H_qk, d_k]      v, w : [B, T, H_v, d_v]
  a, b : [B, T, H_v, d_k]       S0   : [B, H_v, d_k, d_v] or None (zeros)

Draw order with numpy ``default_rng(seed)``, all float32 draws:
q, k, v, a_pre, b_pre, w_pre, hard-erase mask, S0. The decode workload draws
each step from ``SeedSequence([seed, step])`` in the same order (no S0).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Config", "CONFIGS", "config", "scaled", "make_inputs", "make_decode_step",
           "make_decode_state", "to_torch", "draw_on_device"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    T: int
    H_qk: int
    H_v: int
    d_k: int
    d_v: int
    chunk: int
    dtype: str            # "f32" or "bf16": dtype of q, k, v and o
    seed: int
    a_mu: float = 0.0     # mean of the decay pre-activation
    hard_erase_p: float = 0.0   # Bernoulli rate of (batch, token) positions with b pre-activation = 6
    s0_std: Optional[float] = None  # None: S0 = 0 (null); else S0 ~ N(0, s0_std)
    decode_steps: int = 0  # > 0: a decode workload of this many single-token steps (T is 1)

    @property
    def group(self) -> int:
        return self.H_v // self.H_qk

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five synthetic workloads. Shapes follow the pages: head dim 128 and
# 16 QK / 32 V heads come from the aiki wiki entry on Gated DeltaNet (how it
# works); the 1.3B-class model from the tilnote post (scale and limits).
CONFIGS = [
    Config("c0_tiny_f32", B=1, T=64, H_qk=2, H_v=2, d_k=16, d_v=16, chunk=16, dtype="f32",
           seed=0, a_mu=0.0),
    Config("c1_1p3b_layer", B=8, T=4096, H_qk=16, H_v=16, d_k=128, d_v=128, chunk=64,
           dtype="bf16", seed=1, a_mu=-4.0),
    Config("c2_long_context", B=1, T=65536, H_qk=16, H_v=16, d_k=128, d_v=128, chunk=64,
           dtype="bf16", seed=2, a_mu=-4.0, hard_erase_p=0.01),
    Config("c3_grouped_heads", B=4, T=16384, H_qk=16, H_v=32, d_k=128, d_v=128, chunk=64,
           dtype="bf16", seed=3, a_mu=-4.0),
    Config("c4_batched_decode", B=256, T=1, H_qk=16, H_v=16, d_k=128, d_v=128, chunk=64,
           dtype="bf16", seed=4, a_mu=-4.0, s0_std=0.02, decode_steps=1024),
]


def config(i: int) -> Config:
    return CONFIGS[i]


def scaled(i: int, **kw) -> Config:
    """A scaled-down copy of workload i (same distributions, smaller sizes)."""
    c = CONFIGS[i]
    return c.replace(name=c.name + "_scaled", **kw)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    n = np.maximum(n, 1e-30)
    return (x / n).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _decay(x: np.ndarray) -> np.ndarray:
    # exp(-softplus(x)) == 1 / (1 + e^x); computed in float64, stored as float32.
    return (1.0 / (1.0 + np.exp(x.astype(np.float64)))).astype(np.float32)


def _draw(rng: np.random.Generator, c: Config, B: int, T: int, with_s0: bool, preact: bool = False):
    f32 = np.float32
    q = _l2_normalise(rng.standard_normal((B, T, c.H_qk, c.d_k), dtype=f32))
    k = _l2_normalise(rng.standard_normal((B, T, c.H_qk, c.d_k), dtype=f32))
    v = rng.standard_normal((B, T, c.H_v, c.d_v), dtype=f32)
    a_pre = rng.standard_normal((B, T, c.H_v, c.d_k), dtype=f32)
    if c.a_mu != 0.0:
        a_pre += f32(c.a_mu)
    b_pre = rng.standard_normal((B, T, c.H_v, c.d_k), dtype=f32)
    w_pre = rng.standard_normal((B, T, c.H_v, c.d_v), dtype=f32)
    if c.hard_erase_p > 0.0:
        mask = rng.random((B, T), dtype=np.float64) < c.hard_erase_p
        b_pre[mask] = f32(6.0)
    if preact:
        a, b, w = a_pre, b_pre, w_pre
    else:
        a, b, w = _decay(a_pre), _sigmoid(b_pre), _sigmoid(w_pre)
    del a_pre, b_pre, w_pre
    S0 = None
    if with_s0 and c.s0_std is not None:
        S0 = (rng.standard_normal((B, c.H_v, c.d_k, c.d_v), dtype=f32) * f32(c.s0_std)).astype(f32)
    return dict(q=q, k=k, v=v, a=a, b=b, w=w, S0=S0)


def make_inputs(c: Config) -> dict:
    """Prefill inputs for config c as float32 numpy arrays (q, k, v not yet cast).

    Use :func:`to_torch` to get the stored dtypes; the oracle must be fed the
    values *after* that cast (bf16 values upcast exactly).
    """
    rng = np.random.default_rng(c.seed)
    return _draw(rng, c, c.B, c.T, with_s0=True)


def make_preact_inputs(c: Config) -> dict:
    """The same draws as :func:`make_inputs`, with the gates left as their
    float32 pre-activations (a: decay, b, w: erase and write gates). Use
    :func:`to_torch_preact` to store them in the input dtype."""
    rng = np.random.default_rng(c.seed)
    return _draw(rng, c, c.B, c.T, with_s0=True, preact=True)


def to_torch_preact(d: dict, dtype: str, device=None):
    """Like :func:`to_torch`, with the gate pre-activations a, b, w also cast
    to `dtype` (round-to-nearest-even for bf16)."""
    import torch
    out = to_torch(d, dtype, device)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for name in ("a", "b", "w"):
        out[name] = out[name].to(tdt)
    return out


def make_decode_state(c: Config) -> Optional[np.ndarray]:
    """Starting state of a decode workload: S0 ~ N(0, s0_std), from seed [seed, 'S0']."""
    if c.s0_std is None:
        return None
    rng = np.random.default_rng(np.random.SeedSequence([c.seed, 1 << 30]))
    return (rng.standard_normal((c.B, c.H_v, c.d_k, c.d_v), dtype=np.float32)
            * np.float32(c.s0_std)).astype(np.float32)


def make_decode_step(c: Config, step: int) -> dict:
    """Single-token inputs of decode step `step`: arrays shaped [B, 1, H, d]."""
    rng = np.random.default_rng(np.random.SeedSequence([c.seed, step]))
    d = _draw(rng, c, c.B, 1, with_s0=False)
    d.pop("S0")
    return d


def to_torch(d: dict, dtype: str, device=None):
    """Cast a drawn input dict to torch tensors in their stored dtypes.

    q, k, v take `dtype` ("bf16" or "f32", fp32 -> bf16 with round-to-nearest-
    even); a, b, w and S0 stay float32.
    """
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for name, x in d.items():
        if x is None:
            out[name] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(x))
        if name in ("q", "k", "v"):
            t = t.to(tdt)
        if device is not None:
            t = t.to(device)
        out[name] = t
    return out


def draw_on_device(B: int, T: int, H_qk: int, H_v: int, d_k: int, d_v: int, dtype: str, gates: str,
                   device, seed: int, a_mu: float = -4.0, packed: bool = False,
                   hard_erase_p: float = 0.0) -> dict:
    """Inputs drawn on the device with torch's seeded generator, for problems
    too large to draw on the host (sequences of hundreds of thousands of
    tokens). Same distributions as the workloads: q, k ~ N(0, 1) then
    L2-normalised (fp32, before the cast), v ~ N(0, 1); gates by `gates`:
      "channel": a = 1 / (1 + e^x), x ~ N(a_mu, 1); b, w = sigmoid(N(0, 1)), fp32
      "preact":  the pre-activations themselves, in `dtype`
      "coupled": a as "channel"; beta = sigmoid(N(0, 1)) per token and value head
      "scalar":  alpha = 1 / (1 + e^x), x ~ N(a_mu, 1), and beta, per token and value head
    With hard_erase_p > 0, Bernoulli(hard_erase_p) (batch, token) positions
    get erase-gate pre-activation 6 on every head and key channel (per-channel
    forms). Shapes [B, T, H, d] (gates of the coupled forms [B, T, H_v]);
    with `packed`, B must be 1 and the leading dimension is dropped."""
    import torch
    gen = torch.Generator(device=device).manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def normal(shape, mu=0.0):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return x.add_(mu) if mu else x

    def unit(shape):
        x = normal(shape)
        x.div_(x.norm(dim=-1, keepdim=True).clamp_min_(1e-30))
        return x.to(tdt)

    out = {"q": unit((B, T, H_qk, d_k)), "k": unit((B, T, H_qk, d_k)), "v": normal((B, T, H_v, d_v)).to(tdt)}
    decay = lambda x: torch.reciprocal(1.0 + torch.exp(x))
    def erase_pre():
        x = normal((B, T, H_v, d_k))
        if hard_erase_p > 0.0:
            hit = torch.rand((B, T), generator=gen, device=device) < hard_erase_p
            x[hit] = 6.0
        return x

    if gates == "channel":
        out["a"] = decay(normal((B, T, H_v, d_k), a_mu))
        out["b"] = torch.sigmoid(erase_pre())
        out["w"] = torch.sigmoid(normal((B, T, H_v, d_v)))
    elif gates == "preact":
        out["a"] = normal((B, T, H_v, d_k), a_mu).to(tdt)
        out["b"] = erase_pre().to(tdt)
        out["w"] = normal((B, T, H_v, d_v)).to(tdt)
    elif gates in ("coupled", "scalar"):
        out["a"] = decay(normal((B, T, H_v) if gates == "scalar" else (B, T, H_v, d_k), a_mu))
        out["b"] = torch.sigmoid(normal((B, T, H_v)))
        out["w"] = None
    else:
        raise ValueError(f"unknown gate form {gates}")
    if packed:
        assert B == 1
        out = {k: (None if x is None else x[0]) for k, x in out.items()}
    return out
