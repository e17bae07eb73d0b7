"""Shared helpers for the GPU parity tests (test infrastructure).

Error metric: per tensor (o, and S_T), normwise max|x - ref| / max|ref|, the
reading of "max relative error" that stays meaningful near zero. Tolerances
are those of the workloads' acceptance bar: 1e-4 for fp32 inputs and 2e-2
for bf16 inputs (fp32 state). The oracle is always fed the values the GPU
sees (bf16 inputs upcast exactly).
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def normwise(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    return float(np.max(np.abs(x - ref))) / max(scale, 1e-30)


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rand_inputs(rng, B, T, Hqk, Hv, dk, dv, with_s0=True, a_lo=0.5, s0_scale=0.5, normalise=True):
    """Small random problems (float32 numpy), gates in their stated ranges."""
    def unit(x):
        return (x / np.linalg.norm(x, axis=-1, keepdims=True)) if normalise else x
    f = np.float32
    q = unit(rng.standard_normal((B, T, Hqk, dk))).astype(f)
    k = unit(rng.standard_normal((B, T, Hqk, dk))).astype(f)
    v = rng.standard_normal((B, T, Hv, dv)).astype(f)
    a = rng.uniform(a_lo, 1.0, (B, T, Hv, dk)).astype(f)
    b = rng.uniform(0.0, 1.0, (B, T, Hv, dk)).astype(f)
    w = rng.uniform(0.0, 1.0, (B, T, Hv, dv)).astype(f)
    S0 = (rng.standard_normal((B, Hv, dk, dv)) * s0_scale).astype(f) if with_s0 else None
    return dict(q=q, k=k, v=v, a=a, b=b, w=w, S0=S0)


def gpu_prefill(td: dict, chunk: int, S_T=True):
    """Run gdn2_chunk_forward on torch tensors already on the GPU."""
    import gated_delta_rule_83_amd as g
    return g.chunk_forward(td["q"], td["k"], td["v"], td["a"], td["b"], td["w"], td.get("S0"),
                           chunk=chunk, want_state=S_T)


def per_head_normwise(x, ref, head_axes):
    """Normwise error of every (sequence, head) slice: max|x - ref| / max|ref|
    over the axes NOT in `head_axes` (e.g. head_axes=(0, 2) for [B, T, H, d]).
    Returns (worst error, index of the worst slice, array of all errors)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        return float("inf"), None, None
    red = tuple(i for i in range(x.ndim) if i not in head_axes)
    num = np.max(np.abs(x - ref), axis=red)
    den = np.maximum(np.max(np.abs(ref), axis=red), 1e-30)
    err = num / den
    idx = np.unravel_index(int(np.argmax(err)), err.shape)
    return float(err[idx]), tuple(int(i) for i in idx), err
