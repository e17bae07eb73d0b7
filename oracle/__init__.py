"""fp64 CPU oracle for the Gated DeltaNet-2 forward recurrence.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the product path never does. It shares
no code with the HIP library (``gated_delta_rule_83_amd``), and neither side
imports the other.

The arithmetic lives in ``gdn2_oracle.c`` (plain sequential double-precision
recurrence, one token at a time; see the header of that file for the steps
and the passages they follow). This module only builds it with gcc, loads it
with ctypes and marshals numpy arrays.

Pins (checked by ``tests/test_oracle_pins.py`` against things other than the
oracle itself): the delta-rule tutorial's worked 2x2 example and its printed
variants, the linear-attention closed form, the "difference is zero"
invariant, the query-change identity, a per-step key-read identity for
channel-wise gates, the decay-only closed form, the reductions to the delta
rule, a chunked fp64 evaluation, column separability and split prefill.
The backward pass (``backward``: reverse-mode gradients of the same
recurrence, every state kept) is pinned by ``tests/test_oracle_backward.py``:
central finite differences of the forward, closed-form linear-attention
gradients, the decay and erase-gate gradients at a = 1, b = 0, and the
grouped-head sum.
Gate activations from pre-activations (``activate_gates``, the
parameterisation of the gates in the synthetic workloads: softplus decay,
sigmoid gates) are pinned by ``tests/test_oracle_preact.py`` against
closed-form values, identities and scipy's logistic function.
The coupled and scalar gate forms (``expand_scalar_gates``,
``backward_coupled``: one beta, and alpha, per token and value head,
broadcast to the channels) are pinned by ``tests/test_oracle_coupled.py``:
the broadcast itself, finite differences of the forward on the broadcast
gates, and the closed form at alpha = beta = 1 with unit keys.
Parity unpinned: the exact placement of channel-wise erase and write gates
when b and w are not uniform (the pages state it only in prose); the oracle
takes erase (b * k) r^T and write k (w * v)^T.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn2_oracle.c")
_LIB = os.path.join(_HERE, "libgdn2_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-D_POSIX_C_SOURCE=200809L",
                               "-o", tmp, _SRC, "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def bind(path: str):
    """Load an oracle shared library from `path` (the tests also bind mutated copies)."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.gdn2_oracle_forward.restype = ctypes.c_int
    lib.gdn2_oracle_forward.argtypes = [ctypes.c_int] * 6 + [dp] * 9 + [ctypes.c_int, dp]
    lib.gdn2_oracle_backward.restype = ctypes.c_int
    lib.gdn2_oracle_backward.argtypes = [ctypes.c_int] * 6 + [dp] * 16 + [ctypes.c_int]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = bind(_LIB)
    return _lib


def _f64(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor: upcast exactly via float32
        x = x.detach().cpu().float().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    if x is None:
        return ctypes.POINTER(ctypes.c_double)()
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def forward(q, k, v, a, b, w, S0=None, nthreads: Optional[int] = None,
            want_o: bool = True, timing: bool = False, lib=None):
    """Run the recurrence in fp64.

    Shapes: q, k [B, T, H_qk, d_k]; v, w [B, T, H_v, d_v]; a, b [B, T, H_v, d_k];
    S0 [B, H_v, d_k, d_v] or None. Returns (o [B, T, H_v, d_v], S_T), plus the
    recurrence's wall time in seconds if `timing`.
    """
    lib = _load() if lib is None else lib
    q, k, v, a, b, w, S0 = (_f64(x) for x in (q, k, v, a, b, w, S0))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    assert k.shape == q.shape and v.shape == (B, T, Hv, dv)
    assert a.shape == (B, T, Hv, dk) and b.shape == a.shape and w.shape == v.shape
    if S0 is not None:
        assert S0.shape == (B, Hv, dk, dv)
    o = np.empty((B, T, Hv, dv), dtype=np.float64) if want_o else None
    ST = np.empty((B, Hv, dk, dv), dtype=np.float64)
    el = ctypes.c_double(0.0)
    nt = cores() if nthreads is None else int(nthreads)
    rc = lib.gdn2_oracle_forward(B, T, Hqk, Hv, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                 _ptr(w), _ptr(S0), _ptr(o), _ptr(ST), nt, ctypes.byref(el))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    if timing:
        return o, ST, el.value
    return o, ST


def activate_gates(a_pre, b_pre, w_pre):
    """Gates from their pre-activations, in fp64: decay a = exp(-softplus(x)),
    erase and write gates b, w = sigmoid(x) = exp(-softplus(-x)), with
    softplus(x) = log(1 + e^x) evaluated as logaddexp(0, x)."""
    a = np.exp(-np.logaddexp(0.0, _f64(a_pre)))
    b = np.exp(-np.logaddexp(0.0, -_f64(b_pre)))
    w = np.exp(-np.logaddexp(0.0, -_f64(w_pre)))
    return a, b, w


def forward_preact(q, k, v, a_pre, b_pre, w_pre, S0=None, **kw):
    """The recurrence with its gates given as pre-activations (see
    :func:`activate_gates`); other arguments as :func:`forward`."""
    a, b, w = activate_gates(a_pre, b_pre, w_pre)
    return forward(q, k, v, a, b, w, S0, **kw)


def backward(q, k, v, a, b, w, S0, dO, dS_T=None, nthreads: Optional[int] = None, lib=None) -> dict:
    """Gradients of the recurrence in fp64 (reverse mode, every state kept).

    Shapes as :func:`forward`, plus dO like o and dS_T like S_T (None: zero).
    Returns a dict with dq, dk [B, T, H_qk, d_k] (summed over the value heads
    that share a query/key head), dv, dw [B, T, H_v, d_v], da, db
    [B, T, H_v, d_k] and dS0 [B, H_v, d_k, d_v].
    """
    lib = _load() if lib is None else lib
    q, k, v, a, b, w, S0, dO, dS_T = (_f64(x) for x in (q, k, v, a, b, w, S0, dO, dS_T))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    assert k.shape == q.shape and v.shape == (B, T, Hv, dv) and dO.shape == v.shape
    assert a.shape == (B, T, Hv, dk) and b.shape == a.shape and w.shape == v.shape
    for s in (S0, dS_T):
        if s is not None:
            assert s.shape == (B, Hv, dk, dv)
    dq_h = np.empty((B, T, Hv, dk)); dk_h = np.empty((B, T, Hv, dk))
    out = {"dv": np.empty((B, T, Hv, dv)), "dw": np.empty((B, T, Hv, dv)), "da": np.empty((B, T, Hv, dk)),
           "db": np.empty((B, T, Hv, dk)), "dS0": np.empty((B, Hv, dk, dv))}
    nt = cores() if nthreads is None else int(nthreads)
    rc = lib.gdn2_oracle_backward(B, T, Hqk, Hv, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(w),
                                  _ptr(S0), _ptr(dO), _ptr(dS_T), _ptr(dq_h), _ptr(dk_h), _ptr(out["dv"]),
                                  _ptr(out["da"]), _ptr(out["db"]), _ptr(out["dw"]), _ptr(out["dS0"]), nt)
    if rc != 0:
        raise RuntimeError(f"oracle backward failed with code {rc}")
    G = Hv // Hqk
    out["dq"] = dq_h.reshape(B, T, Hqk, G, dk).sum(axis=3)
    out["dk"] = dk_h.reshape(B, T, Hqk, G, dk).sum(axis=3)
    return out


def backward_preact(q, k, v, a_pre, b_pre, w_pre, S0, dO, dS_T=None, nthreads: Optional[int] = None,
                    lib=None) -> dict:
    """Gradients of :func:`forward_preact`: the recurrence's gradients
    (:func:`backward`) on the activated gates, then through the activations
    by the chain rule, d/dx exp(-softplus(x)) = -a (1 - a) and
    d/dx sigmoid(x) = s (1 - s). Returns dq, dk, dv, dS0 as :func:`backward`
    and da, db, dw with respect to the pre-activations."""
    a, b, w = activate_gates(a_pre, b_pre, w_pre)
    g = backward(q, k, v, a, b, w, S0, dO, dS_T, nthreads=nthreads, lib=lib)
    g["da"] = g["da"] * (-a * (1.0 - a))
    g["db"] = g["db"] * (b * (1.0 - b))
    g["dw"] = g["dw"] * (w * (1.0 - w))
    return g


def expand_scalar_gates(a, beta, d_k: int, d_v: int, scalar_decay: bool):
    """Per-channel gates of the coupled form (GDN-2 note, section on the delta
    rule's basic idea and its limits; wiki, how it works): erase and write
    gate both the scalar beta per token and value head, b = beta * ones(d_k),
    w = beta * ones(d_v); with scalar_decay the decay is alpha * ones(d_k)."""
    beta = _f64(beta)
    a = _f64(a)
    if scalar_decay:
        a = np.repeat(a[..., None], d_k, axis=-1)
    return a, np.repeat(beta[..., None], d_k, axis=-1), np.repeat(beta[..., None], d_v, axis=-1)


def backward_coupled(q, k, v, a, beta, S0, dO, dS_T=None, scalar_decay: bool = False,
                     nthreads: Optional[int] = None, lib=None) -> dict:
    """Gradients of the coupled (and, with scalar_decay, scalar) gate form:
    the recurrence's gradients (:func:`backward`) on the expanded gates, then
    through the broadcasts by the chain rule: dbeta = sum over the key
    channels of db plus sum over the value columns of dw; with scalar_decay
    da = sum over the key channels of da. Returns dq, dk, dv, da, db (= dbeta)
    and dS0."""
    d_k, d_v = q.shape[-1], v.shape[-1]
    A, Bg, W = expand_scalar_gates(a, beta, d_k, d_v, scalar_decay)
    g = backward(q, k, v, A, Bg, W, S0, dO, dS_T, nthreads=nthreads, lib=lib)
    g["db"] = g["db"].sum(axis=-1) + g.pop("dw").sum(axis=-1)
    if scalar_decay:
        g["da"] = g["da"].sum(axis=-1)
    return g


def forward_heads(inputs: dict, heads, nthreads: Optional[int] = None) -> Tuple[dict, dict]:
    """Run the oracle only on selected (n, h_v) pairs of a prefill input dict.

    `inputs` holds q, k, v, a, b, w, S0 (numpy or torch, full shapes). Returns
    ({(n, h): o[T, d_v]}, {(n, h): S_T[d_k, d_v]}).
    """
    heads = list(heads)
    q, k = inputs["q"], inputs["k"]
    Hqk = q.shape[2]
    Hv = inputs["v"].shape[2]
    G = Hv // Hqk
    S0 = inputs.get("S0")

    def gather(x, per_qk):
        rows = [_f64(x[n:n + 1, :, (h // G if per_qk else h):(h // G if per_qk else h) + 1])
                for (n, h) in heads]
        return np.concatenate(rows, axis=0)

    s0 = None
    if S0 is not None:
        s0 = np.concatenate([_f64(S0[n:n + 1, h:h + 1]) for (n, h) in heads], axis=0)
    o, ST = forward(gather(q, True), gather(k, True), gather(inputs["v"], False),
                    gather(inputs["a"], False), gather(inputs["b"], False),
                    gather(inputs["w"], False), s0, nthreads=nthreads)
    outs = {hd: o[i, :, 0] for i, hd in enumerate(heads)}
    states = {hd: ST[i, 0] for i, hd in enumerate(heads)}
    return outs, states
