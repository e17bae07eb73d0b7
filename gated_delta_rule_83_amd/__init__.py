"""libgdn2: Gated DeltaNet-2 forward sequence mixing on MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/gdn2.h``. Every step of
the computation runs in the HIP kernels of ``libgdn2.so``; this module only
marshals arguments. PyTorch supplies device memory and the stream.

Raw entry points (same names and arguments as the C ABI; pointers are ints):
    gdn2_chunk_forward, gdn2_chunk_forward_coupled, gdn2_chunk_forward_scalar,
    gdn2_chunk_forward_varlen, gdn2_decode_step,
    gdn2_chunk_forward_workspace_bytes, gdn2_status_string, gdn2_version
Torch conveniences:
    chunk_forward(q, k, v, a, b, w, S0=None, chunk=64) -> (o, S_T)
    chunk_forward_coupled(q, k, v, a, beta, S0=None, chunk=64) -> (o, S_T)
    chunk_forward_scalar(q, k, v, alpha, beta, S0=None, chunk=64) -> (o, S_T)
    chunk_forward_varlen(q, k, v, a, b, w, cu_seqlens, S0=None, chunk=64) -> (o, S_T)
    decode_step(q, k, v, a, b, w, S) -> o        (S updated in place)

If ``libgdn2.so`` has not been built, loading fails loudly: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn2.so")

GDN2_OK = 0
GDN2_ERR_NULL_POINTER = 1
GDN2_ERR_BAD_SHAPE = 2
GDN2_ERR_UNSUPPORTED = 3
GDN2_ERR_BAD_DTYPE = 4
GDN2_ERR_WORKSPACE = 5
GDN2_ERR_HIP = 6
GDN2_ERR_ALIAS = 7
GDN2_ERR_SCRATCH = 8
GDN2_NOALLOC_SCRATCH_BYTES = 64 << 20

GDN2_F32 = 0
GDN2_BF16 = 1

EXPORTED = ("gdn2_chunk_forward", "gdn2_chunk_forward_coupled", "gdn2_chunk_forward_scalar",
            "gdn2_chunk_forward_preact",
            "gdn2_chunk_forward_varlen", "gdn2_decode_step",
            "gdn2_chunk_forward_workspace_bytes", "gdn2_chunk_forward_plan", "gdn2_chunk_forward_noalloc",
            "gdn2_chunk_backward", "gdn2_chunk_backward_workspace_bytes",
            "gdn2_chunk_backward_varlen", "gdn2_chunk_backward_varlen_workspace_bytes", "gdn2_chunk_backward_preact",
            "gdn2_chunk_backward_coupled", "gdn2_chunk_backward_scalar", "gdn2_chunk_forward_varlen_gates",
            "gdn2_chunk_backward_varlen_gates", "gdn2_decode_step_gates",
            "gdn2_status_string", "gdn2_version")


class gdn2_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H_qk", ctypes.c_int32),
                ("H_v", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Gdn2Error(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"libgdn2 status {status}: {gdn2_status_string(status)}")


_lib = None


def load(path: Optional[str] = None):
    """Load libgdn2.so (raises if it is missing: build it with gated_delta_rule_83_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libgdn2.so not found at {p}; run `python -m gated_delta_rule_83_amd.build`")
    lib = ctypes.CDLL(p)
    vp, sz, dp = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(gdn2_desc)
    lib.gdn2_chunk_forward.restype = ctypes.c_int
    lib.gdn2_chunk_forward.argtypes = [dp] + [vp] * 9 + [vp, sz, vp]
    lib.gdn2_chunk_forward_noalloc.restype = ctypes.c_int
    lib.gdn2_chunk_forward_noalloc.argtypes = [dp] + [vp] * 9 + [vp]
    lib.gdn2_chunk_forward_preact.restype = ctypes.c_int
    lib.gdn2_chunk_forward_preact.argtypes = [dp] + [vp] * 9 + [vp, sz, vp]
    lib.gdn2_chunk_forward_coupled.restype = ctypes.c_int
    lib.gdn2_chunk_forward_coupled.argtypes = [dp] + [vp] * 8 + [vp, sz, vp]
    lib.gdn2_chunk_forward_scalar.restype = ctypes.c_int
    lib.gdn2_chunk_forward_scalar.argtypes = [dp] + [vp] * 8 + [vp, sz, vp]
    lib.gdn2_chunk_forward_varlen_gates.restype = ctypes.c_int
    lib.gdn2_chunk_forward_varlen_gates.argtypes = [dp, vp, ctypes.c_int] + [vp] * 9 + [vp]
    lib.gdn2_chunk_backward_varlen_gates.restype = ctypes.c_int
    lib.gdn2_chunk_backward_varlen_gates.argtypes = [dp, vp, ctypes.c_int] + [vp] * 16 + [vp, sz, vp]
    lib.gdn2_chunk_forward_varlen.restype = ctypes.c_int
    lib.gdn2_chunk_forward_varlen.argtypes = [dp] + [vp] * 10 + [vp]
    lib.gdn2_decode_step_gates.restype = ctypes.c_int
    lib.gdn2_decode_step_gates.argtypes = [dp, ctypes.c_int] + [vp] * 8 + [vp]
    lib.gdn2_decode_step.restype = ctypes.c_int
    lib.gdn2_decode_step.argtypes = [dp] + [vp] * 8 + [vp]
    lib.gdn2_chunk_forward_workspace_bytes.restype = sz
    lib.gdn2_chunk_forward_workspace_bytes.argtypes = [dp]
    lib.gdn2_chunk_forward_plan.restype = ctypes.c_int
    lib.gdn2_chunk_forward_plan.argtypes = [dp, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.gdn2_chunk_backward.restype = ctypes.c_int
    lib.gdn2_chunk_backward.argtypes = [dp] + [vp] * 16 + [vp, sz, vp]
    lib.gdn2_chunk_backward_workspace_bytes.restype = sz
    lib.gdn2_chunk_backward_workspace_bytes.argtypes = [dp]
    lib.gdn2_chunk_backward_preact.restype = ctypes.c_int
    lib.gdn2_chunk_backward_preact.argtypes = [dp] + [vp] * 16 + [vp, sz, vp]
    lib.gdn2_chunk_backward_coupled.restype = ctypes.c_int
    lib.gdn2_chunk_backward_coupled.argtypes = [dp] + [vp] * 14 + [vp, sz, vp]
    lib.gdn2_chunk_backward_scalar.restype = ctypes.c_int
    lib.gdn2_chunk_backward_scalar.argtypes = [dp] + [vp] * 14 + [vp, sz, vp]
    lib.gdn2_chunk_backward_varlen.restype = ctypes.c_int
    lib.gdn2_chunk_backward_varlen.argtypes = [dp] + [vp] * 17 + [vp, sz, vp]
    lib.gdn2_chunk_backward_varlen_workspace_bytes.restype = sz
    lib.gdn2_chunk_backward_varlen_workspace_bytes.argtypes = [dp]
    lib.gdn2_status_string.restype = ctypes.c_char_p
    lib.gdn2_status_string.argtypes = [ctypes.c_int]
    lib.gdn2_version.restype = ctypes.c_int
    lib.gdn2_version.argtypes = []
    if path is None:
        _lib = lib
    return lib


def make_desc(B, T, H_qk, H_v, d_k, d_v, chunk=64, dtype=GDN2_BF16) -> gdn2_desc:
    return gdn2_desc(B, T, H_qk, H_v, d_k, d_v, chunk, dtype)


# ------------------------------------------------------------------ raw C ABI
def gdn2_version() -> int:
    return load().gdn2_version()


def gdn2_status_string(status: int) -> str:
    return load().gdn2_status_string(int(status)).decode()


def gdn2_chunk_forward_workspace_bytes(desc) -> int:
    return load().gdn2_chunk_forward_workspace_bytes(None if desc is None else ctypes.byref(desc))


def gdn2_chunk_forward_plan(desc):
    """(status, chunk_run, segments): how the prefill would run `desc`."""
    c, n = ctypes.c_int32(0), ctypes.c_int32(0)
    st = load().gdn2_chunk_forward_plan(None if desc is None else ctypes.byref(desc), ctypes.byref(c),
                                        ctypes.byref(n))
    return st, c.value, n.value


def gdn2_chunk_forward(desc, q, k, v, a, b, w, S0, o, S_T, workspace=0, workspace_bytes=0,
                       stream=0) -> int:
    return load().gdn2_chunk_forward(None if desc is None else ctypes.byref(desc), q, k, v, a, b, w,
                                     S0, o, S_T, workspace, workspace_bytes, stream)


def gdn2_chunk_forward_noalloc(desc, q, k, v, a, b, w, S0, o, S_T, stream=0) -> int:
    return load().gdn2_chunk_forward_noalloc(None if desc is None else ctypes.byref(desc), q, k, v, a, b, w, S0,
                                             o, S_T, stream)


def gdn2_chunk_forward_preact(desc, q, k, v, a_pre, b_pre, w_pre, S0, o, S_T, workspace=0, workspace_bytes=0,
                              stream=0) -> int:
    return load().gdn2_chunk_forward_preact(None if desc is None else ctypes.byref(desc), q, k, v, a_pre, b_pre,
                                            w_pre, S0, o, S_T, workspace, workspace_bytes, stream)


def gdn2_chunk_forward_coupled(desc, q, k, v, a, beta, S0, o, S_T, workspace=0, workspace_bytes=0,
                               stream=0) -> int:
    return load().gdn2_chunk_forward_coupled(None if desc is None else ctypes.byref(desc), q, k, v, a, beta,
                                             S0, o, S_T, workspace, workspace_bytes, stream)


def gdn2_chunk_forward_scalar(desc, q, k, v, a, beta, S0, o, S_T, workspace=0, workspace_bytes=0,
                              stream=0) -> int:
    return load().gdn2_chunk_forward_scalar(None if desc is None else ctypes.byref(desc), q, k, v, a, beta,
                                            S0, o, S_T, workspace, workspace_bytes, stream)


def gdn2_chunk_forward_varlen(desc, cu_seqlens, q, k, v, a, b, w, S0, o, S_T, stream=0) -> int:
    return load().gdn2_chunk_forward_varlen(None if desc is None else ctypes.byref(desc), cu_seqlens, q, k,
                                            v, a, b, w, S0, o, S_T, stream)


def gdn2_chunk_forward_varlen_gates(desc, cu_seqlens, gates, q, k, v, a, b, w, S0, o, S_T, stream=0) -> int:
    return load().gdn2_chunk_forward_varlen_gates(None if desc is None else ctypes.byref(desc), cu_seqlens, gates,
                                                  q, k, v, a, b, w, S0, o, S_T, stream)


def gdn2_chunk_backward_varlen_gates(desc, cu_seqlens, gates, q, k, v, a, b, w, S0, dO, dS_T, dq, dk, dv, da, db,
                                     dw, dS0, workspace=0, workspace_bytes=0, stream=0) -> int:
    return load().gdn2_chunk_backward_varlen_gates(None if desc is None else ctypes.byref(desc), cu_seqlens, gates,
                                                   q, k, v, a, b, w, S0, dO, dS_T, dq, dk, dv, da, db, dw, dS0,
                                                   workspace, workspace_bytes, stream)


def gdn2_decode_step_gates(desc, gates, q, k, v, a, b, w, S, o, stream=0) -> int:
    return load().gdn2_decode_step_gates(None if desc is None else ctypes.byref(desc), gates, q, k, v, a, b, w, S, o,
                                         stream)


def gdn2_chunk_backward_workspace_bytes(desc) -> int:
    return load().gdn2_chunk_backward_workspace_bytes(None if desc is None else ctypes.byref(desc))


def gdn2_chunk_backward(desc, q, k, v, a, b, w, S0, dO, dS_T, dq, dk, dv, da, db, dw, dS0, workspace=0,
                        workspace_bytes=0, stream=0) -> int:
    return load().gdn2_chunk_backward(None if desc is None else ctypes.byref(desc), q, k, v, a, b, w, S0, dO,
                                      dS_T, dq, dk, dv, da, db, dw, dS0, workspace, workspace_bytes, stream)


def gdn2_chunk_backward_preact(desc, q, k, v, a_pre, b_pre, w_pre, S0, dO, dS_T, dq, dk, dv, da_pre, db_pre,
                               dw_pre, dS0, workspace=0, workspace_bytes=0, stream=0) -> int:
    return load().gdn2_chunk_backward_preact(None if desc is None else ctypes.byref(desc), q, k, v, a_pre, b_pre,
                                             w_pre, S0, dO, dS_T, dq, dk, dv, da_pre, db_pre, dw_pre, dS0, workspace,
                                             workspace_bytes, stream)


def gdn2_chunk_backward_coupled(desc, q, k, v, a, beta, S0, dO, dS_T, dq, dk, dv, da, dbeta, dS0, workspace=0,
                                workspace_bytes=0, stream=0) -> int:
    return load().gdn2_chunk_backward_coupled(None if desc is None else ctypes.byref(desc), q, k, v, a, beta, S0,
                                              dO, dS_T, dq, dk, dv, da, dbeta, dS0, workspace, workspace_bytes,
                                              stream)


def gdn2_chunk_backward_scalar(desc, q, k, v, alpha, beta, S0, dO, dS_T, dq, dk, dv, dalpha, dbeta, dS0,
                               workspace=0, workspace_bytes=0, stream=0) -> int:
    return load().gdn2_chunk_backward_scalar(None if desc is None else ctypes.byref(desc), q, k, v, alpha, beta,
                                             S0, dO, dS_T, dq, dk, dv, dalpha, dbeta, dS0, workspace,
                                             workspace_bytes, stream)


def gdn2_chunk_backward_varlen_workspace_bytes(desc) -> int:
    return load().gdn2_chunk_backward_varlen_workspace_bytes(None if desc is None else ctypes.byref(desc))


def gdn2_chunk_backward_varlen(desc, cu_seqlens, q, k, v, a, b, w, S0, dO, dS_T, dq, dk, dv, da, db, dw, dS0,
                               workspace=0, workspace_bytes=0, stream=0) -> int:
    return load().gdn2_chunk_backward_varlen(None if desc is None else ctypes.byref(desc), cu_seqlens, q, k, v, a,
                                             b, w, S0, dO, dS_T, dq, dk, dv, da, db, dw, dS0, workspace,
                                             workspace_bytes, stream)


def gdn2_decode_step(desc, q, k, v, a, b, w, S, o, stream=0) -> int:
    return load().gdn2_decode_step(None if desc is None else ctypes.byref(desc), q, k, v, a, b, w, S,
                                   o, stream)


# ------------------------------------------------------------------ torch conveniences
def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDN2_BF16
    if t.dtype == torch.float32:
        return GDN2_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _check(t, name, dtype=None):
    import torch
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a torch tensor on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _want(t, name, shape, dtype, device):
    """t (or None) must be a contiguous `dtype` tensor of exactly `shape` on
    `device`: the kernels index every tensor from the sizes of q and v, so a
    tensor of another shape would be read or written out of its bounds."""
    if t is None:
        return
    _check(t, name, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, but q is on {device}")


def _want_rows(t, name, rows, tail, dtype, device):
    """Like _want for token tensors given as [rows, *tail] with any leading
    size-1 dimensions (e.g. [1, T, H, d] or [T, H, d])."""
    if t is None:
        return
    _check(t, name, dtype)
    n = len(tail) + 1
    lead = tuple(t.shape[:-n])
    if tuple(t.shape[-n:]) != (rows,) + tuple(tail) or any(x != 1 for x in lead):
        raise ValueError(f"{name} must have shape [..., {rows}, {', '.join(map(str, tail))}] "
                         f"(leading dimensions 1), got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, but q is on {device}")


def _dims(q, v):
    """(B, T, H_qk, H_v, d_k, d_v) of a [B, T, H, d] problem from q and v."""
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError(f"q and v must be [B, T, H, d], got {tuple(q.shape)} and {tuple(v.shape)}")
    B, T, H_qk, d_k = q.shape
    if tuple(v.shape[:2]) != (B, T):
        raise ValueError(f"v must have B={B}, T={T} like q, got {tuple(v.shape)}")
    H_v, d_v = v.shape[2], v.shape[3]
    if H_v % H_qk:
        raise ValueError(f"value heads ({H_v}) must be a multiple of query/key heads ({H_qk})")
    return B, T, H_qk, H_v, d_k, d_v


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def chunk_forward(q, k, v, a, b, w, S0=None, chunk: int = 64, o=None, S_T=None,
                  want_state: bool = True, stream=None):
    """Prefill. q, k [B,T,H_qk,d_k]; v [B,T,H_v,d_v]; a, b [B,T,H_v,d_k] fp32;
    w [B,T,H_v,d_v] fp32; S0 [B,H_v,d_k,d_v] fp32 or None. Returns (o, S_T)."""
    import torch
    B, T, H_qk, H_v, d_k, d_v = _dims(q, v)
    dev, f32 = q.device, torch.float32
    _want(q, "q", (B, T, H_qk, d_k), q.dtype, dev)
    _want(k, "k", (B, T, H_qk, d_k), q.dtype, dev)
    _want(v, "v", (B, T, H_v, d_v), q.dtype, dev)
    _want(a, "a", (B, T, H_v, d_k), f32, dev)
    _want(b, "b", (B, T, H_v, d_k), f32, dev)
    _want(w, "w", (B, T, H_v, d_v), f32, dev)
    _want(S0, "S0", (B, H_v, d_k, d_v), f32, dev)
    if o is None:
        o = torch.empty((B, T, H_v, d_v), dtype=q.dtype, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H_v, d_k, d_v), dtype=f32, device=dev)
    _want(o, "o", (B, T, H_v, d_v), q.dtype, dev)
    _want(S_T, "S_T", (B, H_v, d_k, d_v), f32, dev)
    desc = make_desc(B, T, H_qk, H_v, d_k, d_v, chunk, _dtype_code(q))
    ws = gdn2_chunk_forward_workspace_bytes(desc)
    work = torch.empty(ws, dtype=torch.uint8, device=dev) if ws else None
    st = gdn2_chunk_forward(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(w), _ptr(S0),
                            _ptr(o), _ptr(S_T), _ptr(work), ws, _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st)
    return o, S_T


def chunk_backward(q, k, v, a, b, w, S0, dO, dS_T=None, want_dS0: bool = True, grads=None, workspace=None,
                   stream=None) -> dict:
    """Gradients of chunk_forward. Inputs as chunk_forward, plus dO (like o)
    and dS_T (like S_T, or None for zero). Returns a dict with dq, dk, dv (the
    input dtype), da, db, dw (fp32) and dS0 (fp32, or None without want_dS0).
    `grads` may hold preallocated outputs under those names, and `workspace`
    a uint8 device tensor of at least gdn2_chunk_backward_workspace_bytes."""
    return _backward(q, k, v, a, b, w, S0, dO, dS_T, None, want_dS0, grads, workspace, stream)


def chunk_backward_preact(q, k, v, a_pre, b_pre, w_pre, S0, dO, dS_T=None, want_dS0: bool = True, grads=None,
                          workspace=None, stream=None) -> dict:
    """Gradients of chunk_forward_preact: as chunk_backward, with da, db, dw
    the gradients of the gate pre-activations, in the input dtype."""
    return _backward(q, k, v, a_pre, b_pre, w_pre, S0, dO, dS_T, None, want_dS0, grads, workspace, stream,
                     form="preact")


def chunk_backward_coupled(q, k, v, a, beta, S0, dO, dS_T=None, want_dS0: bool = True, grads=None,
                           workspace=None, stream=None) -> dict:
    """Gradients of chunk_forward_coupled: dq, dk, dv, da (like a), db (the
    gradient of beta, [B,T,H_v] fp32: erase and write uses together) and dS0;
    no dw."""
    return _backward(q, k, v, a, beta, None, S0, dO, dS_T, None, want_dS0, grads, workspace, stream,
                     form="coupled")


def chunk_backward_scalar(q, k, v, alpha, beta, S0, dO, dS_T=None, want_dS0: bool = True, grads=None,
                          workspace=None, stream=None) -> dict:
    """Gradients of chunk_forward_scalar: as chunk_backward_coupled, with da
    the gradient of alpha ([B,T,H_v] fp32)."""
    return _backward(q, k, v, alpha, beta, None, S0, dO, dS_T, None, want_dS0, grads, workspace, stream,
                     form="scalar")


def chunk_backward_varlen(q, k, v, a, b, w, cu_seqlens, S0, dO, dS_T=None, want_dS0: bool = True, grads=None,
                          workspace=None, stream=None, gates: str = "channel") -> dict:
    """Gradients of chunk_forward_varlen (packed sequences; shapes and `gates`
    as there, dO like v, dS_T [N,H_v,d_k,d_v] or None). Returns the dict of
    chunk_backward, token gradients shaped like their inputs (no dw for the
    coupled and scalar forms, whose db is the gradient of beta)."""
    form = {"channel": "general"}.get(gates, gates)
    if form not in ("general", "preact", "coupled", "scalar"):
        raise ValueError(f"unknown gate form {gates}")
    return _backward(q, k, v, a, b, w, S0, dO, dS_T, cu_seqlens, want_dS0, grads, workspace, stream, form=form)


def _backward(q, k, v, a, b, w, S0, dO, dS_T, cu, want_dS0, grads, workspace, stream, form="general") -> dict:
    import torch
    T, H_qk, d_k = q.shape[-3:]
    H_v, d_v = v.shape[-2], v.shape[-1]
    dev = q.device
    if cu is None:
        B, T, H_qk, H_v, d_k, d_v = _dims(q, v)
        chk = lambda t, nm, tail, dt: _want(t, nm, (B, T) + tuple(tail), dt, dev)
    else:
        _want(cu, "cu_seqlens", (cu.numel(),), torch.int32, dev)
        B = cu.numel() - 1
        if B < 0:
            raise ValueError("cu_seqlens needs at least one offset")
        chk = lambda t, nm, tail, dt: _want_rows(t, nm, T, tail, dt, dev)
    _check_gate_form(chk, q, k, v, a, b, w, form, H_qk, H_v, d_k, d_v)
    chk(dO, "dO", (H_v, d_v), q.dtype)
    preact, coupled = form == "preact", form in ("coupled", "scalar")
    gdt = q.dtype if preact else torch.float32  # gates (and their gradients)
    for t, nm in ((S0, "S0"), (dS_T, "dS_T")):
        _want(t, nm, (B, H_v, d_k, d_v), torch.float32, dev)
    g = dict(grads or {})
    shapes = {"dq": (q.shape, q.dtype), "dk": (k.shape, q.dtype), "dv": (v.shape, q.dtype),
              "da": (a.shape, gdt), "db": (b.shape, gdt)}
    if not coupled:
        shapes["dw"] = (w.shape, gdt)
    if want_dS0:
        shapes["dS0"] = ((B, H_v, d_k, d_v), torch.float32)
    for nm, (shape, dt) in shapes.items():
        if g.get(nm) is None:
            g[nm] = torch.empty(shape, dtype=dt, device=dev)
        _want(g[nm], nm, shape, dt, dev)
    g.setdefault("dS0", None)
    g.setdefault("dw", None)
    desc = make_desc(B, T, H_qk, H_v, d_k, d_v, 64, _dtype_code(q))
    ws = (gdn2_chunk_backward_workspace_bytes(desc) if cu is None
          else gdn2_chunk_backward_varlen_workspace_bytes(desc))
    if workspace is None and ws:
        workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _want(workspace, "workspace", (workspace.numel(),), torch.uint8, dev)
    wbytes = workspace.numel() if workspace is not None else 0
    ptrs = (_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(w), _ptr(S0), _ptr(dO), _ptr(dS_T), _ptr(g["dq"]),
            _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["da"]), _ptr(g["db"]), _ptr(g["dw"]), _ptr(g["dS0"]),
            _ptr(workspace), wbytes, _stream(stream))
    if cu is not None and form != "general":
        st = gdn2_chunk_backward_varlen_gates(desc, _ptr(cu), GDN2_GATES["channel" if form == "general" else form],
                                              *ptrs)
    elif coupled:
        entry = gdn2_chunk_backward_coupled if form == "coupled" else gdn2_chunk_backward_scalar
        st = entry(desc, *(ptrs[:5] + ptrs[6:14] + ptrs[15:]))
    elif preact:
        st = gdn2_chunk_backward_preact(desc, *ptrs)
    elif cu is None:
        st = gdn2_chunk_backward(desc, *ptrs)
    else:
        st = gdn2_chunk_backward_varlen(desc, _ptr(cu), *ptrs)
    if st != GDN2_OK:
        raise Gdn2Error(st)
    return g


def chunk_forward_preact(q, k, v, a_pre, b_pre, w_pre, S0=None, chunk: int = 64, o=None, S_T=None,
                         want_state: bool = True, stream=None):
    """Prefill with the per-channel gates given as pre-activations in the
    input dtype (decay a = exp(-softplus(a_pre)), b = sigmoid(b_pre),
    w = sigmoid(w_pre)), activated in the kernel. Shapes as chunk_forward."""
    import torch
    B, T, H_qk, H_v, d_k, d_v = _dims(q, v)
    dev, f32 = q.device, torch.float32
    _want(q, "q", (B, T, H_qk, d_k), q.dtype, dev)
    _want(k, "k", (B, T, H_qk, d_k), q.dtype, dev)
    _want(v, "v", (B, T, H_v, d_v), q.dtype, dev)
    _want(a_pre, "a_pre", (B, T, H_v, d_k), q.dtype, dev)
    _want(b_pre, "b_pre", (B, T, H_v, d_k), q.dtype, dev)
    _want(w_pre, "w_pre", (B, T, H_v, d_v), q.dtype, dev)
    _want(S0, "S0", (B, H_v, d_k, d_v), f32, dev)
    if o is None:
        o = torch.empty((B, T, H_v, d_v), dtype=q.dtype, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H_v, d_k, d_v), dtype=f32, device=dev)
    _want(o, "o", (B, T, H_v, d_v), q.dtype, dev)
    _want(S_T, "S_T", (B, H_v, d_k, d_v), f32, dev)
    desc = make_desc(B, T, H_qk, H_v, d_k, d_v, chunk, _dtype_code(q))
    ws = gdn2_chunk_forward_workspace_bytes(desc)
    work = torch.empty(ws, dtype=torch.uint8, device=dev) if ws else None
    st = gdn2_chunk_forward_preact(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(a_pre), _ptr(b_pre), _ptr(w_pre),
                                   _ptr(S0), _ptr(o), _ptr(S_T), _ptr(work), ws, _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st)
    return o, S_T


def chunk_forward_coupled(q, k, v, a, beta, S0=None, chunk: int = 64, o=None, S_T=None,
                          want_state: bool = True, stream=None):
    """Prefill with coupled gates b = w = beta (one scalar per token and value
    head). q, k [B,T,H_qk,d_k]; v [B,T,H_v,d_v]; a [B,T,H_v,d_k] fp32;
    beta [B,T,H_v] fp32; S0 [B,H_v,d_k,d_v] fp32 or None. Returns (o, S_T)."""
    return _forward_scalar_gates(gdn2_chunk_forward_coupled, False, q, k, v, a, beta, S0, chunk, o, S_T,
                                 want_state, stream)


def chunk_forward_scalar(q, k, v, alpha, beta, S0=None, chunk: int = 64, o=None, S_T=None,
                         want_state: bool = True, stream=None):
    """Prefill with scalar gates (Gated DeltaNet form): decay alpha and coupled
    erase/write gate beta, each [B,T,H_v] fp32. Other arguments as chunk_forward."""
    return _forward_scalar_gates(gdn2_chunk_forward_scalar, True, q, k, v, alpha, beta, S0, chunk, o, S_T,
                                 want_state, stream)


def _forward_scalar_gates(entry, scalar_decay, q, k, v, a, beta, S0, chunk, o, S_T, want_state, stream):
    import torch
    B, T, H_qk, H_v, d_k, d_v = _dims(q, v)
    dev, f32 = q.device, torch.float32
    _want(q, "q", (B, T, H_qk, d_k), q.dtype, dev)
    _want(k, "k", (B, T, H_qk, d_k), q.dtype, dev)
    _want(v, "v", (B, T, H_v, d_v), q.dtype, dev)
    _want(a, "alpha" if scalar_decay else "a", (B, T, H_v) if scalar_decay else (B, T, H_v, d_k), f32, dev)
    _want(beta, "beta", (B, T, H_v), f32, dev)
    _want(S0, "S0", (B, H_v, d_k, d_v), f32, dev)
    if o is None:
        o = torch.empty((B, T, H_v, d_v), dtype=q.dtype, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H_v, d_k, d_v), dtype=f32, device=dev)
    _want(o, "o", (B, T, H_v, d_v), q.dtype, dev)
    _want(S_T, "S_T", (B, H_v, d_k, d_v), f32, dev)
    desc = make_desc(B, T, H_qk, H_v, d_k, d_v, chunk, _dtype_code(q))
    ws = gdn2_chunk_forward_workspace_bytes(desc)
    work = torch.empty(ws, dtype=torch.uint8, device=dev) if ws else None
    st = entry(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T), _ptr(work), ws,
               _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st)
    return o, S_T


GDN2_GATES = {"channel": 0, "preact": 1, "coupled": 2, "scalar": 3}


def _check_gate_form(chk, q, k, v, a, b, w, gates, H_qk, H_v, d_k, d_v):
    """Token tensors of gate form `gates`; chk(t, name, tail, dtype) checks
    one tensor against its token dimensions followed by `tail`."""
    import torch
    if H_v % H_qk:
        raise ValueError(f"value heads ({H_v}) must be a multiple of query/key heads ({H_qk})")
    chk(q, "q", (H_qk, d_k), q.dtype)
    chk(k, "k", (H_qk, d_k), q.dtype)
    chk(v, "v", (H_v, d_v), q.dtype)
    if gates in ("channel", "general", "preact"):
        gdt = q.dtype if gates == "preact" else torch.float32
        if a is None or b is None or w is None:
            raise ValueError(f"a, b and w are required for gates={gates!r}")
        chk(a, "a", (H_v, d_k), gdt)
        chk(b, "b", (H_v, d_k), gdt)
        chk(w, "w", (H_v, d_v), gdt)
    elif gates in ("coupled", "scalar"):
        if a is None or b is None:
            raise ValueError(f"a (alpha) and beta are required for gates={gates!r}")
        chk(a, "alpha" if gates == "scalar" else "a", (H_v,) if gates == "scalar" else (H_v, d_k), torch.float32)
        chk(b, "beta", (H_v,), torch.float32)
    else:
        raise ValueError(f"unknown gate form {gates}")


def _check_packed(q, k, v, a, b, w, gates, T, H_qk, H_v, d_k, d_v, dev):
    """Token tensors of a packed ([T, H, d], or with leading 1s) problem."""
    _check_gate_form(lambda t, nm, tail, dt: _want_rows(t, nm, T, tail, dt, dev),
                     q, k, v, a, b, w, gates, H_qk, H_v, d_k, d_v)


def chunk_forward_varlen(q, k, v, a, b, w, cu_seqlens, S0=None, chunk: int = 64, o=None, S_T=None,
                         want_state: bool = True, stream=None, gates: str = "channel"):
    """Prefill of packed sequences of different lengths. q, k [T,H_qk,d_k] (or
    [1,T,H_qk,d_k]); v [T,H_v,d_v]; a, b [T,H_v,d_k] fp32; w [T,H_v,d_v] fp32;
    cu_seqlens int32 [N+1] on the device (sequence n = tokens cu[n]..cu[n+1]-1);
    S0 [N,H_v,d_k,d_v] fp32 or None. Returns (o shaped like v, S_T [N,H_v,d_k,d_v]).
    `gates` selects the gate form: "channel" (as above), "preact" (a, b, w as
    pre-activations in the input dtype), "coupled" (b = beta [T,H_v] fp32,
    w None), "scalar" (a = alpha and b = beta, each [T,H_v] fp32, w None)."""
    import torch
    T, H_qk, d_k = q.shape[-3:]
    H_v, d_v = v.shape[-2], v.shape[-1]
    if gates not in GDN2_GATES:
        raise ValueError(f"unknown gate form {gates}")
    form = GDN2_GATES[gates]
    dev, f32 = q.device, torch.float32
    _want(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32, dev)
    N = cu_seqlens.numel() - 1
    if N < 0:
        raise ValueError("cu_seqlens needs at least one offset")
    _check_packed(q, k, v, a, b, w, gates, T, H_qk, H_v, d_k, d_v, dev)
    _want(S0, "S0", (N, H_v, d_k, d_v), f32, dev)
    if o is None:
        o = torch.empty(v.shape, dtype=q.dtype, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((N, H_v, d_k, d_v), dtype=f32, device=dev)
    _want(o, "o", v.shape, q.dtype, dev)
    _want(S_T, "S_T", (N, H_v, d_k, d_v), f32, dev)
    desc = make_desc(N, T, H_qk, H_v, d_k, d_v, chunk, _dtype_code(q))
    st = gdn2_chunk_forward_varlen_gates(desc, _ptr(cu_seqlens), form, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                         _ptr(w), _ptr(S0), _ptr(o), _ptr(S_T), _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st)
    return o, S_T


def decode_step(q, k, v, a, b, w, S, o=None, stream=None, gates: str = "channel"):
    """One decode token. q, k [N,1,H_qk,d_k] (or [N,H_qk,d_k]); v [N,1,H_v,d_v];
    a, b [N,1,H_v,d_k]; w [N,1,H_v,d_v]; S [N,H_v,d_k,d_v] fp32, updated in place.
    Returns o shaped like v. `gates` as for chunk_forward_varlen: "preact"
    (a, b, w pre-activations in the input dtype), "coupled" (b = beta
    [N,1,H_v] fp32, w None), "scalar" (a = alpha, b = beta, each [N,1,H_v])."""
    import torch
    if S.dim() != 4:
        raise ValueError(f"S must be [N, H_v, d_k, d_v], got {tuple(S.shape)}")
    N, H_v, d_k, d_v = S.shape
    H_qk = q.shape[-2]
    if gates not in GDN2_GATES:
        raise ValueError(f"unknown gate form {gates}")
    form = GDN2_GATES[gates]
    dev = q.device
    _want(S, "S", (N, H_v, d_k, d_v), torch.float32, dev)
    # one token per sequence: [N, 1, H, d] or [N, H, d]
    one = lambda t, tail: None if t is None else (tuple(t.shape) in ((N, 1) + tail, (N,) + tail))
    for t, nm, tail in ((q, "q", (H_qk, d_k)), (k, "k", (H_qk, d_k)), (v, "v", (H_v, d_v))):
        _check(t, nm, q.dtype)
        if not one(t, tail) or t.device != dev:
            raise ValueError(f"{nm} must be [N, 1, {tail[0]}, {tail[1]}] on {dev}, got {tuple(t.shape)}")
    gshape = {"a": (H_v,) if gates == "scalar" else (H_v, d_k),
              "b": (H_v,) if gates in ("coupled", "scalar") else (H_v, d_k), "w": (H_v, d_v)}
    gdt = q.dtype if gates == "preact" else torch.float32
    for t, nm in ((a, "a"), (b, "b"), (w, "w")):
        if nm == "w" and gates in ("coupled", "scalar"):
            continue
        if t is None:
            raise ValueError(f"{nm} is required for gates={gates!r}")
        _check(t, nm, gdt)
        if not one(t, gshape[nm]) or t.device != dev:
            raise ValueError(f"{nm} must be [N, 1, {', '.join(map(str, gshape[nm]))}] on {dev}, "
                             f"got {tuple(t.shape)}")
    if o is None:
        o = torch.empty(v.shape, dtype=q.dtype, device=dev)
    _want(o, "o", v.shape, q.dtype, dev)
    desc = make_desc(N, 1, H_qk, H_v, d_k, d_v, 64, _dtype_code(q))
    st = gdn2_decode_step_gates(desc, form, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(w), _ptr(S),
                                _ptr(o), _stream(stream))
    if st != GDN2_OK:
        raise Gdn2Error(st)
    return o


# ------------------------------------------------------------------ autograd
def _autograd_function():
    import torch

    class GatedDeltaRule2(torch.autograd.Function):
        """o, S_T = prefill(q, k, v, a, b, w, S0); backward through
        gdn2_chunk_backward. The saved tensors are the inputs themselves."""

        @staticmethod
        def forward(ctx, q, k, v, a, b, w, S0, chunk):
            o, S_T = chunk_forward(q, k, v, a, b, w, S0, chunk=chunk)
            ctx.save_for_backward(q, k, v, a, b, w, S0)
            return o, S_T

        @staticmethod
        def backward(ctx, dO, dS_T):
            q, k, v, a, b, w, S0 = ctx.saved_tensors
            g = chunk_backward(q, k, v, a, b, w, S0, dO.contiguous(),
                               None if dS_T is None else dS_T.contiguous(), want_dS0=S0 is not None)
            return g["dq"], g["dk"], g["dv"], g["da"], g["db"], g["dw"], g["dS0"], None

    return GatedDeltaRule2


_GDR2 = None
_GDR2P = None


def _autograd_function_preact():
    import torch

    class GatedDeltaRule2Preact(torch.autograd.Function):
        """gated_delta_rule with the gates as pre-activations (chunk_forward_preact
        / gdn2_chunk_backward_preact)."""

        @staticmethod
        def forward(ctx, q, k, v, a_pre, b_pre, w_pre, S0, chunk):
            o, S_T = chunk_forward_preact(q, k, v, a_pre, b_pre, w_pre, S0, chunk=chunk)
            ctx.save_for_backward(q, k, v, a_pre, b_pre, w_pre, S0)
            return o, S_T

        @staticmethod
        def backward(ctx, dO, dS_T):
            q, k, v, a_pre, b_pre, w_pre, S0 = ctx.saved_tensors
            g = chunk_backward_preact(q, k, v, a_pre, b_pre, w_pre, S0, dO.contiguous(),
                                      None if dS_T is None else dS_T.contiguous(), want_dS0=S0 is not None)
            return g["dq"], g["dk"], g["dv"], g["da"], g["db"], g["dw"], g["dS0"], None

    return GatedDeltaRule2Preact


def gated_delta_rule_preact(q, k, v, a_pre, b_pre, w_pre, S0=None, chunk: int = 64):
    """Differentiable prefill with the gates as pre-activations in the input
    dtype (decay a = exp(-softplus(a_pre)), b = sigmoid(b_pre),
    w = sigmoid(w_pre)); gradients reach the pre-activations."""
    global _GDR2P
    if _GDR2P is None:
        _GDR2P = _autograd_function_preact()
    return _GDR2P.apply(q, k, v, a_pre, b_pre, w_pre, S0, chunk)


def gated_delta_rule(q, k, v, a, b, w, S0=None, chunk: int = 64):
    """Differentiable prefill for PyTorch training: returns (o, S_T) like
    chunk_forward; gradients of q, k, v, a, b, w and S0 come from
    gdn2_chunk_backward."""
    global _GDR2
    if _GDR2 is None:
        _GDR2 = _autograd_function()
    return _GDR2.apply(q, k, v, a, b, w, S0, chunk)


_GDR2C = {}


def _autograd_function_scalar_gates(form: str):
    import torch
    fwd = chunk_forward_coupled if form == "coupled" else chunk_forward_scalar
    bwd = chunk_backward_coupled if form == "coupled" else chunk_backward_scalar

    class GatedDeltaRule2ScalarGates(torch.autograd.Function):
        """gated_delta_rule with the coupled gate beta (and, in the scalar form,
        the scalar decay alpha): chunk_forward_coupled / chunk_forward_scalar
        and their backward passes."""

        @staticmethod
        def forward(ctx, q, k, v, a, beta, S0, chunk):
            o, S_T = fwd(q, k, v, a, beta, S0, chunk=chunk)
            ctx.save_for_backward(q, k, v, a, beta, S0)
            return o, S_T

        @staticmethod
        def backward(ctx, dO, dS_T):
            q, k, v, a, beta, S0 = ctx.saved_tensors
            g = bwd(q, k, v, a, beta, S0, dO.contiguous(), None if dS_T is None else dS_T.contiguous(),
                    want_dS0=S0 is not None)
            return g["dq"], g["dk"], g["dv"], g["da"], g["db"], g["dS0"], None

    return GatedDeltaRule2ScalarGates


def gated_delta_rule_coupled(q, k, v, a, beta, S0=None, chunk: int = 64):
    """Differentiable prefill with coupled erase/write gates b = w = beta
    ([B,T,H_v] fp32) and a per-channel decay a; gradients reach beta through
    both of its uses."""
    if "coupled" not in _GDR2C:
        _GDR2C["coupled"] = _autograd_function_scalar_gates("coupled")
    return _GDR2C["coupled"].apply(q, k, v, a, beta, S0, chunk)


def gated_delta_rule_scalar(q, k, v, alpha, beta, S0=None, chunk: int = 64):
    """Differentiable prefill in the Gated DeltaNet form: scalar decay alpha
    and coupled gate beta, each [B,T,H_v] fp32."""
    if "scalar" not in _GDR2C:
        _GDR2C["scalar"] = _autograd_function_scalar_gates("scalar")
    return _GDR2C["scalar"].apply(q, k, v, alpha, beta, S0, chunk)


_GDR2V = None


def _autograd_function_varlen():
    import torch

    class GatedDeltaRule2Varlen(torch.autograd.Function):
        """Packed sequences in any gate form: chunk_forward_varlen /
        chunk_backward_varlen with the same `gates`."""

        @staticmethod
        def forward(ctx, q, k, v, a, b, w, cu_seqlens, S0, chunk, gates):
            o, S_T = chunk_forward_varlen(q, k, v, a, b, w, cu_seqlens, S0, chunk=chunk, gates=gates)
            ctx.save_for_backward(q, k, v, a, b, w, cu_seqlens, S0)
            ctx.gates = gates
            return o, S_T

        @staticmethod
        def backward(ctx, dO, dS_T):
            q, k, v, a, b, w, cu, S0 = ctx.saved_tensors
            g = chunk_backward_varlen(q, k, v, a, b, w, cu, S0, dO.contiguous(),
                                      None if dS_T is None else dS_T.contiguous(), want_dS0=S0 is not None,
                                      gates=ctx.gates)
            return g["dq"], g["dk"], g["dv"], g["da"], g["db"], g.get("dw"), None, g["dS0"], None, None

    return GatedDeltaRule2Varlen


def gated_delta_rule_varlen(q, k, v, a, b, w, cu_seqlens, S0=None, chunk: int = 64, gates: str = "channel"):
    """Differentiable prefill of packed sequences (cu_seqlens, one state per
    sequence) in any gate form (`gates` as for chunk_forward_varlen; w is None
    for "coupled" and "scalar"); returns (o, S_T [N,H_v,d_k,d_v])."""
    global _GDR2V
    if _GDR2V is None:
        _GDR2V = _autograd_function_varlen()
    return _GDR2V.apply(q, k, v, a, b, w, cu_seqlens, S0, chunk, gates)
