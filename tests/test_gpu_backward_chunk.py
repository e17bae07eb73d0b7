"""Parity of the chunk-form backward (bf16 inputs, d_k = d_v = 128,
per-channel gates: the prefill's states at every chunk boundary, the state's
adjoint swept over chunks, every gradient of a chunk on the matrix cores)
with the fp64 oracle's gradients.

GDN2_BACKWARD_CHUNKED=2 makes the library fail instead of falling back to
the per-token backward, so these tests check the chunk form itself. The
cases: whole and ragged chunks and sequences shorter than one chunk, grouped
heads, absent S0 / dS_T, decays that need the middle anchor, and decays too
fast for either anchor (the library then runs the per-token backward, and
refuses when the chunk form is required). Tolerance: the bf16 bar, 2e-2
normwise per gradient tensor, and per (sequence, head) slice."""
import numpy as np
import pytest
import torch

import gated_delta_rule_83_amd as g
from gated_delta_rule_83_amd import inputs as gi
from tests.parity import rand_inputs
from tests.test_gpu_backward import compare, per_head_error, upstream

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("B,T,Hqk,Hv", [(2, 32, 1, 1), (2, 3 * 32 + 11, 1, 2), (1, 5, 2, 2), (1, 200, 2, 4)])
def test_chunk_form_matches_oracle(B, T, Hqk, Hv, monkeypatch):
    monkeypatch.setenv("GDN2_BACKWARD_CHUNKED", "2")
    rng = np.random.default_rng(5000 + T + 7 * Hv)
    d = rand_inputs(rng, B, T, Hqk, Hv, 128, 128)
    td = gi.to_torch(d, "bf16", DEV)
    dO, dST = upstream(rng, d, "bf16")
    compare(td, dO, dST, "bf16", f"chunk form B{B} T{T} Hqk{Hqk} Hv{Hv}")


def test_chunk_form_without_state(monkeypatch):
    """S0 and dS_T absent (zero)."""
    monkeypatch.setenv("GDN2_BACKWARD_CHUNKED", "2")
    rng = np.random.default_rng(5100)
    d = rand_inputs(rng, 2, 70, 1, 1, 128, 128, with_s0=False)
    td = gi.to_torch(d, "bf16", DEV)
    dO, _ = upstream(rng, d, "bf16", with_dst=False)
    compare(td, dO, None, "bf16", "chunk form no S0/dS_T")


def _decays(rng, shape, lo, hi):
    return np.exp(-rng.uniform(lo, hi, shape)).astype(np.float32)


def test_chunk_form_middle_anchor(monkeypatch):
    """Some channels decay by about e^-80 over a chunk (e^-40 per half): the
    chunks take the anchor at their middle token."""
    monkeypatch.setenv("GDN2_BACKWARD_CHUNKED", "2")
    rng = np.random.default_rng(5200)
    d = rand_inputs(rng, 1, 2 * 32 + 9, 1, 2, 128, 128)
    d["a"][..., :8] = _decays(rng, d["a"][..., :8].shape, 2.2, 2.8)
    td = gi.to_torch(d, "bf16", DEV)
    dO, dST = upstream(rng, d, "bf16")
    compare(td, dO, dST, "bf16", "chunk form middle anchor")


def test_fast_decay_falls_back_to_token_steps(monkeypatch):
    """One channel decays by about e^-90 within each half chunk: neither
    anchor keeps the operands below e^60, so the chunk form refuses when
    required, and the automatic choice runs the per-token backward."""
    rng = np.random.default_rng(5300)
    d = rand_inputs(rng, 1, 64, 1, 1, 128, 128)
    d["a"][..., 3] = _decays(rng, d["a"][..., 3].shape, 5.5, 6.0)
    td = gi.to_torch(d, "bf16", DEV)
    dO, dST = upstream(rng, d, "bf16")
    monkeypatch.setenv("GDN2_BACKWARD_CHUNKED", "2")
    with pytest.raises(RuntimeError):
        g.chunk_backward(td["q"], td["k"], td["v"], td["a"], td["b"], td["w"], td["S0"], dO, dST)
    torch.cuda.synchronize()
    monkeypatch.delenv("GDN2_BACKWARD_CHUNKED")
    compare(td, dO, dST, "bf16", "fast decay, per-token fallback")


def test_chunk_form_layer_distributions(monkeypatch):
    """The 1.3B-class layer's gate distributions (decay pre-activation
    N(-4, 1)) at B2 H4 T520, against the oracle."""
    monkeypatch.setenv("GDN2_BACKWARD_CHUNKED", "2")
    c = gi.scaled(1, B=2, T=520, H_qk=4, H_v=4)
    d = gi.make_inputs(c)
    rng = np.random.default_rng(5400)
    td = gi.to_torch(d, "bf16", DEV)
    dO, dST = upstream(rng, d, "bf16")
    compare(td, dO, dST, "bf16", "chunk form c1-scaled")


def _heads_vs_oracle(td, dO, dST, gg, pairs, label):
    """Gradients of (sequence n, value head h) against the oracle run on that
    pair alone (one query/key head per value head)."""
    import oracle
    from tests.parity import TOL, normwise, to_np
    for (n, h) in pairs:
        sl = lambda x: x[n:n + 1, :, h:h + 1].contiguous()
        ref = oracle.backward(sl(td["q"]), sl(td["k"]), sl(td["v"]), sl(td["a"]), sl(td["b"]), sl(td["w"]),
                              None if td["S0"] is None else td["S0"][n:n + 1, h:h + 1].contiguous(), sl(dO),
                              dST[n:n + 1, h:h + 1].contiguous())
        errs = {nm: normwise(to_np(gg[nm][n:n + 1, :, h:h + 1] if nm != "dS0" else gg[nm][n:n + 1, h:h + 1]),
                             ref[nm]) for nm in ("dq", "dk", "dv", "da", "db", "dw", "dS0")}
        print(f"[{label} n{n} h{h}] " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
        bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
        assert not bad, ((n, h), bad)


def test_chunk_form_long_context_sampled_heads(monkeypatch):
    """B1 T65536 H16 d128 bf16 with 1% hard erases (the long-context shape):
    the chunk form, three heads against the oracle."""
    monkeypatch.setenv("GDN2_BACKWARD_CHUNKED", "2")
    c = gi.config(2)
    d = gi.make_inputs(c)
    rng = np.random.default_rng(5500)
    td = gi.to_torch(d, "bf16", DEV)
    dO, dST = upstream(rng, d, "bf16")
    gg = g.chunk_backward(td["q"], td["k"], td["v"], td["a"], td["b"], td["w"], td["S0"], dO, dST)
    torch.cuda.synchronize()
    _heads_vs_oracle(td, dO, dST, gg, ((0, 0), (0, 7), (0, 15)), "chunk form long context")


def test_chunk_form_layer_shape_sampled_heads(monkeypatch):
    """B8 T4096 H16 d128 bf16 (the layer shape): the chunk form, four
    (sequence, head) pairs against the oracle."""
    monkeypatch.setenv("GDN2_BACKWARD_CHUNKED", "2")
    c = gi.config(1)
    d = gi.make_inputs(c)
    rng = np.random.default_rng(5600)
    td = gi.to_torch(d, "bf16", DEV)
    dO, dST = upstream(rng, d, "bf16")
    gg = g.chunk_backward(td["q"], td["k"], td["v"], td["a"], td["b"], td["w"], td["S0"], dO, dST)
    torch.cuda.synchronize()
    _heads_vs_oracle(td, dO, dST, gg, ((0, 0), (3, 5), (5, 11), (7, 15)), "chunk form layer shape")


@pytest.mark.parametrize("scalar", [False, True])
def test_chunk_form_coupled_layer_shape_sampled_heads(scalar, monkeypatch):
    """The layer shape (B8 T4096 H16 d128 bf16) in the coupled and scalar gate
    forms (beta, and alpha, = the drawn gates' first channel per token and
    value head): the chunk form, four (sequence, head) pairs against the
    oracle's gradients through the broadcasts, dbeta (and dalpha) included."""
    import oracle
    from tests.parity import TOL, normwise, to_np
    monkeypatch.setenv("GDN2_BACKWARD_CHUNKED", "2")
    c = gi.config(1)
    d = gi.make_inputs(c)
    rng = np.random.default_rng(5700 + scalar)
    beta = torch.from_numpy(np.ascontiguousarray(d["b"][..., 0])).to(DEV)
    td = gi.to_torch(d, "bf16", DEV)
    a = torch.from_numpy(np.ascontiguousarray(d["a"][..., 0])).to(DEV) if scalar else td["a"]
    dO, dST = upstream(rng, d, "bf16")
    fn = g.chunk_backward_scalar if scalar else g.chunk_backward_coupled
    gg = fn(td["q"], td["k"], td["v"], a, beta, td["S0"], dO, dST)
    torch.cuda.synchronize()
    for (n, h) in ((0, 0), (3, 5), (5, 11), (7, 15)):
        sl = lambda x: x[n:n + 1, :, h:h + 1].contiguous()
        ref = oracle.backward_coupled(sl(td["q"]), sl(td["k"]), sl(td["v"]), sl(a), sl(beta),
                                      None if td["S0"] is None else td["S0"][n:n + 1, h:h + 1].contiguous(),
                                      sl(dO), dST[n:n + 1, h:h + 1].contiguous(), scalar_decay=scalar)
        errs = {nm: normwise(to_np(gg[nm][n:n + 1, :, h:h + 1] if nm != "dS0" else gg[nm][n:n + 1, h:h + 1]),
                             ref[nm]) for nm in ("dq", "dk", "dv", "da", "db", "dS0")}
        print(f"[chunk form {'scalar' if scalar else 'coupled'} layer shape n{n} h{h}] "
              + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
        bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
        assert not bad, ((n, h), bad)


def test_chunk_form_preact_layer_shape_sampled_heads(monkeypatch):
    """The layer shape (B8 T4096 H16 d128 bf16) with bf16 gate pre-activations:
    the chunk form (its chunk states from the prefill whose column waves
    activate the erase gates), four (sequence, head) pairs against the
    oracle's gradients through the activations."""
    import oracle
    from tests.parity import TOL, normwise, to_np
    monkeypatch.setenv("GDN2_BACKWARD_CHUNKED", "2")
    c = gi.config(1)
    d = gi.make_preact_inputs(c)
    rng = np.random.default_rng(5800)
    td = gi.to_torch_preact(d, "bf16", DEV)
    dO, dST = upstream(rng, d, "bf16")
    gg = g.chunk_backward_preact(td["q"], td["k"], td["v"], td["a"], td["b"], td["w"], td["S0"], dO, dST)
    torch.cuda.synchronize()
    for (n, h) in ((0, 0), (3, 5), (5, 11), (7, 15)):
        sl = lambda x: x[n:n + 1, :, h:h + 1].contiguous()
        ref = oracle.backward_preact(sl(td["q"]), sl(td["k"]), sl(td["v"]), sl(td["a"]), sl(td["b"]), sl(td["w"]),
                                     None if td["S0"] is None else td["S0"][n:n + 1, h:h + 1].contiguous(),
                                     sl(dO), dST[n:n + 1, h:h + 1].contiguous())
        errs = {nm: normwise(to_np(gg[nm][n:n + 1, :, h:h + 1] if nm != "dS0" else gg[nm][n:n + 1, h:h + 1]),
                             ref[nm]) for nm in ("dq", "dk", "dv", "da", "db", "dw", "dS0")}
        print(f"[chunk form preact layer shape n{n} h{h}] " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()),
              flush=True)
        bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
        assert not bad, ((n, h), bad)


@pytest.mark.parametrize("form,T", [("channel", 1100), ("preact", 1100), ("coupled", 1100), ("scalar", 1100),
                                    ("scalar", 520), ("channel", 520)])
def test_per_token_rounds_in_chunk_workspace(form, T, monkeypatch):
    """Where the chunk form's shape applies (bf16, d_k = d_v = 128) the
    workspace query returns the chunk form's size, smaller than the per-token
    backward needs at once; the per-token backward (for decays too fast for
    the chunk form: here key channel 5 decays by about e^-90 within each half
    chunk, or every channel in the scalar form) then runs in rounds of
    segments within it. B2, T1100 (3 segments
    of 384 tokens, the last ragged) and T520 (3 of 256, the last shorter than
    a chunk: asked for 2 segments, which the prefill's plan turns into 3),
    two value heads per query/key head, S0 and dS_T: against the oracle of
    the form."""
    from tests.gate_forms import backward_alone, form_inputs, oracle_backward
    from tests.parity import TOL, normwise, to_np
    monkeypatch.delenv("GDN2_BACKWARD_CHUNKED", raising=False)
    rng = np.random.default_rng(5700 + len(form) + T)
    B, Hv = 2, 2
    x = form_inputs(rng, form, T, Hv, 128, 128, "bf16", DEV, B=B)
    a = x["a"].clone()
    fast = lambda y: torch.empty_like(y, dtype=torch.float32).uniform_(5.5, 6.0)
    if form == "preact":  # a = 1 / (1 + e^x): x in [5.5, 6]
        a[..., 5] = fast(a[..., 5]).to(a.dtype)
    elif form == "scalar":
        a = torch.exp(-fast(a))
    else:
        a[..., 5] = torch.exp(-fast(a[..., 5]))
    x["a"] = a
    desc = g.make_desc(B, T, 1, Hv, 128, 128, 64, g.GDN2_BF16)
    ws = g.gdn2_chunk_backward_workspace_bytes(desc)
    monkeypatch.setenv("GDN2_BACKWARD_CHUNKED", "0")
    assert g.gdn2_chunk_backward_workspace_bytes(desc) > ws  # the per-token backward at once needs more
    monkeypatch.delenv("GDN2_BACKWARD_CHUNKED")
    S0 = torch.from_numpy((rng.standard_normal((B, Hv, 128, 128)) * 0.5).astype(np.float32)).to(DEV)
    dO = torch.from_numpy(rng.standard_normal((B, T, Hv, 128)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    dST = torch.from_numpy(rng.standard_normal((B, Hv, 128, 128)).astype(np.float32)).to(DEV)
    got = backward_alone(form, x, S0, dO, dST)
    torch.cuda.synchronize()
    ref = oracle_backward(form, x, S0, dO, dST)
    names = [nm for nm in ("dq", "dk", "dv", "da", "db", "dw", "dS0") if got.get(nm) is not None]
    errs = {nm: normwise(to_np(got[nm]), ref[nm]) for nm in names}
    errs.update({nm + " per head": per_head_error(to_np(got[nm]), ref[nm], (0, 1) if nm == "dS0" else (0, 2))
                 for nm in names})
    print(f"[per-token rounds {form}] " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
    assert not bad, bad


@pytest.mark.parametrize("form,B,T,Hqk,Hv", [("preact", 2, 107, 1, 2), ("coupled", 2, 107, 1, 2),
                                            ("scalar", 2, 107, 1, 2), ("preact", 1, 200, 2, 2),
                                            ("coupled", 1, 200, 2, 2), ("scalar", 1, 200, 2, 2)])
def test_chunk_form_gate_forms(form, B, T, Hqk, Hv, monkeypatch):
    """The chunk form for the other gate forms: pre-activations in bf16
    (activated as read, gradients through the activations), coupled beta
    (d(beta) summed over the erase side's channels and the write side's
    columns) and scalar alpha (d(alpha) summed over the channels); ragged
    chunks, grouped heads, S0 and dS_T: against the oracle of the form."""
    from tests.gate_forms import backward_alone, form_inputs, oracle_backward
    from tests.parity import TOL, normwise, to_np
    monkeypatch.setenv("GDN2_BACKWARD_CHUNKED", "2")
    rng = np.random.default_rng(5800 + len(form) + T + Hqk)
    x = form_inputs(rng, form, T, Hv, 128, 128, "bf16", DEV, B=B, Hqk=Hqk)
    S0 = torch.from_numpy((rng.standard_normal((B, Hv, 128, 128)) * 0.5).astype(np.float32)).to(DEV)
    dO = torch.from_numpy(rng.standard_normal((B, T, Hv, 128)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    dST = torch.from_numpy(rng.standard_normal((B, Hv, 128, 128)).astype(np.float32)).to(DEV)
    got = backward_alone(form, x, S0, dO, dST)
    torch.cuda.synchronize()
    ref = oracle_backward(form, x, S0, dO, dST)
    names = [nm for nm in ("dq", "dk", "dv", "da", "db", "dw", "dS0") if got.get(nm) is not None]
    errs = {nm: normwise(to_np(got[nm]), ref[nm]) for nm in names}
    errs.update({nm + " per head": per_head_error(to_np(got[nm]), ref[nm], (0, 1) if nm == "dS0" else (0, 2))
                 for nm in names})
    print(f"[chunk form {form} B{B} T{T} Hqk{Hqk} Hv{Hv}] " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()),
          flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
    assert not bad, bad


@pytest.mark.parametrize("form,B,T,Hqk,split", [("channel", 1, 8192, 1, None), ("channel", 1, 8192, 1, "1"),
                                                ("channel", 2, 2048, 1, None), ("coupled", 2, 2048, 1, None),
                                                ("preact", 1, 2048, 2, None), ("scalar", 1, 2048, 2, None)])
def test_chunk_states_from_segments(form, B, T, Hqk, split, monkeypatch):
    """Few long sequences (B1-2, two value heads): the prefill's split plan
    cuts them into segments of 512 tokens (16 at T8192, 4 at T2048), so the
    chunk-boundary states come from all segments at once, each run from its
    entering state (GDN2_PREFILL_SPLIT=1: one launch over whole sequences
    instead); S0 and dS_T present, against the oracle of the form. At T8192
    the workspace shows the plan: the segments' transitions, exiting and
    entering states (3 x 16 x 2 fp32 states) on top of the whole-sequence
    form's."""
    from tests.gate_forms import backward_alone, form_inputs, oracle_backward
    from tests.parity import TOL, normwise, to_np
    Hv = 2
    if T == 8192:
        desc = g.make_desc(B, T, Hqk, Hv, 128, 128, 64, g.GDN2_BF16)
        monkeypatch.setenv("GDN2_PREFILL_SPLIT", "1")
        whole = g.gdn2_chunk_backward_workspace_bytes(desc)
        monkeypatch.delenv("GDN2_PREFILL_SPLIT")
        seg = g.gdn2_chunk_backward_workspace_bytes(desc)
        assert seg - whole == 3 * 16 * B * Hv * 128 * 128 * 4
    if split is not None:
        monkeypatch.setenv("GDN2_PREFILL_SPLIT", split)
    monkeypatch.setenv("GDN2_BACKWARD_CHUNKED", "2")
    rng = np.random.default_rng(5900 + len(form) + B + 3 * Hqk + T)
    x = form_inputs(rng, form, T, Hv, 128, 128, "bf16", DEV, B=B, Hqk=Hqk)
    S0 = torch.from_numpy((rng.standard_normal((B, Hv, 128, 128)) * 0.5).astype(np.float32)).to(DEV)
    dO = torch.from_numpy(rng.standard_normal((B, T, Hv, 128)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    dST = torch.from_numpy(rng.standard_normal((B, Hv, 128, 128)).astype(np.float32)).to(DEV)
    got = backward_alone(form, x, S0, dO, dST)
    torch.cuda.synchronize()
    ref = oracle_backward(form, x, S0, dO, dST)
    names = [nm for nm in ("dq", "dk", "dv", "da", "db", "dw", "dS0") if got.get(nm) is not None]
    errs = {nm: normwise(to_np(got[nm]), ref[nm]) for nm in names}
    errs.update({nm + " per head": per_head_error(to_np(got[nm]), ref[nm], (0, 1) if nm == "dS0" else (0, 2))
                 for nm in names})
    print(f"[chunk states from segments {form} B{B} T{T} Hqk{Hqk} split {split}] "
          + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
    assert not bad, bad
