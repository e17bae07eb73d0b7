"""Parity of the HIP decode step (gdn2_decode_step) with the fp64 oracle."""
import numpy as np
import pytest
import torch

import gated_delta_rule_83_amd as g
import oracle
from gated_delta_rule_83_amd import inputs as gi
from tests.parity import TOL, normwise, rand_inputs, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def decode_run(td, steps):
    """Step the GPU decode over the T axis of a prefill-shaped input dict."""
    S = td["S0"].clone()
    outs = []
    for t in range(steps):
        sl = lambda x: x[:, t:t + 1].contiguous()
        outs.append(g.decode_step(sl(td["q"]), sl(td["k"]), sl(td["v"]), sl(td["a"]), sl(td["b"]),
                                  sl(td["w"]), S))
    return torch.cat(outs, dim=1), S


@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 32), (32, 16), (64, 64), (128, 128), (128, 64),
                                   (16, 128), (128, 16)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_shapes(dk, dv, dtype):
    rng = np.random.default_rng(dk * 1000 + dv)
    steps = 6
    d = rand_inputs(rng, 3, steps, 2, 4, dk, dv)
    td = gi.to_torch(d, dtype, DEV)
    o, S = decode_run(td, steps)
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.forward(td["q"], td["k"], td["v"], td["a"], td["b"], td["w"], td["S0"])
    eo, es = normwise(to_np(o), ref_o), normwise(to_np(S), ref_S)
    print(f"[decode dk{dk} dv{dv} {dtype}] o err {eo:.3e}  S err {es:.3e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_config0_as_decode_steps():
    """Workload c0's tokens fed one at a time through the decode step (fp32, 1e-4)."""
    c = gi.config(0)
    d = gi.make_inputs(c)
    d["S0"] = np.zeros((c.B, c.H_v, c.d_k, c.d_v), np.float32)
    td = gi.to_torch(d, "f32", DEV)
    o, S = decode_run(td, c.T)
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.forward(td["q"], td["k"], td["v"], td["a"], td["b"], td["w"], None)
    assert normwise(to_np(o), ref_o) <= 1e-4 and normwise(to_np(S), ref_S) <= 1e-4


def _decode_workload(c, steps, heads):
    """Run `steps` decode steps of workload c on the GPU; oracle on sampled (n, h)."""
    S0 = gi.make_decode_state(c)
    S = torch.from_numpy(S0).to(DEV)
    rec = {k: [] for k in ("q", "k", "v", "a", "b", "w")}
    outs = []
    ns = [n for n, _ in heads]
    for step in range(steps):
        d = gi.make_decode_step(c, step)
        for k_ in rec:
            rec[k_].append(d[k_][ns])
        td = gi.to_torch(d, c.dtype, DEV)
        o = g.decode_step(td["q"], td["k"], td["v"], td["a"], td["b"], td["w"], S)
        outs.append(o[ns].cpu())
    torch.cuda.synchronize()
    # sampled sequences as a prefill over the step axis
    sub = {k_: np.concatenate(v_, axis=1) for k_, v_ in rec.items()}
    sub_t = gi.to_torch(sub, c.dtype)
    sub_t["S0"] = torch.from_numpy(S0[ns])
    sel = [(i, h) for i, (_, h) in enumerate(heads)]
    ref_o, ref_S = oracle.forward_heads(sub_t, sel)
    o_all = torch.cat(outs, dim=1)  # [len(heads), steps, H, d_v]
    worst = 0.0
    for i, (n, h) in enumerate(heads):
        eo = normwise(to_np(o_all[i, :, h]), ref_o[(i, h)])
        es = normwise(to_np(S[n, h]), ref_S[(i, h)])
        print(f"[decode {c.name} steps={steps}] (n={n}, h={h}) o err {eo:.3e}  S err {es:.3e}", flush=True)
        worst = max(worst, eo, es)
    assert worst <= TOL[c.dtype], worst


def test_decode_workload_scaled():
    c = gi.scaled(4, B=16)
    _decode_workload(c, 64, [(0, 0), (5, 9), (15, 15)])


def test_decode_workload_full_1024_steps():
    """Workload c4 as stated: 256 sequences x 16 heads, 1024 steps; sampled heads."""
    c = gi.config(4)
    _decode_workload(c, c.decode_steps, [(0, 0), (100, 7), (255, 15)])


@pytest.mark.parametrize("form,dtype,dk,dv", [("preact", "bf16", 128, 128), ("preact", "f32", 64, 32),
                                              ("coupled", "bf16", 128, 128), ("coupled", "f32", 32, 64),
                                              ("scalar", "bf16", 128, 128), ("scalar", "f32", 16, 128)])
def test_decode_gate_forms(form, dtype, dk, dv):
    """gdn2_decode_step_gates: T successive decode steps of each gate form from
    a random state equal the oracle's recurrence of that form over T tokens
    (every output and the final state); the coupled and scalar forms equal,
    bit for bit, the per-channel decode fed the broadcast gates."""
    from tests.gate_forms import form_inputs, oracle_forward
    rng = np.random.default_rng(230 + dk + dv + len(form))
    N, T, Hv = 3, 6, 4
    x = form_inputs(rng, form, T, Hv, dk, dv, dtype, DEV, B=N, Hqk=2)
    S0 = torch.from_numpy((rng.standard_normal((N, Hv, dk, dv)) * 0.5).astype(np.float32)).to(DEV)
    S, S_ch = S0.clone(), S0.clone()
    outs = []
    for t in range(T):
        st = {nm: None if v is None else v[:, t:t + 1].contiguous() for nm, v in x.items()}
        outs.append(g.decode_step(st["q"], st["k"], st["v"], st["a"], st["b"], st["w"], S, gates=form))
        if form in ("coupled", "scalar"):
            a = st["a"][..., None].expand(N, 1, Hv, dk).contiguous() if form == "scalar" else st["a"]
            bb = st["b"][..., None]
            o_ch = g.decode_step(st["q"], st["k"], st["v"], a, bb.expand(N, 1, Hv, dk).contiguous(),
                                 bb.expand(N, 1, Hv, dv).contiguous(), S_ch)
            torch.cuda.synchronize()
            assert torch.equal(outs[-1], o_ch) and torch.equal(S, S_ch), t
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=1)
    ref_o, ref_S = oracle_forward(form, x, S0)
    eo, es = normwise(to_np(o), ref_o), normwise(to_np(S), ref_S)
    print(f"[decode {form} {dtype} dk{dk} dv{dv}] o err {eo:.3e} S err {es:.3e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]
