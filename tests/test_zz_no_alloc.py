"""gdn2_chunk_forward_noalloc: the prefill whose split-sequence scratch is a
static device array of the library (for callers that cannot allocate).

Called through the C ABI and compared with gdn2_chunk_forward (caller
workspace) on the same inputs: the two run the same kernels and plan, so
outputs and final states must agree bit for bit; both are also held to the
oracle's tolerance. Two calls in a row, the second with a smaller problem
(fewer segments, so the static array keeps part of the first call's
contents), an unsplit problem that needs no scratch at all, and the
long-context shape, whose output-correction split needs more scratch than
the static array holds: there the entry point runs the segments a second
time instead (within the scratch), so it is held to the oracle's tolerance
rather than to bitwise equality.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_83_amd as g
import oracle
from gated_delta_rule_83_amd import inputs as gi
from tests.parity import TOL, normwise, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(B, T, Hqk, Hv, seed):
    c = gi.scaled(2, B=B, T=T, H_qk=Hqk, H_v=Hv, seed=seed)
    return gi.to_torch(gi.make_inputs(c), "bf16", DEV)


def _both(x, B, T, Hqk, Hv, d=128, check_oracle=True):
    desc = g.make_desc(B, T, Hqk, Hv, d, d, 64, g.GDN2_BF16)
    st, crun, nseg = g.gdn2_chunk_forward_plan(desc)
    assert st == g.GDN2_OK
    ws = g.gdn2_chunk_forward_workspace_bytes(desc)
    print(f"[noalloc] B{B} T{T} H_qk{Hqk} H_v{Hv}: chunk {crun}, {nseg} segments, scratch {ws} bytes", flush=True)
    assert ws <= g.GDN2_NOALLOC_SCRATCH_BYTES
    stream = torch.cuda.current_stream().cuda_stream
    ptrs = [x[n].data_ptr() for n in ("q", "k", "v", "a", "b", "w")]
    o1 = torch.full((B, T, Hv, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    s1 = torch.full((B, Hv, d, d), float("nan"), dtype=torch.float32, device=DEV)
    assert g.gdn2_chunk_forward_noalloc(desc, *ptrs, None, o1.data_ptr(), s1.data_ptr(), stream) == g.GDN2_OK
    o2 = torch.empty_like(o1)
    s2 = torch.empty_like(s1)
    work = torch.empty(max(ws, 1), dtype=torch.uint8, device=DEV)
    assert g.gdn2_chunk_forward(desc, *ptrs, None, o2.data_ptr(), s2.data_ptr(), work.data_ptr(), ws,
                                stream) == g.GDN2_OK
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2), "noalloc differs from the workspace entry point"
    if check_oracle:
        ref_o, ref_S = oracle.forward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], None)
        eo, es = normwise(to_np(o1), ref_o), normwise(to_np(s1), ref_S)
        print(f"[noalloc] o err {eo:.3e}  S_T err {es:.3e}", flush=True)
        assert eo <= TOL["bf16"] and es <= TOL["bf16"], (eo, es)
    return nseg, ws


def test_noalloc_matches_workspace_entry_twice_then_smaller():
    # first: 4 heads of one long sequence, split into many segments
    n1, w1 = _both(_inputs(1, 8192, 2, 4, 11), 1, 8192, 2, 4)
    # second, in the same process: a smaller problem (fewer segments)
    n2, w2 = _both(_inputs(1, 2048 + 37, 1, 2, 12), 1, 2048 + 37, 1, 2)
    assert n1 > 1 and n2 > 1 and w2 < w1


def test_noalloc_unsplit_needs_no_scratch():
    nseg, ws = _both(_inputs(8, 256, 4, 8, 13), 8, 256, 4, 8)
    assert nseg == 1 and ws == 0


def test_noalloc_rejects_scratch_beyond_its_buffer(monkeypatch):
    """Forcing 64 segments of 32 value heads needs 268 MB of scratch: refused
    before anything is enqueued (no tensor is touched)."""
    monkeypatch.setenv("GDN2_PREFILL_SPLIT", "64")
    B, T, H = 1, 64 * 64, 32
    desc = g.make_desc(B, T, H, H, 128, 128, 64, g.GDN2_BF16)
    assert g.gdn2_chunk_forward_workspace_bytes(desc) > g.GDN2_NOALLOC_SCRATCH_BYTES
    dummy = torch.zeros(16, device=DEV).data_ptr()
    st = g.gdn2_chunk_forward_noalloc(desc, dummy, dummy, dummy, dummy, dummy, dummy, None, dummy, None, 0)
    assert st == g.GDN2_ERR_SCRATCH


def test_noalloc_long_context_runs_within_its_scratch():
    c = gi.config(2)
    desc = g.make_desc(c.B, c.T, c.H_qk, c.H_v, c.d_k, c.d_v, c.chunk, g.GDN2_BF16)
    assert g.gdn2_chunk_forward_workspace_bytes(desc) > g.GDN2_NOALLOC_SCRATCH_BYTES
    print(f"[noalloc] {c.name}: drawing inputs", flush=True)
    x = gi.to_torch(gi.make_inputs(c), "bf16", DEV)
    ptrs = [x[n].data_ptr() for n in ("q", "k", "v", "a", "b", "w")]
    o = torch.full((c.B, c.T, c.H_v, c.d_v), float("nan"), dtype=torch.bfloat16, device=DEV)
    S = torch.full((c.B, c.H_v, c.d_k, c.d_v), float("nan"), dtype=torch.float32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    print(f"[noalloc] {c.name}: launching", flush=True)
    assert g.gdn2_chunk_forward_noalloc(desc, *ptrs, None, o.data_ptr(), S.data_ptr(), stream) == g.GDN2_OK
    o2, S2 = g.chunk_forward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], None, chunk=c.chunk)
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.forward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], None)
    for lbl, oo, ss in (("noalloc", o, S), ("workspace", o2, S2)):
        eo, es = normwise(to_np(oo), ref_o), normwise(to_np(ss), ref_S)
        print(f"[noalloc] {c.name} {lbl}: o err {eo:.3e}  S_T err {es:.3e}", flush=True)
        assert eo <= TOL["bf16"] and es <= TOL["bf16"], (lbl, eo, es)
