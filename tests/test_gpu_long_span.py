"""Parity at buffer spans beyond 4 GiB per tensor: prefill sequences, and a
decode step over a state larger than 2^32 bytes.

A sequence whose rows of one tensor span 4 GiB or more (e.g. bf16 values of
32 value heads at T >= 524,288, or bf16 gate pre-activations of 64 value
heads at T >= 262,144: the context lengths of the aiki wiki's "why it
matters" section) must be computed like any other. The prefill's buffer
descriptors cover one chunk of rows each, so no 32-bit range can wrap; these
tests run such spans unsplit (two sequences; and a packed batch, which is
never split) with the outputs pre-filled with NaN, so that a dropped store or
a request that read zeros shows up, and check sampled heads against the
oracle over the whole sequence.
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


def _oracle_heads(x, heads, G, gates, start=0, length=None):
    """Oracle (o, S_T) of sampled (n, h) pairs, as one batch of single heads."""
    sl = lambda t, n, h: t[n:n + 1, start:start + length if length else None, h:h + 1]
    q = torch.cat([sl(x["q"], n, h // G) for n, h in heads]).cpu()
    k = torch.cat([sl(x["k"], n, h // G) for n, h in heads]).cpu()
    v = torch.cat([sl(x["v"], n, h) for n, h in heads]).cpu()
    a = torch.cat([sl(x["a"], n, h) for n, h in heads]).cpu()
    b = torch.cat([sl(x["b"], n, h) for n, h in heads]).cpu()
    if gates == "preact":
        w = torch.cat([sl(x["w"], n, h) for n, h in heads]).cpu()
        return oracle.forward_preact(q, k, v, a, b, w, None)
    A, Bg, W = oracle.expand_scalar_gates(a, b, q.shape[-1], v.shape[-1], gates == "scalar")
    return oracle.forward(q, k, v, A, Bg, W, None)


def test_scalar_gates_values_span_over_4gib():
    """Scalar gates (Gated DeltaNet form) at B2 T524,328 H_qk16 H_v32 d128
    bf16: each sequence's values and outputs span 4 GiB + 40 tokens, so
    32-bit rest-of-sequence ranges would wrap at the second chunk."""
    B, T, Hqk, Hv, d = 2, 524_328, 16, 32, 128
    print(f"[long span] scalar gates B{B} T{T} H_qk{Hqk} H_v{Hv} d{d} bf16: drawing on the GPU", flush=True)
    x = gi.draw_on_device(B, T, Hqk, Hv, d, d, "bf16", "scalar", DEV, seed=524)
    o = torch.full((B, T, Hv, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    S_T = torch.full((B, Hv, d, d), float("nan"), dtype=torch.float32, device=DEV)
    st, c, nseg = g.gdn2_chunk_forward_plan(g.make_desc(B, T, Hqk, Hv, d, d, 64, g.GDN2_BF16))
    assert st == g.GDN2_OK and nseg == 1, "this shape must run unsplit"
    print(f"[long span] launching prefill (chunk {c}, unsplit)", flush=True)
    g.chunk_forward_scalar(x["q"], x["k"], x["v"], x["a"], x["b"], None, chunk=64, o=o, S_T=S_T)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()), "outputs left unwritten (NaN)"
    assert bool(torch.isfinite(S_T).all())
    heads = [(0, 5), (1, 30)]
    print(f"[long span] oracle on heads {heads}", flush=True)
    ref_o, ref_S = _oracle_heads(x, heads, Hv // Hqk, "scalar")
    for i, (n, h) in enumerate(heads):
        eo = normwise(to_np(o[n, :, h]), ref_o[i, :, 0])
        es = normwise(to_np(S_T[n, h]), ref_S[i, 0])
        # the first chunks, where a wrapped range would have zeroed the reads
        e0 = normwise(to_np(o[n, :256, h]), ref_o[i, :256, 0])
        print(f"[long span] scalar (n={n}, h={h}) o err {eo:.3e} (first 256 tokens {e0:.3e}) "
              f"S_T err {es:.3e}", flush=True)
        assert eo <= TOL["bf16"] and es <= TOL["bf16"] and e0 <= TOL["bf16"], (n, h, eo, es, e0)


def test_packed_preact_gates_span_over_4gib():
    """A packed batch (never split) of a 100-token and a 262,200-token
    sequence with bf16 gate pre-activations at H_qk16 H_v64 d128: the long
    sequence's gate rows span 4 GiB + 56 tokens."""
    lens = [100, 262_200]
    T, Hqk, Hv, d = sum(lens), 16, 64, 128
    print(f"[long span] packed preact lens {lens} H_qk{Hqk} H_v{Hv} d{d} bf16: drawing on the GPU", flush=True)
    x = gi.draw_on_device(1, T, Hqk, Hv, d, d, "bf16", "preact", DEV, seed=262, a_mu=-4.0)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device=DEV)
    sq = lambda t: t[0]
    o = torch.full((T, Hv, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    S_T = torch.full((len(lens), Hv, d, d), float("nan"), dtype=torch.float32, device=DEV)
    print("[long span] launching packed prefill", flush=True)
    g.chunk_forward_varlen(sq(x["q"]), sq(x["k"]), sq(x["v"]), sq(x["a"]), sq(x["b"]), sq(x["w"]), cu, None,
                           chunk=64, o=o, S_T=S_T, gates="preact")
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()), "outputs left unwritten (NaN)"
    assert bool(torch.isfinite(S_T).all())
    heads = [(0, 3), (0, 62)]
    print(f"[long span] oracle on heads {heads} of the long sequence", flush=True)
    ref_o, ref_S = _oracle_heads(x, heads, Hv // Hqk, "preact", start=lens[0], length=lens[1])
    for i, (_, h) in enumerate(heads):
        eo = normwise(to_np(o[lens[0]:, h]), ref_o[i, :, 0])
        es = normwise(to_np(S_T[1, h]), ref_S[i, 0])
        e0 = normwise(to_np(o[lens[0]:lens[0] + 256, h]), ref_o[i, :256, 0])
        print(f"[long span] preact h={h} o err {eo:.3e} (first 256 tokens {e0:.3e}) S_T err {es:.3e}",
              flush=True)
        assert eo <= TOL["bf16"] and es <= TOL["bf16"] and e0 <= TOL["bf16"], (h, eo, es, e0)


def test_decode_state_over_4gib():
    """One decode step of N4200 H16 d128 (bf16 q/k/v, fp32 gates): the fp32
    state is 4200 * 16 * 64 KiB = 4.1 GiB, so the last 104 sequences' states
    lie past byte 2^32 of the allocation. Sampled sequences on both sides of
    that boundary against the oracle's single token from the same state."""
    N, H, d = 4200, 16, 128
    print(f"[long span] decode N{N} H{H} d{d} bf16: drawing on the GPU", flush=True)
    x = gi.draw_on_device(N, 1, H, H, d, d, "bf16", "channel", DEV, seed=4200)
    gen = torch.Generator(device=DEV).manual_seed(4201)
    S = torch.randn((N, H, d, d), generator=gen, device=DEV).mul_(0.5)
    pairs = [(0, 3), (2047, 11), (4095, 15), (4096, 0), (4150, 7), (4199, 15)]
    S0 = {p: S[p[0], p[1]].cpu() for p in pairs}
    o = torch.full((N, 1, H, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    print("[long span] launching the decode step (in place)", flush=True)
    g.decode_step(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], S, o=o)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()), "outputs left unwritten (NaN)"
    for n, h in pairs:
        sl = lambda t: t[n:n + 1, :, h:h + 1].cpu()
        ref_o, ref_S = oracle.forward(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["a"]), sl(x["b"]), sl(x["w"]),
                                      S0[(n, h)][None, None])
        eo = normwise(to_np(o[n, :, h]), ref_o[0, :, 0])
        es = normwise(to_np(S[n, h]), ref_S[0, 0])
        print(f"[long span] decode (n={n}, h={h}) o err {eo:.3e} S err {es:.3e}", flush=True)
        assert eo <= TOL["bf16"] and es <= TOL["bf16"], (n, h, eo, es)
