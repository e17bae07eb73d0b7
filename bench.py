#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet-2 forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the whole hot path over one batch of synthetic
input: a prefill (gdn2_chunk_forward) over the 1.3B-class layer shape
(B=8, T=4096, H=16, d_k=d_v=128, chunk 64, bf16 q/k/v, fp32 gates and state)
followed by one decode step (gdn2_decode_step) over the batched-decode shape
(256 sequences x 16 heads, fp32 128x128 state). Inputs are resident in HBM
before the timed region. Per-kernel durations come from HIP events recorded
on the stream the kernels are launched on.

After the timed steps, the decode workload as stated (1024 successive decode
steps from a random state) runs once for the decode bandwidth figure, the
prefill with the gates as bf16 pre-activations (gdn2_chunk_forward_preact)
and the backward pass (gdn2_chunk_backward) of the prefill run a few times
for their own figures, and the fp64 oracle runs on the host over the prefill batch for
the CPU baseline.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP32_VECTOR_PEAK_TFS = 157.3     # MI355X fp32 vector ALUs, TFLOP/s
PREFILL_KERNEL_SOURCES = ["gated_delta_rule_83_amd/csrc/gdn2_prefill.hpp",
                          "gated_delta_rule_83_amd/csrc/gdn2_device.hpp",
                          "gated_delta_rule_83_amd/csrc/gdn2_prefill_inst.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_B8_T4096_H16_d128_bf16_hbm_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_algorithmic(c):
    """Bytes and flops the method itself must move / compute for one prefill call.

    Bytes: q, k (H_qk heads) and v, o in the input dtype; a, b, w in fp32; the
    final state S_T in fp32 (S0 is null). Flops per (token, value head):
    4*C*d_k (four Gram triangles) + 4*C*d_v (Akk U, T Z, Mqk U, Mqb R) +
    8*d_k*d_v (gamma*K S0, gamma*Q S0, two carry products) + C^2/3 (solve)
    + d_k*d_v/C (carry scaling)."""
    es = 2 if c.dtype == "bf16" else 4
    toks = c.B * c.T
    by = toks * (c.H_qk * c.d_k * es * 2 + c.H_v * c.d_v * es * 2 + c.H_v * c.d_k * 4 * 2
                 + c.H_v * c.d_v * 4) + c.B * c.H_v * c.d_k * c.d_v * 4
    C = c.chunk
    fl_th = 4 * C * c.d_k + 4 * C * c.d_v + 8 * c.d_k * c.d_v + C * C / 3 + c.d_k * c.d_v / C
    return by, fl_th * toks * c.H_v


def decode_algorithmic(c):
    """Bytes per decode step: state read + write, q, k, v, o, a, b, w."""
    es = 2 if c.dtype == "bf16" else 4
    per_head = c.d_k * c.d_v * 4 * 2 + c.d_v * es * 2 + c.d_k * 4 * 2 + c.d_v * 4
    qk = c.B * c.H_qk * c.d_k * es * 2
    return c.B * c.H_v * per_head + qk


def preact_algorithmic(c):
    """Bytes of one prefill launch with the gates as pre-activations in the
    input dtype (a, b, w at es bytes instead of 4)."""
    es = 2 if c.dtype == "bf16" else 4
    toks = c.B * c.T
    return (toks * (c.H_qk * c.d_k * es * 2 + c.H_v * c.d_v * es * 2 + c.H_v * c.d_k * es * 2
                    + c.H_v * c.d_v * es) + c.B * c.H_v * c.d_k * c.d_v * 4)


def backward_algorithmic(c):
    """Flops of the gradient by the recurrence, per state element and token:
    the forward states (decay 1, k-read 2, erase 2, write 2) and the adjoint
    (query read 2+2, du 2, dr 2, erase-gate sum 2, write-gate sum 2, read
    adjoint 2+3, decay sum 2, decay 1): 27 * d_k * d_v per token and value
    head. Bytes: inputs, dO and every gradient once."""
    es = 2 if c.dtype == "bf16" else 4
    toks = c.B * c.T
    fl = 27.0 * c.d_k * c.d_v * toks * c.H_v
    by = toks * (c.H_qk * c.d_k * es * 4 + c.H_v * c.d_v * es * 3 + c.H_v * c.d_k * 4 * 4
                 + c.H_v * c.d_v * 4 * 2) + 2 * c.B * c.H_v * c.d_k * c.d_v * 4
    return fl, by


def source_digest(paths):
    """sha256 of the kernel sources without comments and blank lines, so that
    an edit of a comment does not invalidate counters taken on the code."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()[:16]


def read_traffic(digest):
    """HBM bytes per prefill launch from the committed rocprofv3 counter runs,
    if they were taken on the current kernel source; else None."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_digest") != digest:
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="length of the decode workload leg (default: the workload's 1024)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--preact-steps", type=int, default=50,
                    help="timed launches of the prefill with gate pre-activations (0: skip)")
    ap.add_argument("--backward-steps", type=int, default=5,
                    help="timed launches of the backward pass over the prefill shape (0: skip)")
    ap.add_argument("--long-backward", type=int, default=0,
                    help="also time this many launches of the backward of the long-context shape "
                         "(B1 T65536 H16 d128 bf16, split into segments), reported under backward_long "
                         "(default 0: off)")
    ap.add_argument("--chunk", type=int, default=None, help="override the prefill chunk length")
    ap.add_argument("--counters", action="store_true",
                    help="for hardware-counter runs: launch the prefill and the decode kernel twice each "
                         "and a plain 256 MiB device copy twice (counter calibration), then exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_rule_83_amd as g
    from gated_delta_rule_83_amd import inputs as gi

    g.load()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    cp = gi.config(1)
    if args.chunk:
        cp = cp.replace(chunk=args.chunk)
    cd = gi.config(4)
    dec_steps = args.decode_steps or cd.decode_steps

    log(f"[bench] drawing prefill inputs {cp.name}")
    t0 = time.time()
    dp = gi.make_inputs(cp)
    tp = gi.to_torch(dp, cp.dtype, dev)
    o = torch.empty((cp.B, cp.T, cp.H_v, cp.d_v), dtype=tp["q"].dtype, device=dev)
    S_T = torch.empty((cp.B, cp.H_v, cp.d_k, cp.d_v), dtype=torch.float32, device=dev)
    log(f"[bench] drawing {dec_steps} decode steps {cd.name} ({time.time() - t0:.1f}s so far)")
    S_dec0 = torch.from_numpy(gi.make_decode_state(cd)).to(dev)
    dsteps = [gi.to_torch(gi.make_decode_step(cd, s), cd.dtype, dev) for s in range(dec_steps)]
    o_dec = torch.empty((cd.B, 1, cd.H_v, cd.d_v), dtype=dsteps[0]["q"].dtype, device=dev)
    S_dec = S_dec0.clone()
    torch.cuda.synchronize()
    log(f"[bench] inputs resident ({time.time() - t0:.1f}s)")

    def prefill():
        g.chunk_forward(tp["q"], tp["k"], tp["v"], tp["a"], tp["b"], tp["w"], None, chunk=cp.chunk,
                        o=o, S_T=S_T, stream=stream)

    def decode(i):
        x = dsteps[i % dec_steps]
        g.decode_step(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], S_dec, o=o_dec, stream=stream)

    if args.counters:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for i in range(2):
            prefill()
            decode(i)
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] counter launches done: 2 x prefill, 2 x decode, 2 x copy of 256 MiB")
        return

    for i in range(args.warmup):
        prefill()
        decode(i)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed steps
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(K):
        e = ev[i]
        e[0].record(stream)
        prefill()
        e[1].record(stream)
        e[2].record(stream)
        decode(i)
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    pre_ms = [e[0].elapsed_time(e[1]) for e in ev]
    dec_ms = [e[2].elapsed_time(e[3]) for e in ev]
    pre_avg = float(np.mean(pre_ms)) / 1e3
    log(f"[bench] {K} steps: prefill avg {pre_avg * 1e6:.1f} us (min {min(pre_ms) * 1e3:.1f}), "
        f"decode avg {np.mean(dec_ms) * 1e3:.1f} us; wall {wall * 1e3:.1f} ms")

    tokens = cp.B * cp.T
    pbytes, pflops = prefill_algorithmic(cp)
    value = tokens / pre_avg
    digest = source_digest(PREFILL_KERNEL_SOURCES)
    traffic = read_traffic(digest)

    # ---------------------------------------------------------------- decode workload leg
    S_dec.copy_(S_dec0)
    torch.cuda.synchronize()
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(dec_steps)]
    l0, l1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    l0.record(stream)
    for s in range(dec_steps):
        dev_ev[s][0].record(stream)
        decode(s)
        dev_ev[s][1].record(stream)
    l1.record(stream)
    torch.cuda.synchronize()
    dk_ms = [a.elapsed_time(b) for a, b in dev_ev]
    loop_ms = l0.elapsed_time(l1)
    dbytes = decode_algorithmic(cd)
    d_avg = float(np.mean(dk_ms)) / 1e3
    d_gbs = dbytes / d_avg / 1e9
    log(f"[bench] decode workload: {dec_steps} steps in {loop_ms:.1f} ms; kernel avg {d_avg * 1e6:.1f} us "
        f"= {d_gbs:.0f} GB/s algorithmic")

    # ---------------------------------------------------------------- gate pre-activation leg
    pre_leg = None
    if args.preact_steps > 0:
        tpp = gi.to_torch_preact(gi.make_preact_inputs(cp), cp.dtype, dev)

        def prefill_preact():
            g.chunk_forward_preact(tpp["q"], tpp["k"], tpp["v"], tpp["a"], tpp["b"], tpp["w"], None, chunk=cp.chunk,
                                   o=o, S_T=S_T, stream=stream)

        for _ in range(100):
            prefill_preact()
        torch.cuda.synchronize()
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.preact_steps)]
        for e0, e1 in pev:
            e0.record(stream)
            prefill_preact()
            e1.record(stream)
        torch.cuda.synchronize()
        p_ms = [a.elapsed_time(b) for a, b in pev]
        p_avg = float(np.mean(p_ms)) / 1e3
        pby = preact_algorithmic(cp)
        pre_leg = {"launches": args.preact_steps, "kernel_us": p_avg * 1e6, "min_us": min(p_ms) * 1e3,
                   "tokens_per_s": tokens / p_avg, "achieved": pby / p_avg / 1e9, "peak": HBM_PEAK_GBS,
                   "unit": "GB/s", "frac": pby / p_avg / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": pby}
        log(f"[bench] prefill with gate pre-activations: {p_avg * 1e6:.1f} us per launch")
        del tpp

    # ---------------------------------------------------------------- backward leg
    bwd = None
    if args.backward_steps > 0:
        gen = torch.Generator(device=dev).manual_seed(5)
        dO = torch.randn(o.shape, generator=gen, device=dev, dtype=torch.float32).to(o.dtype)
        dST = torch.randn(S_T.shape, generator=gen, device=dev, dtype=torch.float32)
        desc = g.make_desc(cp.B, cp.T, cp.H_qk, cp.H_v, cp.d_k, cp.d_v, cp.chunk,
                           g.GDN2_BF16 if cp.dtype == "bf16" else g.GDN2_F32)
        bws = torch.empty(g.gdn2_chunk_backward_workspace_bytes(desc), dtype=torch.uint8, device=dev)

        def backward(grads=None):
            return g.chunk_backward(tp["q"], tp["k"], tp["v"], tp["a"], tp["b"], tp["w"], None, dO, dST,
                                    grads=grads, workspace=bws, stream=stream)

        grads = backward()
        backward(grads)
        torch.cuda.synchronize()
        bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.backward_steps)]
        for e0, e1 in bev:
            e0.record(stream)
            backward(grads)
            e1.record(stream)
        torch.cuda.synchronize()
        b_ms = [a.elapsed_time(b) for a, b in bev]
        b_avg = float(np.mean(b_ms)) / 1e3
        bfl, bby = backward_algorithmic(cp)
        bwd = {"launches": args.backward_steps, "ms": b_avg * 1e3, "min_ms": min(b_ms),
               "tokens_per_s": tokens / b_avg, "bound": "alu",
               "achieved": bfl / b_avg / 1e12, "peak": FP32_VECTOR_PEAK_TFS, "unit": "TFLOP/s",
               "frac": bfl / b_avg / 1e12 / FP32_VECTOR_PEAK_TFS, "algorithmic_flops": bfl,
               "algorithmic_bytes": bby, "workspace_bytes": bws.numel()}
        log(f"[bench] backward: {b_avg * 1e3:.2f} ms per launch (min {min(b_ms):.2f}), "
            f"{bfl / b_avg / 1e12:.1f} TFLOP/s algorithmic")
        del grads, bws

    # ---------------------------------------------------------------- long-context backward (optional)
    bwd_long = None
    if args.long_backward > 0:
        cl = gi.config(2)
        tl = gi.to_torch(gi.make_inputs(cl), "bf16", dev)
        gen = torch.Generator(device=dev).manual_seed(6)
        dOl = torch.randn(tl["v"].shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        dSTl = torch.randn((cl.B, cl.H_v, cl.d_k, cl.d_v), generator=gen, device=dev, dtype=torch.float32)
        descl = g.make_desc(cl.B, cl.T, cl.H_qk, cl.H_v, cl.d_k, cl.d_v, cl.chunk, g.GDN2_BF16)
        wsl = torch.empty(g.gdn2_chunk_backward_workspace_bytes(descl), dtype=torch.uint8, device=dev)

        def backward_long(grads=None):
            return g.chunk_backward(tl["q"], tl["k"], tl["v"], tl["a"], tl["b"], tl["w"], None, dOl, dSTl,
                                    grads=grads, workspace=wsl, stream=stream)

        gl = backward_long()
        torch.cuda.synchronize()
        lev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.long_backward)]
        for e0, e1 in lev:
            e0.record(stream)
            backward_long(gl)
            e1.record(stream)
        torch.cuda.synchronize()
        l_ms = [a.elapsed_time(b) for a, b in lev]
        l_avg = float(np.mean(l_ms)) / 1e3
        lfl, _ = backward_algorithmic(cl)
        bwd_long = {"workload": "backward B1 T65536 H16 d128 bf16 (split into segments)",
                    "launches": args.long_backward, "ms": l_avg * 1e3, "min_ms": min(l_ms),
                    "tokens_per_s": cl.B * cl.T / l_avg, "achieved": lfl / l_avg / 1e12,
                    "peak": FP32_VECTOR_PEAK_TFS, "unit": "TFLOP/s", "workspace_bytes": wsl.numel()}
        log(f"[bench] long-context backward: {l_avg * 1e3:.2f} ms per launch (min {min(l_ms):.2f})")
        del gl, wsl, tl

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nthreads = min(16, oracle.cores())
        log(f"[bench] oracle on the host, {nthreads} threads, full prefill batch")
        _, _, el = oracle.forward(dp["q"] if cp.dtype == "f32" else tp["q"].cpu(),
                                  dp["k"] if cp.dtype == "f32" else tp["k"].cpu(),
                                  dp["v"] if cp.dtype == "f32" else tp["v"].cpu(),
                                  dp["a"], dp["b"], dp["w"], None, nthreads=nthreads, timing=True)
        cpu = {"value": tokens / el, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
               "sample": f"the whole prefill batch once (B={cp.B}, T={cp.T}, {cp.H_v} heads, "
                         f"d={cp.d_k}), fp64 recurrence, {el:.1f} s"}
        log(f"[bench] oracle {el:.1f} s -> {tokens / el:.0f} tokens/s")

    out = {
        "metric": "prefill tokens/s (T=4096,H=16,d=128) + decode HBM GB/s, % of roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cp.dtype,
        "data": "synthetic",
        "config": {
            "workload": (f"prefill B{cp.B} T{cp.T} H_qk{cp.H_qk} H_v{cp.H_v} d_k{cp.d_k} d_v{cp.d_v} "
                         f"chunk{cp.chunk} {cp.dtype} + decode step N{cd.B} H{cd.H_v} d{cd.d_k} fp32 state"),
            "prefill_kernel_us": pre_avg * 1e6,
            "prefill_kernel_us_median": float(np.median(pre_ms)) * 1e3,
            "prefill_kernel_us_min": float(min(pre_ms)) * 1e3,
            "decode_kernel_us": float(np.mean(dec_ms)) * 1e3,
        },
        "roofline": {
            "kernel": "prefill",
            "bound": "hbm",
            "achieved": pbytes / pre_avg / 1e9,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": pbytes / pre_avg / 1e9 / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes": pbytes,
            "mfma_frac_algorithmic": pflops / pre_avg / 1e12 / MFMA_BF16_PEAK_TFS,
            "kernel_source_digest": digest,
        },
        "decode": {
            "steps": dec_steps,
            "kernel_us": d_avg * 1e6,
            "loop_us_per_step": loop_ms * 1e3 / dec_steps,
            "achieved": d_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": d_gbs / HBM_PEAK_GBS,
            "algorithmic_bytes": dbytes,
        },
        "preact": pre_leg,
        "backward": bwd,
        **({"backward_long": bwd_long} if bwd_long else {}),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
