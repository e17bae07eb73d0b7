#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet-2 forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the whole hot path over one batch of synthetic
input: a prefill (gdn2_chunk_forward) over the 1.3B-class layer shape
(B=8, T=4096, H=16, d_k=d_v=128, bf16 q/k/v, fp32 gates and state; the
workload allows chunks of 64 tokens, the kernel runs the longest that fits,
reported as chunk_run) followed by one decode step (gdn2_decode_step) over
the batched-decode shape (256 sequences x 16 heads, fp32 128x128 state).
Inputs are resident in HBM before any timed region. Kernel durations come
from HIP events recorded on the stream the kernels are launched on.

Legs, in the order they run (each its own figure in the JSON line):
  series    a cold-start series of prefill launches of the layer shape: the
            first launches against the settled ones (the GPU's clocks ramp
            up under load; the JSON reports both);
  headline  W warm-up steps, then K timed steps (prefill + decode step):
            `value`, `roofline`, `ms_per_step`;
  configs   the other prefill workloads: long context (B1 T65536 H16) and
            grouped heads (B4 T16384 H_qk16 H_v32), each with its roofline;
  strong_decay  the layer shape with decay pre-activations N(+2, 1)
            (per-token decay ~0.12): the anchoring's range check at work;
  decode    the decode workload as stated (1024 successive steps from a
            random state), plus states of 1 GiB and 4 GiB (beyond the
            256 MiB Infinity Cache) for the bandwidth attribution;
  preact    the fused gate activation;
  backward  the backward pass of the layer shape in chunk form (HBM roofline
            on the inputs, dO and the gradients), with the per-token
            backward beside it;
  cpu_baseline   the fp64 oracle on the host cores over the layer batch, and
            on one (sequence, head) with one thread.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP32_VECTOR_PEAK_TFS = 157.3     # MI355X fp32 vector ALUs, TFLOP/s
# GDN2_BACKWARD_CHUNKED as the caller set it: the long-context backward leg
# runs that choice (the legs below set the variable for their own runs)
USER_BACKWARD_CHUNKED = os.environ.get("GDN2_BACKWARD_CHUNKED")
PREFILL_KERNEL_SOURCES = ["gated_delta_rule_83_amd/csrc/gdn2_prefill.hpp",
                          "gated_delta_rule_83_amd/csrc/gdn2_device.hpp",
                          "gated_delta_rule_83_amd/csrc/gdn2_range.hpp",
                          "gated_delta_rule_83_amd/csrc/gdn2_prefill_inst.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_B8_T4096_H16_d128_bf16_hbm_traffic.txt")
METRIC = "prefill tokens/s (T=4096,H=16,d=128) + decode HBM GB/s, % of roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_algorithmic(c, chunk_run, gate_bytes=4):
    """Bytes and flops the method itself must move / compute for one prefill call.

    Bytes: q, k (H_qk heads) and v, o in the input dtype; a, b, w at
    `gate_bytes` each (fp32 activated gates: 4); the final state S_T in fp32
    (S0 is null). Flops per (token, value head) at the chunk C that runs:
    4*C*d_k (four Gram triangles) + 4*C*d_v (Akk U, T Z, Mqk U, Mqb R) +
    8*d_k*d_v (gamma*K S0, gamma*Q S0, two carry products) + C^2/3 (solve)
    + d_k*d_v/C (carry scaling)."""
    es = 2 if c.dtype == "bf16" else 4
    toks = c.B * c.T
    by = toks * (c.H_qk * c.d_k * es * 2 + c.H_v * c.d_v * es * 2 + c.H_v * c.d_k * gate_bytes * 2
                 + c.H_v * c.d_v * gate_bytes) + c.B * c.H_v * c.d_k * c.d_v * 4
    C = chunk_run
    fl_th = 4 * C * c.d_k + 4 * C * c.d_v + 8 * c.d_k * c.d_v + C * C / 3 + c.d_k * c.d_v / C
    return by, fl_th * toks * c.H_v


def decode_algorithmic(N, H_qk, H_v, d_k, d_v, es=2):
    """Bytes per decode step: state read + write, q, k, v, o, a, b, w."""
    per_head = d_k * d_v * 4 * 2 + d_v * es * 2 + d_k * 4 * 2 + d_v * 4
    return N * H_v * per_head + N * H_qk * d_k * es * 2


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


def read_traffic(path, digest):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_digest") != digest:
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--series", type=int, default=300,
                    help="cold-start prefill launches timed one by one before the headline (0: skip)")
    ap.add_argument("--config-steps", type=int, default=20,
                    help="timed launches of each other prefill workload (0: skip those legs)")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="length of the decode workload leg (default: the workload's 1024)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--preact-steps", type=int, default=50,
                    help="timed launches of the prefill with gate pre-activations (0: skip)")
    ap.add_argument("--backward-steps", type=int, default=5,
                    help="timed launches of the backward pass over the prefill shape (0: skip)")
    ap.add_argument("--long-backward", type=int, default=0,
                    help="also time this many launches of the backward of the long-context shape "
                         "(B1 T65536 H16 d128 bf16, in chunk form where it applies), reported under backward_long "
                         "(default 0: off)")
    ap.add_argument("--chunk", type=int, default=None, help="override the prefill chunk length")
    ap.add_argument("--counters", type=int, default=None, metavar="CONFIG",
                    help="for hardware-counter runs: launch the prefill of workload CONFIG (1, 2 or 3) "
                         "twice, the decode step twice (with CONFIG 1) and a plain 256 MiB device copy twice "
                         "(counter calibration), then exit")
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

    def plan(c):
        st, crun, nseg = g.gdn2_chunk_forward_plan(
            g.make_desc(c.B, c.T, c.H_qk, c.H_v, c.d_k, c.d_v, c.chunk, g.GDN2_BF16 if c.dtype == "bf16" else g.GDN2_F32))
        if st != g.GDN2_OK:
            raise RuntimeError(f"plan failed for {c.name}: {g.gdn2_status_string(st)}")
        return crun, nseg

    def time_each(fn, n):
        """Per-launch milliseconds of n calls of fn, HIP events on `stream`."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

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
    n_dec_inputs = dec_steps if args.counters is None else 2
    log(f"[bench] drawing {n_dec_inputs} decode steps {cd.name} ({time.time() - t0:.1f}s so far)")
    S_dec0 = torch.from_numpy(gi.make_decode_state(cd)).to(dev)
    dsteps = [gi.to_torch(gi.make_decode_step(cd, s), cd.dtype, dev) for s in range(n_dec_inputs)]
    o_dec = torch.empty((cd.B, 1, cd.H_v, cd.d_v), dtype=dsteps[0]["q"].dtype, device=dev)
    S_dec = S_dec0.clone()
    torch.cuda.synchronize()
    log(f"[bench] inputs resident ({time.time() - t0:.1f}s)")
    chunk_run, nseg1 = plan(cp)

    def prefill():
        g.chunk_forward(tp["q"], tp["k"], tp["v"], tp["a"], tp["b"], tp["w"], None, chunk=cp.chunk,
                        o=o, S_T=S_T, stream=stream)

    def decode(i):
        x = dsteps[i % len(dsteps)]
        g.decode_step(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], S_dec, o=o_dec, stream=stream)

    if args.counters is not None:
        ci = args.counters
        if ci == 1:
            run = prefill
        else:
            cx = gi.config(ci)
            tx = gi.to_torch(gi.make_inputs(cx), cx.dtype, dev)
            ox = torch.empty((cx.B, cx.T, cx.H_v, cx.d_v), dtype=tx["q"].dtype, device=dev)
            sx = torch.empty((cx.B, cx.H_v, cx.d_k, cx.d_v), dtype=torch.float32, device=dev)

            def run():
                g.chunk_forward(tx["q"], tx["k"], tx["v"], tx["a"], tx["b"], tx["w"], None, chunk=cx.chunk,
                                o=ox, S_T=sx, stream=stream)
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for i in range(2):
            run()
            if ci == 1:
                decode(i)
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] counter launches done: 2 x prefill of workload {ci}"
            f"{', 2 x decode' if ci == 1 else ''}, 2 x copy of 256 MiB")
        return

    tokens = cp.B * cp.T
    pbytes, pflops = prefill_algorithmic(cp, chunk_run)

    # ---------------------------------------------------------------- cold-start series
    series = None
    if args.series > 0:
        log(f"[bench] cold-start series: {args.series} prefill launches of {cp.name}")
        ms = time_each(prefill, args.series)
        wins = [(0, 1), (1, 5), (5, 25), (25, 50), (50, 100), (100, 200), (200, 300), (300, 500)]
        series = {"launches": args.series, "windows_us": {}}
        for a, b in wins:
            if a < len(ms):
                seg = ms[a:min(b, len(ms))]
                series["windows_us"][f"{a}-{min(b, len(ms))}"] = round(float(np.mean(seg)) * 1e3, 1)
        tail = ms[len(ms) // 2:]
        series["first_launch_us"] = ms[0] * 1e3
        series["settled_avg_us"] = float(np.mean(tail)) * 1e3
        series["settled_min_us"] = float(min(tail)) * 1e3
        series["settled_frac"] = pbytes / (float(np.mean(tail)) / 1e3) / 1e9 / HBM_PEAK_GBS
        log(f"[bench] series windows (us): {series['windows_us']}")

    # ---------------------------------------------------------------- headline steps
    for i in range(args.warmup):
        prefill()
        decode(i)
    torch.cuda.synchronize()
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
    value = tokens / pre_avg
    digest = source_digest(PREFILL_KERNEL_SOURCES)
    traffic = read_traffic(TRAFFIC_FILE, digest)

    # ---------------------------------------------------------------- other prefill workloads
    configs = {}
    if args.config_steps > 0:
        for ci in (2, 3):
            cx = gi.config(ci)
            if args.chunk:
                cx = cx.replace(chunk=args.chunk)
            log(f"[bench] drawing {cx.name}")
            tx = gi.to_torch(gi.make_inputs(cx), cx.dtype, dev)
            ox = torch.empty((cx.B, cx.T, cx.H_v, cx.d_v), dtype=tx["q"].dtype, device=dev)
            sx = torch.empty((cx.B, cx.H_v, cx.d_k, cx.d_v), dtype=torch.float32, device=dev)
            crun, nseg = plan(cx)
            desc = g.make_desc(cx.B, cx.T, cx.H_qk, cx.H_v, cx.d_k, cx.d_v, cx.chunk, g.GDN2_BF16)
            ws = g.gdn2_chunk_forward_workspace_bytes(desc)
            wsx = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)

            def run_x():
                st = g.gdn2_chunk_forward(desc, tx["q"].data_ptr(), tx["k"].data_ptr(), tx["v"].data_ptr(),
                                          tx["a"].data_ptr(), tx["b"].data_ptr(), tx["w"].data_ptr(), None,
                                          ox.data_ptr(), sx.data_ptr(), wsx.data_ptr(), ws, stream.cuda_stream)
                if st != g.GDN2_OK:
                    raise g.Gdn2Error(st)

            # untimed calls for ~0.15 s first: the clock ramps up over the
            # first ~50 launches after the idle time of drawing the inputs
            t_one = time_each(run_x, 1)[0] / 1e3
            n_warm = max(3, int(0.15 / max(t_one, 1e-6)))
            for _ in range(n_warm):
                run_x()
            ms = time_each(run_x, args.config_steps)
            avg = float(np.mean(ms)) / 1e3
            by, fl = prefill_algorithmic(cx, crun)
            toks = cx.B * cx.T
            configs[cx.name] = {
                "workload": f"prefill B{cx.B} T{cx.T} H_qk{cx.H_qk} H_v{cx.H_v} d{cx.d_k} {cx.dtype}",
                "chunk_requested": cx.chunk, "chunk_run": crun, "segments": nseg, "launches": args.config_steps,
                "untimed_launches": n_warm + 1,
                "kernel_us": avg * 1e6, "min_us": min(ms) * 1e3, "tokens_per_s": toks / avg,
                "bound": "hbm", "achieved": by / avg / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": by / avg / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": by,
                "mfma_frac_algorithmic": fl / avg / 1e12 / MFMA_BF16_PEAK_TFS}
            log(f"[bench] {cx.name}: {avg * 1e6:.1f} us per call ({nseg} segments, chunk {crun}) = "
                f"{by / avg / 1e9:.0f} GB/s, {configs[cx.name]['frac']:.3f} of HBM peak")
            del tx, ox, sx, wsx
            torch.cuda.empty_cache()

    # ---------------------------------------------------------------- strong decay
    strong = None
    if args.config_steps > 0:
        gen = torch.Generator(device=dev).manual_seed(7)
        a_strong = torch.reciprocal(1.0 + torch.exp(torch.randn(tp["a"].shape, generator=gen, device=dev) + 2.0))

        def run_strong():
            g.chunk_forward(tp["q"], tp["k"], tp["v"], a_strong, tp["b"], tp["w"], None, chunk=cp.chunk,
                            o=o, S_T=S_T, stream=stream)

        # interleaved with the layer's own decay in blocks of 5, so that both
        # see the same clock (the GPU's clock moves under load)
        for _ in range(25):  # ~0.15 s untimed: the clock ramps up after the idle time above
            run_strong()
            prefill()
        ms_s, ms_n = [], []
        for _ in range(max(1, args.config_steps // 5)):
            ms_s += time_each(run_strong, 5)
            ms_n += time_each(prefill, 5)
        avg, avg_n = float(np.mean(ms_s)) / 1e3, float(np.mean(ms_n)) / 1e3
        strong = {"workload": f"{cp.name} with decay pre-activation N(+2, 1) (per-token decay ~0.12)",
                  "launches": len(ms_s), "kernel_us": avg * 1e6, "min_us": min(ms_s) * 1e3,
                  "interleaved_layer_us": avg_n * 1e6, "ratio": avg / avg_n}
        log(f"[bench] strong decay: {avg * 1e6:.1f} us per launch against {avg_n * 1e6:.1f} us for the layer's "
            f"decay interleaved ({avg / avg_n:.2f} x)")
        del a_strong

    # ---------------------------------------------------------------- decode workload leg
    S_dec.copy_(S_dec0)
    torch.cuda.synchronize()
    l0, l1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(dec_steps)]
    l0.record(stream)
    for s in range(dec_steps):
        dev_ev[s][0].record(stream)
        decode(s)
        dev_ev[s][1].record(stream)
    l1.record(stream)
    torch.cuda.synchronize()
    dk_ms = [a.elapsed_time(b) for a, b in dev_ev]
    loop_ms = l0.elapsed_time(l1)
    dbytes = decode_algorithmic(cd.B, cd.H_qk, cd.H_v, cd.d_k, cd.d_v)
    d_avg = float(np.mean(dk_ms)) / 1e3
    d_gbs = dbytes / d_avg / 1e9
    log(f"[bench] decode workload: {dec_steps} steps in {loop_ms:.1f} ms; kernel avg {d_avg * 1e6:.1f} us "
        f"= {d_gbs:.0f} GB/s algorithmic")
    decode_leg = {"steps": dec_steps, "kernel_us": d_avg * 1e6, "loop_us_per_step": loop_ms * 1e3 / dec_steps,
                  "achieved": d_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": d_gbs / HBM_PEAK_GBS,
                  "algorithmic_bytes": dbytes, "state_bytes": cd.B * cd.H_v * cd.d_k * cd.d_v * 4}
    # larger states (beyond the 256 MiB Infinity Cache): random inputs, same head shape
    larger = []
    for N in (1024, 4096):
        xs = gi.draw_on_device(N, 1, cd.H_qk, cd.H_v, cd.d_k, cd.d_v, "bf16", "channel", dev, seed=40 + N)
        Sx = torch.randn((N, cd.H_v, cd.d_k, cd.d_v), device=dev) * 0.02
        ox = torch.empty((N, 1, cd.H_v, cd.d_v), dtype=torch.bfloat16, device=dev)

        def dec_x():
            g.decode_step(xs["q"], xs["k"], xs["v"], xs["a"], xs["b"], xs["w"], Sx, o=ox, stream=stream)

        for _ in range(5):
            dec_x()
        ms = time_each(dec_x, 50)
        by = decode_algorithmic(N, cd.H_qk, cd.H_v, cd.d_k, cd.d_v)
        avg = float(np.mean(ms)) / 1e3
        larger.append({"sequences": N, "state_bytes": N * cd.H_v * cd.d_k * cd.d_v * 4, "steps": 50,
                       "kernel_us": avg * 1e6, "achieved": by / avg / 1e9, "frac": by / avg / 1e9 / HBM_PEAK_GBS})
        log(f"[bench] decode N{N} ({N * cd.H_v * cd.d_k * cd.d_v * 4 >> 20} MiB state): {avg * 1e6:.1f} us "
            f"= {by / avg / 1e9:.0f} GB/s")
        del xs, Sx, ox
        torch.cuda.empty_cache()
    decode_leg["larger_states"] = larger

    # ---------------------------------------------------------------- gate pre-activation leg
    pre_leg = None
    if args.preact_steps > 0:
        tpp = gi.to_torch_preact(gi.make_preact_inputs(cp), cp.dtype, dev)

        def prefill_preact():
            g.chunk_forward_preact(tpp["q"], tpp["k"], tpp["v"], tpp["a"], tpp["b"], tpp["w"], None, chunk=cp.chunk,
                                   o=o, S_T=S_T, stream=stream)

        # untimed calls for ~0.15 s first, as for the other prefill workloads:
        # after the decode legs the clock ramps up again over tens of launches
        t_one = time_each(prefill_preact, 1)[0] / 1e3
        n_warm = max(20, int(0.15 / max(t_one, 1e-6)))
        for _ in range(n_warm):
            prefill_preact()
        p_ms = time_each(prefill_preact, args.preact_steps)
        p_avg = float(np.mean(p_ms)) / 1e3
        pby, _ = prefill_algorithmic(cp, chunk_run, gate_bytes=2 if cp.dtype == "bf16" else 4)
        pre_leg = {"launches": args.preact_steps, "untimed_launches": n_warm + 1,
                   "kernel_us": p_avg * 1e6, "min_us": min(p_ms) * 1e3,
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

        # the chunk form (required; the automatic choice if it refuses the inputs)
        form = "chunk"
        os.environ["GDN2_BACKWARD_CHUNKED"] = "2"
        try:
            grads = backward()
        except RuntimeError:
            form = "automatic"
            os.environ.pop("GDN2_BACKWARD_CHUNKED")
            grads = backward()
        backward(grads)
        torch.cuda.synchronize()
        b_ms = time_each(lambda: backward(grads), args.backward_steps)
        os.environ.pop("GDN2_BACKWARD_CHUNKED", None)
        b_avg = float(np.mean(b_ms)) / 1e3
        bfl, bby = backward_algorithmic(cp)
        bwd = {"form": form, "launches": args.backward_steps, "ms": b_avg * 1e3, "min_ms": min(b_ms),
               "tokens_per_s": tokens / b_avg, "bound": "hbm",
               "achieved": bby / b_avg / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": bby / b_avg / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": bby,
               "recurrence_flops": bfl, "workspace_bytes": bws.numel()}
        log(f"[bench] backward ({form}): {b_avg * 1e3:.2f} ms per launch (min {min(b_ms):.2f}), "
            f"workspace {bws.numel() / 1e9:.2f} GB")
        del grads, bws
        # the per-token backward beside it (its own, larger workspace)
        os.environ["GDN2_BACKWARD_CHUNKED"] = "0"
        bws = torch.empty(g.gdn2_chunk_backward_workspace_bytes(desc), dtype=torch.uint8, device=dev)
        grads = backward()
        torch.cuda.synchronize()
        t_ms = time_each(lambda: backward(grads), max(2, args.backward_steps // 2))
        os.environ.pop("GDN2_BACKWARD_CHUNKED")
        bwd["per_token"] = {"ms": float(np.mean(t_ms)), "min_ms": min(t_ms), "workspace_bytes": bws.numel(),
                            "achieved": bfl / (float(np.mean(t_ms)) / 1e3) / 1e12, "unit": "TFLOP/s",
                            "peak": FP32_VECTOR_PEAK_TFS}
        log(f"[bench] backward (per-token): {np.mean(t_ms):.2f} ms per launch, workspace {bws.numel() / 1e9:.2f} GB")
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

        if USER_BACKWARD_CHUNKED is not None:  # the caller's choice (0: the per-token backward)
            os.environ["GDN2_BACKWARD_CHUNKED"] = USER_BACKWARD_CHUNKED
            lform = {"0": "per-token", "2": "chunk"}.get(USER_BACKWARD_CHUNKED, "automatic")
            gl = backward_long()
        else:
            lform = "chunk"
            os.environ["GDN2_BACKWARD_CHUNKED"] = "2"
            try:
                gl = backward_long()
            except RuntimeError:
                lform = "automatic"
                os.environ.pop("GDN2_BACKWARD_CHUNKED")
                gl = backward_long()
        torch.cuda.synchronize()
        l_ms = time_each(lambda: backward_long(gl), args.long_backward)
        os.environ.pop("GDN2_BACKWARD_CHUNKED", None)
        l_avg = float(np.mean(l_ms)) / 1e3
        lfl, lby = backward_algorithmic(cl)
        bwd_long = {"workload": "backward B1 T65536 H16 d128 bf16", "form": lform,
                    "launches": args.long_backward, "ms": l_avg * 1e3, "min_ms": min(l_ms),
                    "tokens_per_s": cl.B * cl.T / l_avg, "bound": "hbm", "achieved": lby / l_avg / 1e9,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": lby / l_avg / 1e9 / HBM_PEAK_GBS,
                    "algorithmic_bytes": lby, "recurrence_flops": lfl, "workspace_bytes": wsl.numel()}
        log(f"[bench] long-context backward ({lform}): {l_avg * 1e3:.2f} ms per launch (min {min(l_ms):.2f})")
        del gl, wsl, tl

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nthreads = oracle.cores()
        qh = dp["q"] if cp.dtype == "f32" else tp["q"].cpu()
        kh = dp["k"] if cp.dtype == "f32" else tp["k"].cpu()
        vh = dp["v"] if cp.dtype == "f32" else tp["v"].cpu()
        log(f"[bench] oracle on the host, {nthreads} threads, whole prefill batch")
        _, _, el = oracle.forward(qh, kh, vh, dp["a"], dp["b"], dp["w"], None, nthreads=nthreads, timing=True)
        one = lambda x: x[:1, :, :1]
        _, _, el1 = oracle.forward(one(qh), one(kh), one(vh), one(dp["a"]), one(dp["b"]), one(dp["w"]), None,
                                   nthreads=1, timing=True)
        cpu = {"value": tokens / el, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": f"the whole prefill batch once (B={cp.B}, T={cp.T}, {cp.H_v} heads, d={cp.d_k}), "
                         f"fp64 recurrence, threads over (sequence, head), {el:.2f} s",
               "single_thread": {"value": cp.T / el1, "unit": "tokens/s of one (sequence, head)",
                                 "seconds": el1, "sample": f"sequence 0, head 0: T={cp.T}, d={cp.d_k}"}}
        log(f"[bench] oracle {el:.2f} s -> {tokens / el:.0f} tokens/s; one head on one thread {el1:.2f} s")

    out = {
        "metric": METRIC,
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
                         f"{cp.dtype} (chunk run {chunk_run}) + decode step N{cd.B} H{cd.H_v} d{cd.d_k} "
                         f"fp32 state"),
            "chunk_requested": cp.chunk,
            "chunk_run": chunk_run,
            "prefill_kernel_us": pre_avg * 1e6,
            "prefill_kernel_us_median": float(np.median(pre_ms)) * 1e3,
            "prefill_kernel_us_min": float(min(pre_ms)) * 1e3,
            "decode_kernel_us": float(np.mean(dec_ms)) * 1e3,
            "before_headline": (f"{args.series} cold-start prefill launches (series) and {args.warmup} "
                                f"warm-up steps" if series else f"{args.warmup} warm-up steps"),
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
        "series": series,
        "configs": configs,
        "strong_decay": strong,
        "decode": decode_leg,
        "preact": pre_leg,
        "backward": bwd,
        **({"backward_long": bwd_long} if bwd_long else {}),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
