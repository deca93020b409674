#!/usr/bin/env python3
"""Benchmark of the gfx950 attention library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload fb-32K]

A step is one pass of the whole path over one batch of seeded synthetic
inputs already resident in device memory: the forward (attn_fwd) and, for a
workload with gradients, the backward (attn_bwd).  The default workload is
B=1, H=8, N=32768, d=128, causal, bf16 forward + backward.

``value`` is algorithmic TFLOP/s of the whole step: matmul FLOPs only, 4d per
unmasked (query, key) pair in the forward and 10d in the backward, with
N(N+1)/2 unmasked pairs per (batch, head) under the causal mask; recomputed and
masked-diagonal work is not counted.  The roofline object is for the kernel
that takes the most time, measured with HIP events on the library's stream;
the CPU baseline times the fp64 oracle on a bounded sample of the same
workload on this host's cores.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (causal bf16, d=128) at N=8K–32K; % of MFMA bf16 peak"
# MI355X published dense bf16 MFMA peak: 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU.
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12
BENCH_WORKLOADS = ("fb-32K", "fwd-8K", "gqa-16K", "fwd-2K")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="fb-32K", choices=BENCH_WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle (for profiler runs)")
    ap.add_argument("--cpu-sample-heads", type=int, default=None,
                    help="query heads in the oracle's timed sample (default: sized for ~10-30 s)")
    return ap.parse_args()


def cpu_baseline(w, x, n_heads):
    """Time the fp64 oracle on the first n_heads query heads (batch 0, full N)."""
    import torch

    from oracle import attention_backward, attention_forward
    from synth_inputs import bf16_bits_to_f64

    hq = max(1, min(n_heads, w.Hq))
    hk = max(1, hq // w.group)            # the K/V heads those query heads read
    sl = lambda name, h: torch.from_numpy(bf16_bits_to_f64(x[name][:1, :h].copy()))
    q, k, v = sl("q", hq), sl("k", hk), sl("v", hk)
    threads = torch.get_num_threads()
    t0 = time.perf_counter()
    attention_forward(q, k, v, True)
    pairs = hq * w.N * (w.N + 1) // 2
    flops = 4 * w.d * pairs
    if w.with_grad:
        attention_backward(q, k, v, sl("do", hq), True)
        flops += 10 * w.d * pairs
    dt = time.perf_counter() - t0
    what = "forward + backward" if w.with_grad else "forward"
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"fp64 oracle {what} on batch 0, query heads 0..{hq - 1} of {w.Hq}, full N={w.N}, "
                  f"same seeded inputs (algorithmic {flops:.3g} FLOP in {dt:.2f} s; the oracle "
                  f"evaluates full masked rows)",
        "host": platform.processor() or platform.machine(),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the library runs on one device; a multi-GPU split is not part of it)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import io_aware_exact_fwd_amd as attn
    from synth_inputs import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (the HIP library has no CPU path)", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    rc = attn.device_check(0)
    if rc != 0:
        print(f"device 0 unusable: {attn.strerror(rc)}", file=sys.stderr)
        sys.exit(1)

    w = WORKLOADS[args.workload]
    steps = args.steps if args.steps is not None else (20 if w.with_grad else 50)
    warmup = args.warmup if args.warmup is not None else 3
    x = make_inputs(w)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
    if w.with_grad:
        do = dev(x["do"])
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(max(16, attn.bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d)),
                         dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        attn.fwd(q, k, v, causal=True, out=o, lse=lse, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        if w.with_grad:
            attn.bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws, stream=stream)
            if ev is not None:
                ev[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    fwd_ms = [e[0].elapsed_time(e[1]) for e in events]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in events] if w.with_grad else []
    ms_per_step = wall * 1e3 / steps
    fwd_flops = w.fwd_flops(True)
    bwd_flops = w.bwd_flops(True) if w.with_grad else 0
    step_flops = fwd_flops + bwd_flops
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    fwd_avg = float(np.mean(fwd_ms))
    parts = {"fwd": {"ms_avg": fwd_avg, "ms_median": float(np.median(fwd_ms)),
                     "tflops": fwd_flops / (fwd_avg * 1e-3) / 1e12}}
    parts["fwd"]["pct_of_peak"] = 100 * parts["fwd"]["tflops"] / PEAK_BF16_TFLOPS
    if w.with_grad:
        bwd_avg = float(np.mean(bwd_ms))
        parts["bwd"] = {"ms_avg": bwd_avg, "ms_median": float(np.median(bwd_ms)),
                        "tflops": bwd_flops / (bwd_avg * 1e-3) / 1e12}
        parts["bwd"]["pct_of_peak"] = 100 * parts["bwd"]["tflops"] / PEAK_BF16_TFLOPS

    # the dominant launch: the forward kernel, or the backward call when it takes longer
    dom = max(parts, key=lambda p: parts[p]["ms_avg"])
    dom_flops = fwd_flops if dom == "fwd" else bwd_flops
    achieved = dom_flops / (parts[dom]["ms_avg"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                "kernel": "attn_fwd_kernel" if dom == "fwd" else "attn_bwd (all backward kernels)"}

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": True, "pass": "fwd+bwd" if w.with_grad else "fwd",
                   "flops_per_step": step_flops, "seed": w.seed, "input_scale": w.in_scale},
        "pct_of_peak": 100 * value / PEAK_BF16_TFLOPS,
        "parts": parts,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        default_heads = {"fb-32K": 1, "gqa-16K": 8, "fwd-8K": 16, "fwd-2K": 64}[w.name]
        result["cpu_baseline"] = cpu_baseline(w, x, args.cpu_sample_heads or default_heads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
