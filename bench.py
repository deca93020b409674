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
import math
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
BENCH_WORKLOADS = ("fb-32K", "fwd-8K", "gqa-16K", "fwd-2K", "swa-32K", "decode-32K", "varlen-32K",
                   "fp8-8K")
PEAK_HBM_GBPS = 8000.0
# dense 8-bit (E4M3) MFMA peak: twice the bf16 rate per CU and clock
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS


COUNTERS_JSON = os.path.join(ROOT, "profiles", "counters.json")
CSRC = os.path.join(ROOT, "io_aware_exact_fwd_amd", "csrc")
# source files each kernel is compiled and launched from (their hash decides
# whether recorded counters still describe the kernel)
_SHARED = ("attn_device.h", "attn_layout.h", "attn_launch.h")
KERNEL_SOURCES = {
    "attn_fwd_kernel": _SHARED + ("attn_fwd.hip",),
    "bwd_pre_kernel": _SHARED + ("attn_bwd.hip",),
    "bwd_dkdv_kernel": _SHARED + ("attn_bwd.hip",),
    "bwd_dq_kernel": _SHARED + ("attn_bwd.hip",),
    "bwd_grads_kernel": _SHARED + ("attn_bwd.hip",),
    "attn_decode_split_kernel": _SHARED + ("attn_decode.hip",),
    "attn_fwd_fp8_kernel": _SHARED + ("attn_fwd_fp8.hip",),
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def source_sha(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _per_kernel(csv_path: str, counter: str):
    """Average value of one counter per dispatch, by kernel short name.  For the
    copy kernel, the largest dispatch: the calibration copy, not the small
    uploads of the inputs that run through the same kernel."""
    import csv
    import collections
    acc = collections.defaultdict(list)
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            short = next((k for k in KERNEL_SOURCES if k in name), COPY_KERNEL if COPY_KERNEL in name else None)
            if short:
                acc[short].append(float(r["Counter_Value"]))
    return {k: (max(v) if k == COPY_KERNEL else sum(v) / len(v)) for k, v in acc.items()}


def ingest_counters(fetch_csv: str, write_csv: str, calib_mib: int, workload: str,
                    mfma_csv: str | None = None) -> dict:
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) -> the workload's record in
    profiles/counters.json (records of other workloads are kept).

    Both counters are scaled by what they read for the plain copy of calib_mib
    MiB that ran in the same process (it reads and writes calib_mib MiB).
    """
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    kib = calib_mib * 1024.0
    fs, ws = kib / fetch[COPY_KERNEL], kib / write[COPY_KERNEL]
    out = {"workload": workload, "fetch_scale": fs, "write_scale": ws,
           "calibration": f"one {calib_mib} MiB device copy ({COPY_KERNEL}) in the same process read "
                          f"FETCH_SIZE={fetch[COPY_KERNEL]:.0f} KiB, WRITE_SIZE={write[COPY_KERNEL]:.0f} KiB",
           "kernels": {}}
    mfma = {}
    if mfma_csv:
        for c in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"):
            mfma[c] = _per_kernel(mfma_csv, c)
    for k in KERNEL_SOURCES:
        if k not in fetch or k not in write:
            continue
        e = {"source_sha": source_sha(k), "fetch_kib": fetch[k], "write_kib": write[k],
             "hbm_bytes": (fetch[k] * fs + write[k] * ws) * 1024.0}
        if mfma and k in mfma["SQ_INSTS_VALU_MFMA_MOPS_BF16"]:
            e["mfma_flop"] = mfma["SQ_INSTS_VALU_MFMA_MOPS_BF16"][k] * 512
            e["mfma_busy_cycles"] = mfma["SQ_VALU_MFMA_BUSY_CYCLES"][k]
            e["grbm_gui_active"] = mfma["GRBM_GUI_ACTIVE"][k]
        out["kernels"][k] = e
    os.makedirs(os.path.dirname(COUNTERS_JSON), exist_ok=True)
    try:
        with open(COUNTERS_JSON) as fh:
            allrec = json.load(fh)
    except (OSError, ValueError):
        allrec = {}
    allrec[workload] = out
    with open(COUNTERS_JSON, "w") as fh:
        json.dump(allrec, fh, indent=1)
    return out


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch from recorded counters, or None when the kernel's
    sources changed since they were taken (or none were taken)."""
    try:
        with open(COUNTERS_JSON) as fh:
            rec = json.load(fh).get(workload, {})
    except (OSError, ValueError):
        return None
    e = rec.get("kernels", {}).get(kernel)
    if not e or e.get("source_sha") != source_sha(kernel):
        return None
    return e["hbm_bytes"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="fb-32K", choices=BENCH_WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle (for profiler runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before warm-up, so a "
                         "counter run can scale FETCH_SIZE/WRITE_SIZE by a kernel of known traffic")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/counters.json from two rocprofv3 --pmc CSVs and exit")
    ap.add_argument("--ingest-mfma", metavar="MFMA_CSV", default=None)
    ap.add_argument("--cold-cache", choices=("auto", "on", "off"), default="auto",
                    help="also time each kernel after a 512 MiB scratch write that flushes L2 and "
                         "the last-level cache (auto: fwd-2K only)")
    ap.add_argument("--cpu-sample-heads", type=int, default=None,
                    help="query heads in the oracle's timed sample (default: sized for ~10-30 s)")
    ap.add_argument("--forward-legs", choices=("auto", "on", "off"), default="auto",
                    help="also time the forward alone at fwd-8K and gqa-16K, reported under "
                         "parts.fwd8k / parts.gqa16k (auto: with the default fb-32K workload)")
    return ap.parse_args()


def host_info() -> dict:
    """What the CPU baseline ran on: model, usable cores, thread settings, BLAS build."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    import numpy as np
    import torch
    blas = None
    try:
        deps = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{deps.get('name')} {deps.get('version')}"
    except Exception:  # older numpy: no dict mode
        pass
    return {"cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0)),
            "torch_threads": torch.get_num_threads(), "numpy_blas": blas}


def cpu_baseline(w, x, n_heads):
    """Time the fp64 oracle on the first n_heads query heads (batch 0, full N)."""
    import torch

    from oracle import (attention_backward, attention_forward, fp8_attention_forward, varlen_backward,
                        varlen_forward)
    from synth_inputs import bf16_bits_to_f64

    hq = max(1, min(n_heads, w.Hq))
    hk = max(1, hq // w.group)            # the K/V heads those query heads read
    nb = w.B if w.nq is not None else 1   # decoding is cheap enough to take every sequence
    threads = torch.get_num_threads()
    pairs = nb * hq * w.keys_per_query(True)
    flops = (4 * w.d + (10 * w.d if w.with_grad else 0)) * pairs
    what = "forward + backward" if w.with_grad else "forward"
    if w.fp8:
        sl8 = lambda name, h: x[name][:1, :h].copy()
        t0 = time.perf_counter()
        fp8_attention_forward(sl8("q8", hq), sl8("k8", hk), sl8("v8", hk), x["q_descale"][:1, :hq],
                              x["k_descale"][:1, :hk], x["v_descale"][:1, :hk], True)
        dt = time.perf_counter() - t0
        return {
            "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle forward of the dequantized E4M3 inputs on query heads 0..{hq - 1} "
                      f"of {w.Hq}, full N={w.N}, same seeded inputs (algorithmic {flops:.3g} FLOP in "
                      f"{dt:.2f} s; the oracle evaluates full masked rows)",
            "host": host_info(),
        }
    if w.pack is not None:
        # packed batch: every sequence of the first hq query heads
        sl = lambda name, h: torch.from_numpy(bf16_bits_to_f64(x[name][:h].copy()))
        q, k, v = sl("q", hq), sl("k", hk), sl("v", hk)
        cu = x["cu_seqlens"].tolist()
        t0 = time.perf_counter()
        varlen_forward(q, k, v, cu, True)
        if w.with_grad:
            varlen_backward(q, k, v, sl("do", hq), cu, True)
        dt = time.perf_counter() - t0
        return {
            "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle {what} on query heads 0..{hq - 1} of {w.Hq}, every packed "
                      f"sequence ({len(cu) - 1}, T={w.N}), same seeded inputs (algorithmic "
                      f"{flops:.3g} FLOP in {dt:.2f} s; the oracle evaluates full masked rows)",
            "host": host_info(),
        }
    sl = lambda name, h: torch.from_numpy(bf16_bits_to_f64(x[name][:nb, :h].copy()))
    q, k, v = sl("q", hq), sl("k", hk), sl("v", hk)
    t0 = time.perf_counter()
    attention_forward(q, k, v, True, window=w.window)
    if w.with_grad:
        attention_backward(q, k, v, sl("do", hq), True, window=w.window)
    dt = time.perf_counter() - t0
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"fp64 oracle {what} on batches 0..{nb - 1}, query heads 0..{hq - 1} of {w.Hq}, full N={w.N}, "
                  f"same seeded inputs (algorithmic {flops:.3g} FLOP in {dt:.2f} s; the oracle "
                  f"evaluates full masked rows)",
        "host": host_info(),
    }


# Secondary forward-only legs: the causal forward at N = 8192 (32 heads) and
# N = 16384 (64 query heads over 8 K/V heads), timed after the headline step
# with the same warm-up and timing rules; they do not enter ``value``.
FORWARD_LEGS = (("fwd8k", "fwd-8K"), ("gqa16k", "gqa-16K"))


def time_forward_leg(attn, name, steps_arg, warmup_arg, min_seconds=1.0):
    """Mean/median/min/p90 of attn_fwd at one workload (inputs resident in HBM,
    each launch bracketed by events on the stream it runs on)."""
    import numpy as np
    import torch

    from synth_inputs import WORKLOADS, make_inputs

    w = WORKLOADS[name]
    x = make_inputs(w)
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    del x
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    launch = lambda: attn.fwd(q, k, v, causal=True, out=o, lse=lse, stream=stream)
    t_w = time.perf_counter()
    if warmup_arg is not None:
        warmup = warmup_arg
        for _ in range(warmup):
            launch()
        torch.cuda.synchronize()
    else:
        warmup = 0
        while True:
            for _ in range(10):
                launch()
            warmup += 10
            torch.cuda.synchronize()
            if time.perf_counter() - t_w >= min_seconds:
                break
    per_launch = (time.perf_counter() - t_w) / max(warmup, 1)
    steps = steps_arg if steps_arg is not None else max(50, min(20000, math.ceil(min_seconds / per_launch)))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        launch()
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    flops = w.fwd_flops(True)
    leg = {"workload": name, "kernel": "attn_fwd_kernel", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N,
           "d": w.d, "causal": True, "input_scale": w.in_scale, "seed": w.seed, "warmup": warmup,
           "steps": steps, "ms_avg": float(np.mean(ms)), "ms_median": float(np.median(ms)),
           "ms_min": float(np.min(ms)), "ms_p90": float(np.percentile(ms, 90)), "algorithmic_flops": flops}
    leg["tflops"] = flops / (leg["ms_avg"] * 1e-3) / 1e12
    leg["tflops_median"] = flops / (leg["ms_median"] * 1e-3) / 1e12
    leg["pct_of_peak"] = 100 * leg["tflops"] / PEAK_BF16_TFLOPS
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return leg


def main():
    args = parse()
    if args.ingest_counters:
        rec = ingest_counters(args.ingest_counters[0], args.ingest_counters[1],
                              args.copy_calibration_mib or 1024, args.workload, args.ingest_mfma)
        print(json.dumps(rec, indent=1))
        return
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
    steps = args.steps if args.steps is not None else 50
    warmup = args.warmup if args.warmup is not None else 10
    x = make_inputs(w)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

    if w.fp8:
        q8, k8, v8 = (torch.from_numpy(x[n]).cuda() for n in ("q8", "k8", "v8"))
        q_ds, k_ds, v_ds = (torch.from_numpy(x[n]).cuda() for n in ("q_descale", "k_descale", "v_descale"))
        q = torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.bfloat16, device="cuda")   # O's shape
    else:
        q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    o = torch.empty_like(q)
    nq = w.N if w.nq is None else w.nq
    packed = w.pack is not None
    # packed batches are [H, T, d] with LSE and D [H, T]
    row_shape = (w.Hq, w.N) if packed else (w.B, w.Hq, nq)
    lse = torch.empty(row_shape, dtype=torch.float32, device="cuda")
    decode = w.nq is not None
    if packed:
        lengths = w.lengths()
        cu = torch.from_numpy(x["cu_seqlens"]).cuda()
        max_len = max(lengths)
    if decode:
        ws = torch.empty(attn.decode_workspace_bytes(w.B, w.Hq, w.Hkv, nq, w.N, w.d), dtype=torch.uint8,
                         device="cuda")
    if w.with_grad:
        do = dev(x["do"])
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty(row_shape, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    # Each phase is one kernel launch (the decode phase: the split kernel and
    # its small merge); events between them give per-kernel durations on the
    # stream the kernels run on.  The two backward phases are exactly what
    # attn_bwd runs, in the same order.
    phases = (["decode"] if decode else ["fwd"]) + (["bwd_pre", "bwd_grads"] if w.with_grad else [])

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        if decode:
            attn.fwd_decode(q, k, v, causal=True, out=o, lse=lse, workspace=ws, stream=stream)
        elif packed:
            attn.fwd_varlen(q, k, v, cu, max_len, causal=True, out=o, lse=lse, stream=stream)
        elif w.fp8:
            attn.fwd_fp8(q8, k8, v8, q_ds, k_ds, v_ds, causal=True, out=o, lse=lse, stream=stream)
        else:
            attn.fwd(q, k, v, causal=True, out=o, lse=lse, stream=stream, window=w.window)
        mark(1)
        if w.with_grad and packed:
            # the pre-pass over packed rows is the plain one with B = 1, N = T
            attn.bwd_preprocess(o[None], do[None], delta[None], stream=stream)
            mark(2)
            attn.bwd_grads_varlen(q, k, v, do, lse, delta, cu, max_len, causal=True, dq=dq, dk=dk,
                                  dv=dv, stream=stream)
            mark(3)
        elif w.with_grad:
            attn.bwd_preprocess(o, do, delta, stream=stream)
            mark(2)
            attn.bwd_grads(q, k, v, do, lse, delta, causal=True, dq=dq, dk=dk, dv=dv,
                           stream=stream, window=w.window)
            mark(3)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)                     # reads n bytes, writes n bytes
        torch.cuda.synchronize()
        del src, dst

    # Without --warmup, warm up for at least 10 steps and 1 s, so that short
    # workloads run at the clock a sustained job sees; without --steps, time at
    # least 50 steps and at least 1 s.  Explicit values are used as given.
    min_seconds = 1.0
    if args.warmup is not None:
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
    else:
        warmup = 0
        t_w = time.perf_counter()
        while True:
            for _ in range(10):
                step()
            warmup += 10
            torch.cuda.synchronize()
            if time.perf_counter() - t_w >= min_seconds:
                break
        if args.steps is None:
            per_step = (time.perf_counter() - t_w) / warmup
            steps = max(steps, min(20000, math.ceil(min_seconds / per_step)))

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_per_step = wall * 1e3 / steps

    # cold-cache leg (untimed in ``value``): before each step a 512 MiB scratch
    # write evicts L2 and the last-level cache, so the inputs come from HBM again
    cold = args.cold_cache == "on" or (args.cold_cache == "auto" and w.name == "fwd-2K")
    cold_events = []
    if cold:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cold_steps = min(steps, 200)
        cold_events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
                       for _ in range(cold_steps)]
        for i in range(cold_steps):
            scratch.fill_(i & 0xFF)
            step(cold_events[i])
        torch.cuda.synchronize()
        del scratch
    pairs = w.pairs(True)
    # algorithmic matmul FLOPs per unmasked pair, by kernel: the forward's QK^T
    # and PV (4d); the gradient kernel's S, dP, dV, dK and dQ (10d -- the dQ
    # blocks' second S and dP are recomputation and not counted); the pre-pass
    # does no matmul.
    per_pair = {"fwd": 4 * w.d, "bwd_pre": 0, "bwd_grads": 10 * w.d, "decode": 4 * w.d}
    kernel_name = {"fwd": "attn_fwd_fp8_kernel" if w.fp8 else "attn_fwd_kernel", "bwd_pre": "bwd_pre_kernel",
                   "bwd_grads": "bwd_grads_kernel", "decode": "attn_decode_split_kernel"}
    fwd_flops = w.fwd_flops(True)
    bwd_flops = w.bwd_flops(True) if w.with_grad else 0
    step_flops = fwd_flops + bwd_flops
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    mfma_peak = PEAK_FP8_TFLOPS if w.fp8 else PEAK_BF16_TFLOPS
    def stats(ms):
        return {"ms_avg": float(np.mean(ms)), "ms_median": float(np.median(ms)), "ms_min": float(np.min(ms)),
                "ms_p90": float(np.percentile(ms, 90))}

    parts = {}
    for i, ph in enumerate(phases):
        st = stats([e[i].elapsed_time(e[i + 1]) for e in events])
        flops = per_pair[ph] * pairs
        parts[ph] = {"kernel": kernel_name[ph], **st, "algorithmic_flops": flops,
                     "tflops": flops / (st["ms_avg"] * 1e-3) / 1e12,
                     "tflops_median": flops / (st["ms_median"] * 1e-3) / 1e12}
        parts[ph]["pct_of_peak"] = 100 * parts[ph]["tflops"] / mfma_peak
        if cold_events:
            cs = stats([e[i].elapsed_time(e[i + 1]) for e in cold_events])
            cs["tflops_median"] = flops / (cs["ms_median"] * 1e-3) / 1e12
            parts[ph]["cold_cache"] = cs
    if w.with_grad:
        bwd_ms = sum(parts[p]["ms_avg"] for p in phases[1:])
        parts["bwd_total"] = {"ms_avg": bwd_ms, "tflops": bwd_flops / (bwd_ms * 1e-3) / 1e12,
                              "pct_of_peak": 100 * bwd_flops / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}

    dom = max(phases, key=lambda p: parts[p]["ms_avg"])
    traffic = recorded_traffic(kernel_name[dom], w.name)
    if decode:
        # HBM-bound: K and V once, Q in, O and LSE out
        alg_bytes = 2 * w.B * w.Hkv * w.N * w.d * 2 + 2 * w.B * w.Hq * nq * w.d * 2 + w.B * w.Hq * nq * 4
        gbps = alg_bytes / (parts[dom]["ms_avg"] * 1e-3) / 1e9
        parts[dom]["algorithmic_bytes"] = alg_bytes
        parts[dom]["gbps"] = gbps
        roofline = {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": gbps / PEAK_HBM_GBPS, "traffic": traffic, "kernel": kernel_name[dom],
                    "ms_per_launch": parts[dom]["ms_avg"], "algorithmic_bytes_per_launch": alg_bytes}
    else:
        achieved = parts[dom]["tflops"]
        peak = PEAK_FP8_TFLOPS if w.fp8 else PEAK_BF16_TFLOPS
        roofline = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                    "frac": achieved / peak, "traffic": traffic, "kernel": kernel_name[dom],
                    "ms_per_launch": parts[dom]["ms_avg"],
                    "algorithmic_flops_per_launch": parts[dom]["algorithmic_flops"]}

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
        "dtype": "fp8" if w.fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": True, "pass": "fwd+bwd" if w.with_grad else ("decode" if decode else "fwd"),
                   "flops_per_step": step_flops, "seed": w.seed, "input_scale": w.in_scale,
                   "window": w.window, "queries": nq,
                   "packed_lengths": w.lengths() if packed else None},
        "pct_of_peak": 100 * value / mfma_peak,
        "parts": parts,
        "roofline": roofline,
        "versions": {"torch": torch.__version__, "hip": torch.version.hip,
                     "arch": torch.cuda.get_device_properties(0).gcnArchName},
    }
    legs = args.forward_legs == "on" or (args.forward_legs == "auto" and w.name == "fb-32K")
    if legs:
        for key, name in FORWARD_LEGS:
            parts[key] = time_forward_leg(attn, name, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        default_heads = {"fb-32K": 1, "gqa-16K": 8, "fwd-8K": 16, "fwd-2K": 64, "swa-32K": 1,
                         "decode-32K": 32, "varlen-32K": 3, "fp8-8K": 16}[w.name]
        result["cpu_baseline"] = cpu_baseline(w, x, args.cpu_sample_heads or default_heads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
