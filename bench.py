#!/usr/bin/env python3
"""Benchmark: single-token MoE-layer decode on one MI355X.

Workload "decode4": one MoE layer at the 397B model's shape (hidden 4096, 512 experts,
intermediate 1024, top-3 routed + 1 shared, 4-bit group-64 experts). It runs 1000 seeded
tokens, each as its own single-token moe_layer_forward call, stream-ordered and captured in
one HIP graph. A step is one pass over those 1000 tokens. The inputs are synthetic (the
trained weights are not available) and resident in HBM before timing starts.

Printed as one JSON line:
- value: tokens/s over the K timed steps.
- roofline: achieved algorithmic GB/s of the dominant kernel against the 8 TB/s HBM peak. Each
  launch is timed live with start/stop HIP events that the dispatch itself records
  (hipExtLaunchKernel), i.e. the kernel's own begin and end timestamps.
- cold: the same decode with the router and shared expert rotated over 64 replicas, so that
  no weight byte is reused from the 256 MB Infinity Cache between tokens.
- cpu_baseline: the fp64 oracle on a bounded sample of the same tokens, on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KERNEL_NAMES = ["router (fp64)", "gate/up + SwiGLU (routed + shared)", "down + combine"]
PAIR_NAME = "router + top-K + gate/up + SwiGLU (one launch)"


def _hip():
    h = ctypes.CDLL("libamdhip64.so")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return h


def algorithmic_bytes(w, bq):
    """Bytes each kernel must read once per token (weights only; activations excluded)."""
    H, I, E, K = w.hidden, w.inter, w.n_experts, w.top_k
    blob = bq.moe_blob_bytes(H, I, w.bits, w.group)
    gate_up = 2 * blob // 3  # gate + up codes and (scale, bias) words
    down = blob // 3
    router = E * H * 2 + H * 2
    return [router, (K + 1) * gate_up, (K + 1) * down], K * blob + blob, router


def kernel_hash():
    src = os.path.join(ROOT, "bit_quantized_expert_gemv_amd", "csrc", "moe_kernels.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def load_traffic(kernel_label, workload):
    """HBM traffic per launch from committed rocprofv3 --pmc summaries, if taken on this workload and on
    this kernel source."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    if d.get("kernel_source_sha256_16") != kernel_hash():
        return None
    return d.get("per_launch_bytes", {}).get(kernel_label)


def stream_read_gbs(torch, gib=4, reps=5):
    """Measured streaming-read rate of this GPU through torch alone: a dot product of two fp32 vectors
    of `gib`/2 GiB each (`gib` GiB read, nothing written), best of `reps` runs. Of the read-only torch
    operations it is the fastest measured here (sum and amax read ~10% slower); a hand-written
    streaming kernel reads faster still, so this is a floor for the reachable read bandwidth, not the
    8 TB/s spec peak."""
    n = (gib << 30) // 8
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.ones(n, dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.dot(a, b)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / 1000.0)
    del a, b
    torch.cuda.empty_cache()
    return (gib << 30) / best / 1e9


def cpu_baseline(w, budget_s):
    """The oracle as it stands, on the host cores: tokens taken in a stride order that spreads over
    all of the workload's tokens, until every token has run or ~budget_s of oracle time has passed
    with every OpenMP thread, then the same tokens again with one thread for ~min(budget_s / 2, 6) s."""
    import ctypes

    import numpy as np

    import oracle
    import synth

    try:
        gomp = ctypes.CDLL("libgomp.so.1")  # the OpenMP runtime the oracle library is built on
    except OSError:
        gomp = None
    router = synth.router_weights(w)
    gate = synth.shared_gate_weights(w)
    shared = synth.expert_arrays(w, 0, synth.SHARED)
    stride = next(p for p in range(w.tokens // 3, w.tokens) if np.gcd(p, w.tokens) == 1)
    order = [(i * stride) % w.tokens for i in range(w.tokens)]

    def run(budget):
        spent, n = 0.0, 0
        while spent < budget and n < w.tokens:
            t = order[n]
            x = synth.tokens_x(w, t, 1)[0].astype(np.float64)
            idx = oracle.topk(oracle.router_logits(router, x), w.top_k)  # untimed: which experts to generate
            arrays = {int(e): synth.expert_arrays(w, 0, int(e)) for e in idx}
            t0 = time.perf_counter()
            oracle.layer(x, x, router, gate, arrays.__getitem__, w.top_k, w.group, shared_expert=shared)
            spent += time.perf_counter() - t0
            n += 1
        return n, spent

    threads = int(gomp.omp_get_max_threads()) if gomp else (os.cpu_count() or 1)
    n, spent = run(budget_s)
    n1, spent1 = 0, 0.0
    if gomp:
        gomp.omp_set_num_threads(1)
        try:
            n1, spent1 = run(min(budget_s / 2, 6.0))
        finally:
            gomp.omp_set_num_threads(threads)
    lo, hi = min(order[:n]), max(order[:n])
    return {"value": n / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "one_core": {"value": n1 / spent1, "unit": "tokens/s", "cores": 1, "tokens": n1} if n1 else None,
            "sample": f"{n} of the {w.tokens} {w.name} tokens (stride {stride} through all of them, so spread over "
                      f"{lo}..{hi}), one at a time: router, top-K, {w.top_k} routed + shared experts dense-dequantised "
                      f"in fp64, combine; expert generation untimed; {spent:.1f} s of oracle time on {threads} "
                      f"threads, then the first {n1} of them on one thread ({spent1:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="decode4", choices=["decode4", "decode2", "decodemx", "prefill4", "prefillmx", "stack60"])
    ap.add_argument("--cpu-budget", type=float, default=28.0,
                    help="at most this many seconds of oracle time for cpu_baseline (all decode4 tokens take ~20-26 s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true")
    ap.add_argument("--dequant", default="xsum", choices=["xsum", "literal", "naive"],
                    help="decode GEMV arithmetic: per-chunk x-sum form (default), the pages' per-element "
                         "fma(q, s*x, b*x) form, or the naive (q*s + b)*x form; an A/B ablation")
    ap.add_argument("--tokens-per-call", type=int, default=1,
                    help="decode workloads: run the step's tokens as calls of this many tokens each (small-batch "
                         "decode below the prefill threshold, or the grouped path from it), one graph per step")
    ap.add_argument("--chain", action="store_true",
                    help="single-token decode as the three-kernel chain even where the two-launch plan applies (A/B)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="first run a plain device copy of this many MiB (a known-size reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU sharding is design-only, "
              "see the sharding section of the design notes", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_quantized_expert_gemv_amd as bq
    import synth
    from synth.gpu_layers import DeviceLayer

    if args.copy_probe_mb:
        nbytes = args.copy_probe_mb << 20
        src = torch.ones(nbytes // 4, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy probe: {nbytes} bytes read, {nbytes} bytes written", file=sys.stderr, flush=True)
        del src, dst
    w = synth.WORKLOADS[args.workload]
    if w.prefill:
        return bench_prefill(args, w)
    if w.layers > 1:
        return bench_stack(args, w)
    if args.tokens_per_call > 1:
        return bench_batched(args, w, args.tokens_per_call)
    N = w.tokens
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] building {w.name} layer", file=sys.stderr, flush=True)
    L = DeviceLayer(w, device=dev)
    flags = {"xsum": 0, "literal": bq.MOE_FLAG_DEQUANT_LITERAL, "naive": bq.MOE_FLAG_DEQUANT_NAIVE}[args.dequant]
    if args.chain:
        flags |= bq.MOE_FLAG_DECODE_CHAIN
    L.desc.flags = flags
    plan = bq.moe_layer_plan(L.desc, 1)
    plan_name = {bq.MOE_PLAN_PAIR: "two launches", bq.MOE_PLAN_CHAIN: "three-kernel chain"}[plan]
    print(f"[bench] plan: {plan_name}", file=sys.stderr, flush=True)
    X = torch.from_numpy(synth.tokens_x(w, 0, N)).to(dev)
    out = torch.empty_like(X)
    idx = torch.empty(N, w.top_k, dtype=torch.int32, device=dev)
    nws = bq.moe_workspace_bytes(L.desc, 1)
    ws = torch.zeros(nws, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()

    def capture(desc_for_token):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for t in range(N):
                bq.moe_layer_forward(desc_for_token(t), X[t], X[t], 1, out[t], idx[t], ws, nws, stream=stream)
        return g

    def timed(g, steps, warmup):
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(steps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1000.0

    print("[bench] capturing graph", file=sys.stderr, flush=True)
    g = capture(lambda t: L.desc)
    secs = timed(g, args.steps, args.warmup)
    tok_s = args.steps * N / secs
    ms_per_step = secs * 1000.0 / args.steps
    print(f"[bench] warm: {tok_s:,.0f} tokens/s ({secs * 1e6 / (args.steps * N):.2f} us/token)", file=sys.stderr,
          flush=True)

    # ---- per-kernel durations, live, with HIP events around each launch (eager, same stream)
    hip = _hip()
    per_kernel_bytes, expert_bytes, router_bytes = algorithmic_bytes(w, bq)
    names, pairs = KERNEL_NAMES, [0, 1, 2]  # per kernel: the index p of its event pair (2p, 2p + 1)
    if plan == bq.MOE_PLAN_PAIR:  # router rows and gate/up in the first launch, down in the second
        names, pairs = [PAIR_NAME, KERNEL_NAMES[2]], [0, 2]
        per_kernel_bytes = [per_kernel_bytes[0] + per_kernel_bytes[1], per_kernel_bytes[2]]
    nk = len(names)
    events = []
    for _ in range(6 * N):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        events.append(e.value)
    with torch.cuda.stream(stream):
        for t in range(N):
            bq.moe_layer_forward_timed(L.desc, X[t], X[t], 1, out[t], idx[t], ws, nws, events[6 * t: 6 * t + 6],
                                       stream=stream)
    torch.cuda.synchronize()
    dur = np.zeros((N, nk))
    f = ctypes.c_float()
    for t in range(N):
        for k in range(nk):
            pk = pairs[k]
            assert hip.hipEventElapsedTime(ctypes.byref(f), events[6 * t + 2 * pk], events[6 * t + 2 * pk + 1]) == 0
            dur[t, k] = f.value * 1e-3
    for e in events:
        hip.hipEventDestroy(e)
    avg = dur[10:].mean(axis=0)  # skip the first tokens (cold instruction caches)
    dom = int(np.argmax(per_kernel_bytes))
    achieved = per_kernel_bytes[dom] / avg[dom] / 1e9
    kernels = {names[k]: {"avg_us": round(avg[k] * 1e6, 3), "bytes": per_kernel_bytes[k],
                          "GB/s": round(per_kernel_bytes[k] / avg[k] / 1e9, 1)} for k in range(nk)}
    print(f"[bench] kernels: {json.dumps(kernels)}", file=sys.stderr, flush=True)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(names[dom], w.name),
                "kernel": names[dom], "algorithmic_bytes_per_launch": per_kernel_bytes[dom],
                "avg_launch_us": round(avg[dom] * 1e6, 3),
                "timing": f"start/stop HIP events recorded by each dispatch itself (hipExtLaunchKernel) on the "
                          f"kernel's stream, averaged over {N - 10} single-token launches",
                "kernels": kernels}

    # ---- cache-cold variant: rotate 64 replicas of router + shared expert + gate
    cold = None
    if not args.no_cold:
        R = 64
        rep_router = L.router.repeat(R, 1) if L.router.dim() == 1 else L.router.reshape(1, -1).repeat(R, 1)
        rep_gate = L.shared_gate.reshape(1, -1).repeat(R, 1)
        rep_shared = torch.empty(R, L.stride, dtype=torch.uint8, device=dev)
        rep_shared[:] = L.shared.reshape(1, -1)
        descs = [bq.make_layer(w.hidden, w.inter, w.n_experts, w.top_k, w.bits, L.experts, L.stride, rep_router[r],
                               rep_shared[r], rep_gate[r], w.group, flags) for r in range(R)]
        gc = capture(lambda t: descs[t % R])
        csecs = timed(gc, args.steps, args.warmup)
        ctok = args.steps * N / csecs
        us = csecs * 1e6 / (args.steps * N)
        cold = {"tokens_per_s": round(ctok, 1), "us_per_token": round(us, 3),
                "expert_GB/s": round(expert_bytes / (us * 1e-6) / 1e9, 1),
                "all_weights_GB/s": round((expert_bytes + router_bytes) / (us * 1e-6) / 1e9, 1),
                "replicas": R, "replica_bytes": int((L.stride + L.router.numel() * 2 + L.shared_gate.numel() * 2) * R)}
        print(f"[bench] cold: {json.dumps(cold)}", file=sys.stderr, flush=True)
        del gc

    us_tok = secs * 1e6 / (args.steps * N)
    read_peak = stream_read_gbs(torch)
    print(f"[bench] measured streaming read: {read_peak:,.0f} GB/s", file=sys.stderr, flush=True)
    result = {
        "metric": "MoE-layer decode tokens/s + achieved HBM GB/s on expert weights (frac of peak)",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32", "data": "synthetic (seeded; trained weights unavailable)",
        "config": {"workload": f"{w.name}: one MoE layer, hidden {w.hidden}, {w.n_experts} experts, inter {w.inter}, "
                               f"top-{w.top_k} + shared, {w.bits}-bit group-{w.group} experts; a step is {N} "
                               f"sequential single-token calls in one HIP graph",
                   "tokens_per_step": N, "hidden": w.hidden, "n_experts": w.n_experts, "inter": w.inter,
                   "top_k": w.top_k, "bits": w.bits, "group": w.group,
                   "decode_plan": plan_name,
                   "dequant_form": args.dequant if w.fmt == "affine" else "mxfp4: e2m1(q) * 2^(e - 127)",
                   "parallelism": "single GPU"},
        "us_per_token": round(us_tok, 3),
        "expert_GB/s": round(expert_bytes / (us_tok * 1e-6) / 1e9, 1),
        "expert_frac_of_peak": round(expert_bytes / (us_tok * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "stream_read_GB/s": round(read_peak, 1),
        "expert_frac_of_measured_read": round(expert_bytes / (us_tok * 1e-6) / 1e9 / read_peak, 4),
        "cold": cold,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_budget),
    }
    print(json.dumps(result), flush=True)


def _common(args, w, value, unit, ms_per_step, config, extra):
    result = {
        "metric": "MoE-layer decode tokens/s + achieved HBM GB/s on expert weights (frac of peak)",
        "value": round(value, 1), "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32", "data": "synthetic (seeded; trained weights unavailable)", "config": config,
    }
    result.update(extra)
    print(json.dumps(result), flush=True)


def bench_batched(args, w, T):
    """One step = the workload's tokens as consecutive moe_layer_forward calls of T tokens (the last
    call takes the remainder), captured in one HIP graph; each call reads its own tokens."""
    import torch

    import bit_quantized_expert_gemv_amd as bq
    import synth
    from synth.gpu_layers import DeviceLayer

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = DeviceLayer(w, device=dev)
    N = w.tokens
    X = torch.from_numpy(synth.tokens_x(w, 0, N)).to(dev)
    out = torch.empty_like(X)
    nws = bq.moe_workspace_bytes(L.desc, T)
    ws = torch.zeros(nws, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)
    calls = [(c, min(T, N - c)) for c in range(0, N, T)]
    with torch.cuda.stream(stream):
        bq.moe_layer_forward(L.desc, X[:T], X[:T], T, out[:T], None, ws, nws, stream=stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c, n in calls:
            bq.moe_layer_forward(L.desc, X[c:c + n], X[c:c + n], n, out[c:c + n], None, ws, nws, stream=stream)
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(args.steps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    secs = e0.elapsed_time(e1) / 1000.0
    path = "grouped (prefill) path" if T >= bq.MOE_PREFILL_MIN_TOKENS else "per-token (decode) path"
    _common(args, w, args.steps * N / secs, "tokens/s", secs * 1000.0 / args.steps,
            {"workload": f"{w.name} tokens as {len(calls)} calls of {T} tokens in one HIP graph ({path}; hidden "
                         f"{w.hidden}, {w.n_experts} experts, inter {w.inter}, top-{w.top_k} + shared, {w.bits}-bit)",
             "tokens_per_step": N, "tokens_per_call": T, "parallelism": "single GPU"},
            {"us_per_call": round(secs * 1e6 / (args.steps * len(calls)), 2),
             "us_per_token": round(secs * 1e6 / (args.steps * N), 3)})


def bench_prefill(args, w):
    """One step = one 2048-token moe_layer_forward (prefill path) through the 4-bit layer."""
    import numpy as np
    import torch

    import bit_quantized_expert_gemv_amd as bq
    import synth
    from synth.gpu_layers import DeviceLayer

    dev = torch.device("cuda:0")
    L = DeviceLayer(w, device=dev)
    T = w.tokens
    X = torch.from_numpy(synth.tokens_x(w, 0, T)).to(dev)
    out = torch.empty_like(X)
    idx = torch.empty(T, w.top_k, dtype=torch.int32, device=dev)
    n = bq.moe_workspace_bytes(L.desc, T)
    ws = torch.zeros(n, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            bq.moe_layer_forward(L.desc, X, X, T, out, idx, ws, n, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(args.steps):
            bq.moe_layer_forward(L.desc, X, X, T, out, idx, ws, n, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    secs = e0.elapsed_time(e1) / 1000.0
    per = secs / args.steps
    blob = bq.moe_blob_bytes(w.hidden, w.inter, w.bits, w.group)
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=w.n_experts)
    touched = int((counts > 0).sum())
    weight_bytes = touched * blob + blob + w.n_experts * w.hidden * 2 + w.hidden * 2
    flops = 2.0 * (T * w.top_k + T) * 3 * w.hidden * w.inter + 2.0 * T * (w.n_experts + 1) * w.hidden
    gbs = weight_bytes / per / 1e9
    read_peak = stream_read_gbs(torch)
    _common(args, w, T / per, "tokens/s", per * 1000.0,
            {"workload": f"{w.name}: {T}-token prefill through one MoE layer (hidden {w.hidden}, {w.n_experts} experts, "
                         f"inter {w.inter}, top-{w.top_k} + shared, {w.bits}-bit), grouped by expert on MFMA",
             "tokens_per_step": T, "parallelism": "single GPU"},
            {"weight_bytes_per_step": weight_bytes, "weight_GB/s": round(gbs, 1),
             "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "stream_read_GB/s": round(read_peak, 1),
             "frac_of_measured_read": round(gbs / read_peak, 4), "useful_TFLOP/s": round(flops / per / 1e12, 2),
             "tokens_per_expert": {"min": int(counts.min()), "mean": round(float(counts.mean()), 2),
                                   "max": int(counts.max()), "untouched": int((counts == 0).sum()),
                                   "histogram": np.bincount(counts).tolist()}})


def bench_stack(args, w):
    """One step = 128 sequential single-token calls through the 60-layer stack (one HIP graph)."""
    import torch

    import bit_quantized_expert_gemv_amd as bq
    import synth
    from synth.gpu_layers import DeviceLayer

    dev = torch.device("cuda:0")
    layers = [DeviceLayer(w, l, device=dev) for l in range(w.layers)]
    N = w.tokens
    X = torch.from_numpy(synth.tokens_x(w, 0, N)).to(dev)
    out = torch.empty_like(X)
    idx = torch.empty(N, w.layers, w.top_k, dtype=torch.int32, device=dev)
    n = bq.moe_stack_workspace_bytes(layers[0].desc, 1)
    ws = torch.zeros(n, dtype=torch.uint8, device=dev)
    descs = [L.desc for L in layers]
    if args.chain:
        for d in descs:
            d.flags |= bq.MOE_FLAG_DECODE_CHAIN
    plan_name = {bq.MOE_PLAN_PAIR: "two launches per layer", bq.MOE_PLAN_CHAIN: "three-kernel chain per layer"}[
        bq.moe_layer_plan(descs[0], 1)]
    print(f"[bench] plan: {plan_name}", file=sys.stderr, flush=True)
    stream = torch.cuda.Stream(device=dev)
    # one eager call before capture
    with torch.cuda.stream(stream):
        bq.moe_stack_forward(descs, 1e-6, X[0], 1, out[0], idx[0], ws, n, stream=stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for t in range(N):
            bq.moe_stack_forward(descs, 1e-6, X[t], 1, out[t], idx[t], ws, n, stream=stream)
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(args.steps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    secs = e0.elapsed_time(e1) / 1000.0
    blob = bq.moe_blob_bytes(w.hidden, w.inter, w.bits, w.group)
    expert_bytes = w.layers * (w.top_k + 1) * blob
    router_bytes = w.layers * (w.n_experts * w.hidden * 2 + w.hidden * 2)
    us = secs * 1e6 / (args.steps * N)
    _common(args, w, args.steps * N / secs, "tokens/s", secs * 1000.0 / args.steps,
            {"workload": f"{w.name}: {w.layers} MoE layers (hidden {w.hidden}, {w.n_experts} experts, inter {w.inter}, "
                         f"top-{w.top_k} + shared, {w.bits}-bit, all experts resident), {N} sequential single-token "
                         f"calls in one HIP graph, RMS norm between layers", "tokens_per_step": N,
             "decode_plan": plan_name, "parallelism": "single GPU"},
            {"us_per_token": round(us, 2), "expert_GB/s": round(expert_bytes / (us * 1e-6) / 1e9, 1),
             "all_weights_GB/s": round((expert_bytes + router_bytes) / (us * 1e-6) / 1e9, 1),
             "expert_frac_of_peak": round(expert_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
             "resident_bytes": sum(L.weight_bytes() for L in layers)})


if __name__ == "__main__":
    main()
