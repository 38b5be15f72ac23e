#!/usr/bin/env python3
"""Throughput of the fused block-scaled FP8 (W8A16) routed-MoE expert FFN on one MI355X.

A step is one pass of the whole hot path over one batch: softmax top-k routing,
sort by expert, gate/up GEMM + SwiGLU, down GEMM, affinity-weighted fp32 expert
sum.  The default workload is the decode batch (T=64 tokens, hidden 2048,
expert intermediate 512, 256 experts, top-8).  Inputs are resident in HBM before
timing starts; successive steps cycle through several independent weight sets
(like successive MoE layers), so the 256 MB last-level cache cannot serve the
weights from one step to the next.

Prints ONE JSON line.  Only --gpus 1 is supported.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused FP8 MoE tokens/s + %HBM BW (decode T=64) / %MFMA peak (prefill T=8192)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, published
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense fp4 (and fp6) MFMA, published


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def expert_bytes(H, I):
    """FP8 weight bytes + fp32 scale bytes of one expert (gate/up and down)."""
    return 3 * H * I + 4 * (2 * I // 128) * (H // 128) + 4 * (H // 128) * (I // 128)


def kernel_work(name, cfg, n_active, with_shared):
    """(bound, algorithmic work of one launch) of a kernel: HBM bytes that the
    method itself must move through it, or MFMA flops.  Only the method's
    data counts (the active experts' weights and scales, x, out, ids and
    affinities, logits); per-route contribution rows, activations between
    the GEMMs and the sort maps are implementation traffic and do not."""
    T, H, I, k = cfg.T, cfg.H, cfg.I, cfg.k
    R = T * k
    nseg = n_active + (1 if with_shared else 0)
    rows = R + (T if with_shared else 0)
    w13 = 2 * I * H + 4 * (2 * I // 128) * (H // 128)
    w2 = H * I + 4 * (H // 128) * (I // 128)
    if name == "decode_fused_expert":
        return "hbm", nseg * (w13 + w2) + 2 * T * H + 8 * R
    if name == "prefill_gateup_swiglu":
        return "mfma", 2.0 * rows * 2 * I * H
    if name == "prefill_down":
        return "mfma", 2.0 * rows * H * I
    if name == "combine":
        return "hbm", 4 * T * H + 8 * R
    if name == "route_topk_softmax":
        return "hbm", 4 * T * cfg.E + 8 * R
    return None, None


def step_bytes(cfg, n_active, with_shared):
    """Algorithmic bytes of one whole step: active experts' weights, x, out,
    ids + affinities, router logits."""
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    nseg = n_active + (1 if with_shared else 0)
    return nseg * expert_bytes(H, I) + 2 * T * H + 4 * T * H + 8 * T * k + 4 * T * E


def step_flops(cfg, with_shared):
    return 6.0 * cfg.H * cfg.I * (cfg.T * cfg.k + (cfg.T if with_shared else 0))


def cpu_baseline(case, cfg, max_tokens):
    """The oracle (numpy float64) on a bounded sample of the same workload."""
    import numpy as np
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    n = min(cfg.T, max_tokens)
    x = case["x"][:n].float().cpu().numpy()
    logits = case["logits"][:n].cpu().numpy()
    t0 = time.perf_counter()
    ids, aff = oracle.route_softmax_topk(logits, cfg.k)
    oracle.sort_by_expert(ids, cfg.E)
    t1 = time.perf_counter()
    # host copies of the experts the sample uses (not timed)
    uniq = np.unique(ids)
    sel = torch.as_tensor(uniq, dtype=torch.long, device=case["w13"].device)
    w13 = case["w13"].index_select(0, sel).cpu().numpy()
    w13s = case["w13_scale"].index_select(0, sel).cpu().numpy()
    w2 = case["w2"].index_select(0, sel).cpu().numpy()
    w2s = case["w2_scale"].index_select(0, sel).cpu().numpy()
    sh = None
    if case.get("shared") is not None:
        sh = {kk: v.cpu().numpy() for kk, v in case["shared"].items()}
    remap = np.searchsorted(uniq, ids)
    t2 = time.perf_counter()
    oracle.moe_ffn(x, w13, w13s, w2, w2s, remap, aff, sh)
    t3 = time.perf_counter()
    secs = (t1 - t0) + (t3 - t2)
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        affinity = None
    return {"value": round(n / secs, 2), "unit": "tokens/s", "cores": int(threads),
            "cores_note": "threads of the BLAS pool the oracle ran on",
            "host_cpus": os.cpu_count(), "host_cpus_usable": affinity,
            "kind": "oracle",
            "sample": f"{n} of {cfg.T} tokens of {cfg.name}: route + sort + expert FFN in numpy "
                      f"float64 ({len(uniq)} experts dequantised); host copy of weights not timed",
            "seconds": round(secs, 3)}


def measure(cfg, L, steps, warmup, variant, layout, seed, dev):
    """Time `steps` passes of the whole hot path (route + fused sort/FFN/combine),
    cycling over L weight sets; then the same region again with per-kernel
    HIP events on the launch stream."""
    import torch

    from block_scaled_fp8_amd import binding, synth
    log(f"workload {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} "
        f"shared={cfg.shared}, {L} weight sets, variant={variant}, layout={layout}")
    x, logits = synth.make_activations(cfg, seed, dev)
    wsets = [synth.make_weights(cfg, seed + 100 * i, dev) for i in range(L)]
    if layout == "tiled":
        # offline weight preparation, once per weight set (not part of a step)
        run_sets = []
        for w in wsets:
            p = dict(w, w13=binding.pack_w8(w["w13"]), w2=binding.pack_w8(w["w2"]))
            if w["shared"] is not None:
                p["shared"] = dict(w["shared"], w13=binding.pack_w8(w["shared"]["w13"]),
                                   w2=binding.pack_w8(w["shared"]["w2"]))
            run_sets.append(p)
    else:
        run_sets = wsets
    runs = [binding.MoeStep(x, logits, cfg.k, w["w13"], w["w13_scale"], w["w2"], w["w2_scale"],
                            shared=w["shared"], variant=variant, layout=layout)
            for w in run_sets]
    torch.cuda.synchronize()
    ids, _ = binding.route(logits, cfg.k)
    counts = torch.bincount(ids.reshape(-1).long(), minlength=cfg.E)
    n_active = int((counts > 0).sum().item())
    log(f"active experts {n_active}, max routes/expert {int(counts.max().item())}")
    for i in range(warmup):
        runs[i % L]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        runs[i % L]()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    log(f"timed {steps} steps: {ms_per_step * 1e3:.1f} us/step")
    binding.profile_enable(True)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(steps):
        runs[i % L]()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    binding.profile_enable(False)
    prof = binding.profile_collect()
    for n, (c, ms) in sorted(prof.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
        log(f"  {n:24s} {c:6d} x {ms * 1e3:9.2f} us")
    return dict(n_active=n_active, ms_per_step=ms_per_step, ms_profiled=(t3 - t2) * 1e3 / steps,
                prof=prof, x=x, logits=logits, wsets=wsets, L=L, runs=runs)


def profiled_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3
    summary profiles/<kernel>__<workload>.md (FETCH_SIZE and WRITE_SIZE passes,
    scaled by a plain copy's reading), or None when there is no summary or the
    kernel's sources changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"{kernel}__{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    got = {k: v.strip() for k, v in re.findall(r"^(traffic_bytes_per_launch|source_files|source_sha256):(.*)$",
                                                 text, re.M)}
    if len(got) != 3:
        return None
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for f in got["source_files"].split():
        fp = os.path.join(root, f)
        if not os.path.exists(fp):
            return None
        h.update(open(fp, "rb").read())
    if h.hexdigest()[:16] != got["source_sha256"]:
        return None
    return int(got["traffic_bytes_per_launch"])


def roofline_of(prof, cfg, n_active, kernel=None):
    """Roofline object for `kernel` (default: the FFN kernel with the largest
    total time): algorithmic work per launch / its average HIP-event
    duration, against the published peak of its bound."""
    if kernel is None:
        ffn = [n for n in prof if n in ("decode_fused_expert", "prefill_gateup_swiglu",
                                        "prefill_down")]
        kernel = max(ffn, key=lambda n: prof[n][0] * prof[n][1])
    bound, work = kernel_work(kernel, cfg, n_active, cfg.shared)
    us = prof[kernel][1] * 1e3
    if bound == "hbm":
        ach, peak, unit = work / (us * 1e-6) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        ach, peak, unit = work / (us * 1e-6) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
    out = {"bound": bound, "kernel": kernel, "achieved": round(ach, 1), "peak": peak,
           "unit": unit, "frac": round(ach / peak, 4),
           "traffic": profiled_traffic(kernel, cfg.name), "traffic_unit": "bytes per launch",
           "avg_us": round(us, 3)}
    out["bytes_per_launch" if bound == "hbm" else "flops_per_launch"] = work
    return out


def workload_report(cfg, m):
    """Step, per-kernel, roofline and fused-call figures of one workload."""
    flops = step_flops(cfg, cfg.shared)
    sb = step_bytes(cfg, m["n_active"], cfg.shared)
    ms = m["ms_per_step"]
    prof = m["prof"]
    out = {"workload": cfg.name, "T": cfg.T, "hidden": cfg.H, "moe_inter": cfg.I,
           "experts": cfg.E, "top_k": cfg.k, "shared_expert": cfg.shared,
           "active_experts": m["n_active"], "weight_sets": m["L"],
           "ms_per_step": round(ms, 5), "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
           "step": {"algorithmic_bytes": sb, "GB_per_s": round(sb / (ms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(sb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "TFLOP_per_s": round(flops / (ms * 1e-3) / 1e12, 1),
                    "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
           "kernels": {n: {"launches": c, "avg_us": round(t * 1e3, 3)} for n, (c, t) in prof.items()},
           "roofline": roofline_of(prof, cfg, m["n_active"])}
    if "prefill_down" in prof:
        out["contributions"] = ("per-route rows in block floating point (8 values share an "
                                "exponent byte, 16-bit mantissas), summed in fp32")
    return out


def fused_call_graph(cfg, m, samples=7, replays=50):
    """One moe_fused_w8a16 call (sort + expert FFN + expert sum, from ids and
    affinities to out) per weight set, captured once in a HIP graph; the
    median over `samples` of `replays` graph launches, per call."""
    import statistics

    import torch
    runs, L = m["runs"], m["L"]
    for r in runs:
        r()  # route once: the graph replays the fused calls on these ids
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for r in runs:
            r.fused()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in runs:
            r.fused()
    for _ in range(10):
        g.replay()
    torch.cuda.synchronize()
    per_call = []
    for _ in range(samples):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(replays):
            g.replay()
        e.record()
        torch.cuda.synchronize()
        per_call.append(s.elapsed_time(e) * 1e3 / (replays * L))
    us = statistics.median(per_call)
    R = cfg.T * cfg.k
    flops = step_flops(cfg, cfg.shared)
    nbytes = step_bytes(cfg, m["n_active"], cfg.shared) - 4 * cfg.T * cfg.E  # no logits
    del g
    return {"protocol": f"HIP graph of one fused call per weight set ({L} sets), median of "
                        f"{samples} samples x {replays} replays",
            "us_per_call": round(us, 2), "tokens_per_s": round(cfg.T / (us * 1e-6), 1),
            "routes": R, "TFLOP_per_s": round(flops / (us * 1e-6) / 1e12, 1),
            "mfma_frac": round(flops / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "GB_per_s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def vendor_gemm(cfg, dev, warmup=200, reps=50):
    """Same-box context for the MFMA fraction: the rate of torch.matmul (the
    vendor bf16 GEMM library) on the dense product with the gate/up shape of
    the prefill workload, [T*k, H] x [H, 2I], random N(0,1) x N(0,0.02) bf16.
    It does none of the method's work (no fp8 decode, row gather, block scales
    or SwiGLU) and is never part of a step."""
    import torch
    M, K, N = cfg.T * cfg.k, cfg.H, 2 * cfg.I
    g = torch.Generator(device=dev).manual_seed(1)
    a = torch.randn(M, K, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(K, N, device=dev, dtype=torch.bfloat16, generator=g) * 0.02
    for _ in range(warmup):
        c = a @ b
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        c = a @ b
    e.record()
    torch.cuda.synchronize()
    us = s.elapsed_time(e) * 1e3 / reps
    tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"what": "torch.matmul bf16, dense [T*k, H] x [H, 2I]", "M": M, "N": N, "K": K,
            "avg_us": round(us, 2), "TFLOP_per_s": round(tf, 1),
            "frac": round(tf / BF16_PEAK_TFLOPS, 4)}


def route_proj_bench(cfg, dev, sets, seed=0, samples=7, replays=20):
    """moe_route_proj (router projection x * W_g^T, then the router) at the
    workload's T, H, E, k: one call per gate-weight set captured in a HIP graph,
    median per call over `samples` x `replays` graph launches; then per-kernel
    times from the library's own events.  Rotating `sets` distinct gate
    matrices (bf16 [E, H] each) beyond the 256 MB last-level cache makes every
    call read its W_g from HBM."""
    import statistics

    import torch

    from block_scaled_fp8_amd import binding, synth
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    log(f"router projection: T={T} H={H} E={E} k={k}, {sets} gate-weight sets")
    x = synth.make_activations(cfg, seed, dev)[0]
    wgs = [synth.make_gate_weights(E, H, seed + 100 + i, dev) for i in range(sets)]
    ws = torch.empty(max(binding.route_proj_workspace_bytes(T, H, E), 1), dtype=torch.uint8,
                     device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    aff = torch.empty((T, k), dtype=torch.float32, device=dev)
    call = lambda w: binding.route_proj(x, w, k, ws=ws, out=(ids, aff))  # noqa: E731
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for w in wgs:
            call(w)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for w in wgs:
            call(w)
    for _ in range(10):
        g.replay()
    torch.cuda.synchronize()
    per_call = []
    for _ in range(samples):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(replays):
            g.replay()
        e.record()
        torch.cuda.synchronize()
        per_call.append(s.elapsed_time(e) * 1e3 / (replays * sets))
    del g
    us = statistics.median(per_call)
    binding.profile_enable(True)
    for i in range(4 * sets):
        call(wgs[i % sets])
    torch.cuda.synchronize()
    binding.profile_enable(False)
    prof = binding.profile_collect()
    splits = max(1, binding.route_proj_workspace_bytes(T, H, E) // (4 * T * E))
    nbytes = 2 * E * H + 2 * T * H + 8 * T * k      # W_g, x, ids + aff
    flops = 2.0 * T * E * H
    gemm_us = prof["router_gemm"][1] * 1e3
    out = {"workload": cfg.name, "T": T, "hidden": H, "experts": E, "top_k": k,
           "k_slices": int(splits), "gate_weight_sets": sets,
           "protocol": f"HIP graph of one call per gate-weight set, median of {samples} x "
                       f"{replays} replays",
           "us_per_call": round(us, 2),
           "kernels": {n: {"launches": c, "avg_us": round(ms * 1e3, 3)} for n, (c, ms) in prof.items()},
           "hbm": {"bytes": nbytes, "GB_per_s": round(nbytes / (us * 1e-6) / 1e9, 1),
                   "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
           "mfma": {"kernel": "router_gemm", "flops": flops, "avg_us": round(gemm_us, 3),
                    "TFLOP_per_s": round(flops / (gemm_us * 1e-6) / 1e12, 1),
                    "frac": round(flops / (gemm_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}}
    log(f"  {us:.2f} us per call; " + ", ".join(f"{n} {ms * 1e3:.2f} us" for n, (c, ms) in prof.items()))
    del wgs, ws, x
    torch.cuda.empty_cache()
    return out


def router_variants_bench(cfg, dev, seed=0, calls=64, samples=7, replays=20):
    """The router alone on the workload's logits: softmax top-k (moe_route) and
    sigmoid top-k with and without renormalisation (moe_route_sigmoid), each
    as `calls` calls in one HIP graph, median per call.  The logits ([T, E]
    fp32) stay in the caches between calls, so this is the launch and latency
    cost that a step pays, not an HBM rate."""
    import statistics

    import torch

    from block_scaled_fp8_amd import binding, synth
    logits = synth.make_activations(cfg, seed, dev)[1]
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    aff = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    lib = binding.load_library()
    stream = lambda: binding._stream(dev)  # noqa: E731
    fns = {
        "softmax": lambda: lib.moe_route(binding._ptr(logits), cfg.T, cfg.E, cfg.k,
                                         binding._ptr(ids), binding._ptr(aff), None, stream()),
        "sigmoid": lambda: lib.moe_route_sigmoid(binding._ptr(logits), cfg.T, cfg.E, cfg.k, 0,
                                                 2.5, binding._ptr(ids), binding._ptr(aff),
                                                 None, stream()),
        "sigmoid_normalized": lambda: lib.moe_route_sigmoid(binding._ptr(logits), cfg.T, cfg.E,
                                                            cfg.k, 1, 2.5, binding._ptr(ids),
                                                            binding._ptr(aff), None, stream()),
    }
    out = {"workload": cfg.name, "T": cfg.T, "experts": cfg.E, "top_k": cfg.k,
           "protocol": f"HIP graph of {calls} calls, median of {samples} x {replays} replays"}
    for name, fn in fns.items():
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            assert fn() == 0
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                assert fn() == 0
        for _ in range(5):
            g.replay()
        torch.cuda.synchronize()
        per = []
        for _ in range(samples):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(replays):
                g.replay()
            e.record()
            torch.cuda.synchronize()
            per.append(s.elapsed_time(e) * 1e3 / (replays * calls))
        del g
        out[name] = {"us_per_call": round(statistics.median(per), 2)}
    log(f"router variants {cfg.name}: " + ", ".join(f"{n} {out[n]['us_per_call']} us" for n in fns))
    return out


def fused_variant_bench(cfg, dev, L, seed=0, activation="swiglu", variant="auto", samples=7,
                        replays=50, weight_format="e4m3_128"):
    """The fused call (sort + expert FFN + expert sum) for another activation
    (relu^2: non-gated experts, up projection [I, H], relu^2, down) or variant
    (prefill_a8: x quantised to E4M3 per token, gate/up on the FP8 MFMA) on the
    workload's shapes: `L` weight sets, one call per set captured in a HIP
    graph, median per call; then per-kernel times from the library's events.
    Algorithmic work per route (or shared row): 2*H*(n13 + I) flops with
    n13 = 2I (SwiGLU) or I (relu^2); weights (n13 + I)*H bytes (+ scales) per
    active expert."""
    import statistics

    import torch

    from block_scaled_fp8_amd import binding, synth
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    log(f"{activation} experts, variant {variant}, {weight_format} weights, on {cfg.name}: "
        f"{L} weight sets")
    x, logits = synth.make_activations(cfg, seed, dev)
    runs = []
    for i in range(L):
        w = synth.make_weights(cfg, seed + 100 * i, dev, activation=activation,
                               weight_format=weight_format)
        p = binding.pack_weights(w, weight_format)
        del w
        runs.append(binding.MoeStep(x, logits, k, p["w13"], p["w13_scale"], p["w2"],
                                    p["w2_scale"], shared=p["shared"], layout="tiled",
                                    variant=variant, activation=activation,
                                    weight_format=weight_format))
    ids, _ = binding.route(logits, k)
    n_active = int((torch.bincount(ids.reshape(-1).long(), minlength=E) > 0).sum().item())
    for r in runs:
        r()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for r in runs:
            r.fused()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in runs:
            r.fused()
    for _ in range(20):
        g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(samples):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(replays):
            g.replay()
        e.record()
        torch.cuda.synchronize()
        per.append(s.elapsed_time(e) * 1e3 / (replays * L))
    del g
    us = statistics.median(per)
    binding.profile_enable(True)
    for i in range(10 * L):
        runs[i % L].fused()
    torch.cuda.synchronize()
    binding.profile_enable(False)
    prof = binding.profile_collect()
    rows = T * k + (T if cfg.shared else 0)
    nseg = n_active + (1 if cfg.shared else 0)
    n13 = I if activation == "relu2" else 2 * I
    flops = 2.0 * H * (n13 + I) * rows
    if weight_format == "mxfp4":   # half a byte a weight + one scale byte per 32
        wbytes = nseg * ((n13 + I) * H // 2 + (n13 + I) * H // 32)
    else:
        wbytes = nseg * ((n13 + I) * H + 4 * (n13 // 128) * (H // 128) + 4 * (H // 128) * (I // 128))
    nbytes = wbytes + 2 * T * H + 4 * T * H + 8 * T * k
    out = {"workload": cfg.name, "activation": activation, "variant": variant,
           "weights": weight_format, "active_experts": n_active, "weight_sets": L,
           "protocol": f"HIP graph of one fused call per weight set, median of {samples} x "
                       f"{replays} replays",
           "us_per_call": round(us, 2), "tokens_per_s": round(T / (us * 1e-6), 1),
           "GB_per_s": round(nbytes / (us * 1e-6) / 1e9, 1),
           "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "TFLOP_per_s": round(flops / (us * 1e-6) / 1e12, 1),
           "mfma_frac_bf16": round(flops / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "kernels": {n: {"launches": c, "avg_us": round(ms * 1e3, 3)} for n, (c, ms) in prof.items()}}
    mxg = [n for n in ("prefill_gateup_swiglu_mxfp4", "prefill_up_relu2_mxfp4") if n in prof]
    if mxg:
        # the grouped gate/up (or up) GEMM on MXFP4 weights, against the bf16
        # MFMA peak it runs on (the codes are widened to bf16 on chip)
        kus = prof[mxg[0]][1] * 1e3
        kfl = 2.0 * H * n13 * rows
        out["roofline"] = {"bound": "mfma", "kernel": mxg[0], "flops_per_launch": kfl,
                           "avg_us": round(kus, 3),
                           "achieved": round(kfl / (kus * 1e-6) / 1e12, 1),
                           "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(kfl / (kus * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                           "traffic": profiled_traffic(mxg[0], cfg.name),
                           "traffic_unit": "bytes per launch"}
        if "prefill_down_mxfp4" in prof:
            dus = prof["prefill_down_mxfp4"][1] * 1e3
            dfl = 2.0 * H * I * rows
            out["down_gemm"] = {"kernel": "prefill_down_mxfp4", "avg_us": round(dus, 3),
                                "TFLOP_per_s": round(dfl / (dus * 1e-6) / 1e12, 1),
                                "frac": round(dfl / (dus * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    elif "decode_fused_expert_mxfp4" in prof and T * k > 16 * E:
        # prefill sizes: the method is MFMA-bound (its weights once are a
        # small part); the weight-streaming kernel re-reads each expert's
        # weights once per 32-row tile, so it is reported against the bf16
        # MFMA peak it runs on, with the bytes it streams beside it
        kus = prof["decode_fused_expert_mxfp4"][1] * 1e3
        tiles = rows / 32.0 + nseg   # (about: full tiles plus a partial one per segment)
        out["roofline"] = {"bound": "mfma", "kernel": "decode_fused_expert_mxfp4",
                           "flops_per_launch": flops, "avg_us": round(kus, 3),
                           "achieved": round(flops / (kus * 1e-6) / 1e12, 1),
                           "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(flops / (kus * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                           "weight_bytes_streamed_approx": int(tiles * wbytes / nseg),
                           "traffic": profiled_traffic("decode_fused_expert_mxfp4", cfg.name),
                           "traffic_unit": "bytes per launch"}
    elif "decode_fused_expert_mxfp4" in prof:
        # the weight-streaming kernel against HBM: weights + scales, x, ids and aff
        kus = prof["decode_fused_expert_mxfp4"][1] * 1e3
        kb = wbytes + 2 * T * H + 8 * T * k
        out["roofline"] = {"bound": "hbm", "kernel": "decode_fused_expert_mxfp4",
                           "bytes_per_launch": kb, "avg_us": round(kus, 3),
                           "achieved": round(kb / (kus * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s",
                           "frac": round(kb / (kus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                           "traffic": profiled_traffic("decode_fused_expert_mxfp4", cfg.name),
                           "traffic_unit": "bytes per launch"}
    a4 = [n for n in prof if n.endswith(("_a4", "_a4h4")) and not n.startswith("prefill_down")]
    if a4:
        # the E2M1 x E2M1 gate/up (or up) GEMM against the FP4 MFMA peak
        kus = prof[a4[0]][1] * 1e3
        kfl = 2.0 * H * n13 * rows
        out["fp4_gemm"] = {"kernel": a4[0], "avg_us": round(kus, 3), "flops": kfl,
                           "TFLOP_per_s": round(kfl / (kus * 1e-6) / 1e12, 1),
                           "peak": FP4_PEAK_TFLOPS, "frac": round(kfl / (kus * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 4)}
    if "prefill_down_mxfp4_a4" in prof:
        # the E2M1 x E2M1 down GEMM (MXFP4 hidden activation) against the FP4 peak
        dus = prof["prefill_down_mxfp4_a4"][1] * 1e3
        dfl = 2.0 * H * I * rows
        out["fp4_down_gemm"] = {"kernel": "prefill_down_mxfp4_a4", "avg_us": round(dus, 3), "flops": dfl,
                                "TFLOP_per_s": round(dfl / (dus * 1e-6) / 1e12, 1),
                                "peak": FP4_PEAK_TFLOPS,
                                "frac": round(dfl / (dus * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 4)}
    a8 = [n for n in prof if n.endswith("_a8")]
    if a8:
        # the fp8 x fp8 gate/up (or up) GEMM against the FP8 MFMA peak
        kus = prof[a8[0]][1] * 1e3
        kfl = 2.0 * H * n13 * rows
        out["fp8_gemm"] = {"kernel": a8[0], "avg_us": round(kus, 3), "flops": kfl,
                           "TFLOP_per_s": round(kfl / (kus * 1e-6) / 1e12, 1),
                           "peak": FP8_PEAK_TFLOPS, "frac": round(kfl / (kus * 1e-6) / 1e12 / FP8_PEAK_TFLOPS, 4)}
    log(f"  {us:.1f} us per call; " + ", ".join(f"{n} {ms * 1e3:.1f} us" for n, (c, ms) in prof.items()))
    del runs, x, logits
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode64")
    ap.add_argument("--weight-sets", type=int, default=4)
    ap.add_argument("--variant", default="auto", choices=["auto", "decode", "prefill"])
    ap.add_argument("--layout", default="tiled", choices=["rowmajor", "tiled"],
                    help="weight layout; tiled = packed once at load time (offline prep)")
    ap.add_argument("--cpu-tokens", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-workload", default="prefill8k_skew",
                    help="secondary MFMA-bound workload reported in the 'prefill' object ('' = skip)")
    ap.add_argument("--prefill-steps", type=int, default=50)
    ap.add_argument("--prefill-warmup", type=int, default=50,
                    help="untimed prefill steps first: the GPU idles while the prefill inputs "
                         "are generated, and its clock needs some milliseconds of work to settle")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-a8", action="store_true",
                    help="skip the fp8-activation prefill measurement (MOE_VARIANT_PREFILL_A8)")
    ap.add_argument("--no-relu2", action="store_true",
                    help="skip the relu^2-expert measurement (MOE_ACT_RELU2)")
    ap.add_argument("--no-route-proj", action="store_true",
                    help="skip the router measurements (moe_route_proj, router variants)")
    ap.add_argument("--no-vendor-gemm", action="store_true",
                    help="skip timing torch.matmul at the gate/up shape (context only)")
    ap.add_argument("--no-mxfp4", action="store_true",
                    help="skip the MXFP4-weight measurement (moe_fused_mxfp4)")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="skip the decode512 and prefill16k_wide objects")
    ap.add_argument("--no-rowmajor", action="store_true",
                    help="skip the fused call on row-major (unpacked) weights")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, 5 times (PMC byte-counter "
                         "calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    from block_scaled_fp8_amd import binding, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        a = torch.ones(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)
        return
    binding.load_library()
    cfg = synth.CONFIGS[args.workload]
    m = measure(cfg, max(1, args.weight_sets), args.steps, args.warmup, args.variant, args.layout,
                args.seed, dev)
    n_active, ms_per_step, ms_profiled, prof = m["n_active"], m["ms_per_step"], m["ms_profiled"], m["prof"]
    x, logits, wsets, L = m["x"], m["logits"], m["wsets"], m["L"]
    kernels = {n: {"launches": c, "avg_us": round(ms * 1e3, 3)} for n, (c, ms) in prof.items()}

    sb = step_bytes(cfg, n_active, cfg.shared)
    sf = step_flops(cfg, cfg.shared)
    tokens_per_s = cfg.T / (ms_per_step * 1e-3)
    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "hidden": cfg.H, "moe_inter": cfg.I,
                   "experts": cfg.E, "top_k": cfg.k, "shared_expert": cfg.shared,
                   "weights": "E4M3FN, fp32 128x128 block scales", "weight_sets": L,
                   "variant": args.variant, "weight_layout": args.layout,
                   "weight_prep": ("packed once at load time into the tile-coalesced layout "
                                   "(moe_pack_w8), outside the timed steps")
                                  if args.layout == "tiled" else "as given (row-major)",
                   "active_experts": n_active},
        "roofline": roofline_of(prof, cfg, n_active),
        "step": {"algorithmic_bytes": sb, "GB_per_s": round(sb / (ms_per_step * 1e-3) / 1e9, 1),
                 "hbm_frac": round(sb / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "TFLOP_per_s": round(sf / (ms_per_step * 1e-3) / 1e12, 2),
                 "ms_per_step_profiled": round(ms_profiled, 5)},
        "kernels": kernels,
    }
    log("fused call in a HIP graph ...")
    result["fused_call"] = fused_call_graph(cfg, m)
    if args.layout == "tiled" and not args.no_rowmajor:
        log("fused call on the row-major weights (no packing) ...")
        rm = dict(m, runs=[binding.MoeStep(x, logits, cfg.k, w["w13"], w["w13_scale"], w["w2"],
                                           w["w2_scale"], shared=w["shared"], variant=args.variant,
                                           layout="rowmajor") for w in wsets])
        result["fused_call_rowmajor"] = fused_call_graph(cfg, rm)
        del rm
    case0 = dict(x=x, logits=logits, **wsets[0]) if not args.no_cpu_baseline else None
    del m, wsets
    torch.cuda.empty_cache()
    # the other workloads: decode at 512 tokens (HBM-bound) and the two
    # prefill workloads (MFMA-bound), each with its own step, kernels,
    # roofline and graph-timed fused call
    extra = [(args.prefill_workload, "prefill", 2, args.prefill_steps)]
    if not args.no_extra_workloads:
        extra += [("decode512", "decode512", max(1, args.weight_sets), args.steps),
                  ("prefill16k_wide", "prefill16k_wide", 2, max(5, args.prefill_steps // 5))]
    for wname, key, nsets, nsteps in extra:
        if not wname:
            continue
        wcfg = synth.CONFIGS[wname]
        wm = measure(wcfg, nsets, nsteps, args.prefill_warmup if wcfg.T > 4096 else args.warmup,
                     "auto", args.layout, args.seed, dev)
        result[key] = workload_report(wcfg, wm)
        log(f"{wname} fused call in a HIP graph ...")
        result[key]["fused_call"] = fused_call_graph(wcfg, wm, replays=50 if wcfg.T <= 8192 else 10)
        del wm
        torch.cuda.empty_cache()
        if key == "prefill" and not args.no_vendor_gemm:
            log("vendor bf16 GEMM at the gate/up shape (context) ...")
            result[key]["vendor_bf16_gemm"] = vendor_gemm(wcfg, dev)
    if not args.no_relu2:
        result["relu2"] = [fused_variant_bench(cfg, dev, max(1, args.weight_sets), args.seed,
                                               activation="relu2")]
        if args.prefill_workload:
            result["relu2"].append(fused_variant_bench(synth.CONFIGS[args.prefill_workload], dev,
                                                       2, args.seed, activation="relu2"))
    if not args.no_mxfp4:
        # MXFP4 weights (E2M1 codes, E8M0 per 32): the weight stream halves
        result["mxfp4"] = [fused_variant_bench(cfg, dev, max(1, args.weight_sets), args.seed,
                                               weight_format="mxfp4")]
        if not args.no_extra_workloads:
            result["mxfp4"].append(fused_variant_bench(synth.CONFIGS["decode512"], dev,
                                                       max(1, args.weight_sets), args.seed,
                                                       weight_format="mxfp4"))
        if args.prefill_workload:
            result["mxfp4"].append(fused_variant_bench(synth.CONFIGS[args.prefill_workload], dev,
                                                       2, args.seed, weight_format="mxfp4"))
        if not args.no_extra_workloads and args.prefill_workload != "prefill16k_wide":
            # the wide geometry of the MXFP4 prefill figures on the pages
            result["mxfp4"].append(fused_variant_bench(synth.CONFIGS["prefill16k_wide"], dev, 1,
                                                       args.seed, weight_format="mxfp4"))
        if args.prefill_workload and not args.no_a8:
            # x quantised to E4M3 per token (gate/up as E4M3 x E2M1 on the FP8
            # MFMA) or to MXFP4 (E2M1 x E2M1), and both GEMMs on MXFP4
            # operands (the hidden activation quantised too)
            for wname in dict.fromkeys([args.prefill_workload] +
                                       ([] if args.no_extra_workloads else ["prefill16k_wide"])):
                for v in ("prefill_a8", "prefill_a4", "prefill_fp4"):
                    result["mxfp4"].append(fused_variant_bench(synth.CONFIGS[wname], dev,
                                                               2 if wname == "prefill8k_skew" else 1,
                                                               args.seed, variant=v,
                                                               weight_format="mxfp4"))
    if args.prefill_workload and not args.no_a8:
        result["prefill_a8"] = fused_variant_bench(synth.CONFIGS[args.prefill_workload], dev, 2,
                                                   args.seed, variant="prefill_a8")
    if not args.no_route_proj:
        result["router_variants"] = [router_variants_bench(cfg, dev, args.seed)]
        if args.prefill_workload:
            result["router_variants"].append(
                router_variants_bench(synth.CONFIGS[args.prefill_workload], dev, args.seed))
        result["route_proj"] = [route_proj_bench(cfg, dev, 320, args.seed)]
        if args.prefill_workload:
            result["route_proj"].append(
                route_proj_bench(synth.CONFIGS[args.prefill_workload], dev, 4, args.seed))
    if case0 is not None:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(case0, cfg, args.cpu_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
