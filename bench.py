#!/usr/bin/env python3
"""Benchmark of the W4A16 MoE expert layer on one MI355X.

Headline workload: the Qwen3-30B-A3B MoE layer (128 experts, top-8, hidden
2048, expert intermediate 768, int4 group-128 weights, bf16 activations) in
decode at 256 tokens. One step = one full layer forward (route, permute,
GEMM1 + SwiGLU, GEMM2, finalize) on one batch. Steps rotate over layer
replicas with distinct weights and logits, so the 256 MB Infinity Cache
cannot serve the weights from one step to the next. Replica 0 is the seeded
workload of the parity tests; the others are drawn on the GPU. All inputs are
resident in HBM before timing starts; the steps are replayed from HIP graphs.

`value` times exactly --steps steps (after --warmup untimed ones). Every
workload is also measured the way the measurement plan asks: one HIP graph of
several layer calls with distinct weights and batches, 10 warm-up replays,
then 50 replays each timed with HIP events on the replaying stream; the
median per call is reported:
  - the decode sweep at 1 / 16 / 64 / 256 tokens (weight HBM GB/s, % of peak),
  - the 2048-token Zipf prefill (TFLOP/s, % of the bf16 MFMA peak),
  - the expert-parallel shard (32 of 256 experts, H 7168, I 2048) at
    1 / 16 / 64 / 256 tokens,
  - the layer with one shared expert, the finalize stream, the dense GEMM.
Prints ONE JSON line with the headline, the roofline of the dominant kernel
(GEMM1, HBM-bound on weight bytes) and of GEMM2, and the CPU oracle timed on
the host (per workload) as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; weight HBM GB/s % peak (decode), MFMA % (prefill)"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["w4a16_grouped_gemm_amd/csrc/gemm_w4a16.hip", "w4a16_grouped_gemm_amd/csrc/gemm_core.hpp",
                  "w4a16_grouped_gemm_amd/csrc/common.hpp"]
WARM_REPLAYS = 10
TIMED_REPLAYS = 50
CACHE_BYTES = 256e6          # Infinity Cache (MALL); the L2s (8 x 4 MB) are smaller


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def weight_bytes_per_expert(H: int, I: int):
    """int4 codes + bf16 scales of one expert: (w13, w2)."""
    w13 = 2 * I * H // 2 + 2 * I * (H // 128) * 2
    w2 = H * I // 2 + H * (I // 128) * 2
    return w13, w2


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

def capture(torch, fns):
    """One HIP graph holding one call of each function in `fns`."""
    for f in fns:                   # eager pass (loads kernels, checks arguments)
        f()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for f in fns:
                f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return graph


def replay_stats(torch, graph, calls, warm=WARM_REPLAYS, reps=TIMED_REPLAYS):
    """`warm` untimed replays, then `reps` replays each bracketed by HIP events
    on the replaying stream; microseconds per call (graph time / calls)."""
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        graph.replay()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        graph.replay()
        ev[i + 1].record(stream)
    ev[-1].synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) * 1e3 / calls for i in range(reps)]
    return {"median_us": round(statistics.median(per), 3), "mean_us": round(sum(per) / reps, 3),
            "min_us": round(min(per), 3), "max_us": round(max(per), 3), "replays": reps,
            "warmup_replays": warm, "calls_per_replay": calls}


# ---------------------------------------------------------------------------
# inputs
# ---------------------------------------------------------------------------

def make_weights(wl, L, torch, ops, layout, seed_base):
    """L weight replicas: replica 0 the seeded numpy workload, the rest drawn
    on the GPU with the same distributions. Codes packed when tiled."""
    from w4a16_grouped_gemm_amd.inputs import make_layer_inputs
    dev = torch.device("cuda")
    H, I, El = wl.hidden, wl.inter, wl.num_local_experts
    inp = make_layer_inputs(wl, 1)

    def d(a, dtype=None):
        t = torch.from_numpy(a).to(dev)
        return t.view(dtype) if dtype is not None else t

    reps = [dict(w13=d(inp.w13_q), s13=d(inp.s13, torch.bfloat16), w2=d(inp.w2_q), s2=d(inp.s2, torch.bfloat16))]
    g = torch.Generator(device=dev)
    for i in range(1, L):
        g.manual_seed(seed_base * 1000 + i)
        reps.append(dict(
            w13=torch.randint(0, 256, (El, 2 * I, H // 2), generator=g, device=dev, dtype=torch.uint8),
            s13=torch.empty((El, 2 * I, H // 128), device=dev).uniform_(0.005, 0.02, generator=g).to(torch.bfloat16),
            w2=torch.randint(0, 256, (El, H, I // 2), generator=g, device=dev, dtype=torch.uint8),
            s2=torch.empty((El, H, I // 128), device=dev).uniform_(0.005, 0.02, generator=g).to(torch.bfloat16)))
    if layout == ops.WEIGHTS_TILED:
        for r in reps:
            r["w13"] = ops.pack_weights(ops.W13_SWIGLU, r["w13"])
            r["w2"] = ops.pack_weights(ops.W2, r["w2"])
    return reps


def make_batches(wl, T, n, torch, seed):
    """n batches (x, logits): batch 0 the seeded numpy workload of T tokens,
    the rest drawn on the GPU (Zipf routing redrawn on the host per batch)."""
    import numpy as np
    from w4a16_grouped_gemm_amd.inputs import make_layer_inputs, zipf_logits
    dev = torch.device("cuda")
    inp = make_layer_inputs(wl, T, weights=False)
    out = [dict(x=torch.from_numpy(inp.x).to(dev).view(torch.bfloat16), logits=torch.from_numpy(inp.logits).to(dev))]
    g = torch.Generator(device=dev)
    rng = np.random.Generator(np.random.PCG64(seed))
    for i in range(1, n):
        g.manual_seed(seed * 1000 + i)
        x = torch.randn((T, wl.hidden), generator=g, device=dev).to(torch.bfloat16)
        if wl.routing == "zipf":
            lg = torch.from_numpy(zipf_logits(rng, T, wl.num_experts)).to(dev)
        else:
            lg = torch.randn((T, wl.num_experts), generator=g, device=dev)
        out.append(dict(x=x, logits=lg))
    return out


def n_calls_for(active_bytes, minimum=8):
    """Layer calls per graph: at least `minimum`, and enough that the weights
    one replay streams are several times the Infinity Cache."""
    n = minimum
    while n < 64 and n * active_bytes < 3 * CACHE_BYTES:
        n *= 2
    return n


def routing_stats(ops, wl, batches, torch):
    """Per batch: active local experts and local rows (from the GPU routing)."""
    res = []
    for b in batches:
        ids, _ = ops.route(b["logits"], wl.top_k)
        counts, offsets, *_ = ops.permute(ids, wl.num_local_experts, num_experts=wl.num_experts,
                                          expert_begin=wl.expert_begin)
        res.append((counts, offsets))
    torch.cuda.synchronize()
    return [dict(active=int((c > 0).sum().item()), rows=int(o[-1].item())) for c, o in res]


def layer_fns(ops, wl, weights, batches, calls, torch, layout, shared=None):
    """`calls` forward calls: call i uses weight replica i % L and batch i % B."""
    T = batches[0]["x"].shape[0]
    shape = ops.make_shape(T, wl.hidden, wl.inter, wl.num_experts, wl.num_local_experts, wl.top_k,
                           wl.expert_begin, weight_layout=layout)
    if shared is None:
        wsz = ops.workspace_size(shape)
    else:
        import ctypes
        wsz = int(ops.load_library().moe_w4a16_workspace_size_shared(ctypes.byref(shape), shared[0][0].shape[0]))
    ws = torch.empty(max(wsz, 256), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((T, wl.hidden), dtype=torch.bfloat16, device="cuda") for _ in range(calls)]

    def fwd(i):
        w, b = weights[i % len(weights)], batches[i % len(batches)]
        ops.moe_w4a16_forward(b["x"], b["logits"], w["w13"], w["s13"], w["w2"], w["s2"], wl.top_k, out=outs[i],
                              expert_begin=wl.expert_begin, workspace=ws, weight_layout=layout,
                              shared=None if shared is None else shared[i % len(shared)])
    return [lambda i=i: fwd(i) for i in range(calls)]


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def decode_point(ops, wl, weights, T, torch, layout, seed, shared=None):
    """One decode point: median per layer call, weight bytes of the active
    experts (int4 + bf16 scales) per call, and the fraction of HBM peak."""
    w13b, w2b = weight_bytes_per_expert(wl.hidden, wl.inter)
    probe = make_batches(wl, T, 4, torch, seed)
    act0 = sum(s["active"] for s in routing_stats(ops, wl, probe, torch)) / len(probe)
    calls = n_calls_for(act0 * (w13b + w2b))
    batches = make_batches(wl, T, calls, torch, seed)
    st = routing_stats(ops, wl, batches, torch)
    act = sum(s["active"] for s in st) / calls
    rows = sum(s["rows"] for s in st) / calls
    nsh = 0 if shared is None else shared[0][0].shape[0]
    g = capture(torch, layer_fns(ops, wl, weights, batches, calls, torch, layout, shared))
    r = replay_stats(torch, g, calls)
    del g
    us = r["median_us"]
    streamed = (act + nsh) * (w13b + w2b)
    gbps = streamed / (us * 1e-6) / 1e9
    rec = {"tokens": T, "us_per_layer": us, "tokens_per_s": round(T / (us * 1e-6), 1),
           "active_experts": act, "local_rows": rows, "weight_bytes": round(streamed),
           "weight_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
           "layer_calls_per_graph": calls, "weight_replicas": len(weights), "timing": r}
    if nsh:
        rec["shared_experts"] = nsh
    return rec


def prefill_point(ops, wl, weights, torch, layout, T=2048):
    """2048 tokens with Zipf(1.1) expert popularity: algorithmic flops
    6 * I * H per routed row against the dense bf16 MFMA peak."""
    batches = make_batches(wl, T, 8, torch, seed=2048)
    g = capture(torch, layer_fns(ops, wl, weights, batches, 8, torch, layout))
    r = replay_stats(torch, g, 8)
    del g
    us = r["median_us"]
    flops = 6.0 * wl.inter * wl.hidden * T * wl.top_k
    tf = flops / (us * 1e-6) / 1e12
    return {"tokens": T, "routing": "zipf(1.1)", "us_per_layer": us, "tokens_per_s": round(T / (us * 1e-6), 1),
            "tflops": round(tf, 1), "mfma_frac": round(tf / MFMA_PEAK_TFLOPS, 4), "flops": flops, "timing": r}


def finalize_point(ops, torch, T=4096, k=8, H=4096, E=128):
    """The finalize on its stress shape: fp32 y [T*k, H] (512 MiB; four
    buffers rotate so the Infinity Cache cannot hold them), bf16 out [T, H]."""
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    logits = torch.randn((T, E), generator=g, device=dev)
    ids, w = ops.route(logits, k)
    _, _, _, inv, _ = ops.permute(ids, E)
    ys = [torch.randn((T * k, H), generator=g, device=dev) for _ in range(4)]
    outs = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(4)]
    gr = capture(torch, [lambda i=i: ops.finalize(ys[i], w, inv, out=outs[i]) for i in range(4)])
    r = replay_stats(torch, gr, 4)
    del gr, ys, outs
    torch.cuda.empty_cache()
    nbytes = T * k * H * 4 + T * k * 8 + T * H * 2
    gbps = nbytes / (r["median_us"] * 1e-6) / 1e9
    return {"shape": f"T={T} k={k} H={H}, fp32 y, bf16 out", "us": r["median_us"], "bytes": nbytes,
            "GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4), "timing": r}


def dense_points(ops, torch, layout, Ms=(1, 16, 256), N=14336, K=4096, L=16):
    """Dense W4A16 GEMM c[M, N] = a[M, K] . W^T over L weight replicas
    (L * 30 MB, more than the Infinity Cache holds)."""
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(99)
    ws = []
    for _ in range(L):
        wq = torch.randint(0, 256, (N, K // 2), generator=g, device=dev, dtype=torch.uint8)
        if layout == ops.WEIGHTS_TILED:
            wq = ops.pack_dense_weights(wq)
        sc = torch.empty((N, K // 128), device=dev).uniform_(0.005, 0.02, generator=g).to(torch.bfloat16)
        ws.append((wq, sc))
    wbytes = N * K // 2 + N * (K // 128) * 2
    res = []
    for M in Ms:
        a = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
        outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(L)]
        gr = capture(torch, [lambda i=i: ops.dense_gemm_w4a16(a, ws[i][0], ws[i][1], out=outs[i],
                                                             weight_layout=layout) for i in range(L)])
        r = replay_stats(torch, gr, L)
        del gr
        sec = r["median_us"] * 1e-6
        res.append({"M": M, "N": N, "K": K, "us": r["median_us"],
                    "weight_GBps": round(wbytes / sec / 1e9, 1), "hbm_frac": round(wbytes / sec / 1e9 / HBM_PEAK_GBPS, 4),
                    "tflops": round(2.0 * M * N * K / sec / 1e12, 2)})
    del ws
    torch.cuda.empty_cache()
    return res


def shared_weights(ops, wl, L, torch, layout, S=1):
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    H, I = wl.hidden, wl.inter
    out = []
    for i in range(L):
        g.manual_seed(31000 + i)
        w13 = torch.randint(0, 256, (S, 2 * I, H // 2), generator=g, device=dev, dtype=torch.uint8)
        w2 = torch.randint(0, 256, (S, H, I // 2), generator=g, device=dev, dtype=torch.uint8)
        if layout == ops.WEIGHTS_TILED:
            w13, w2 = ops.pack_weights(ops.W13_SWIGLU, w13), ops.pack_weights(ops.W2, w2)
        s13 = torch.empty((S, 2 * I, H // 128), device=dev).uniform_(0.005, 0.02, generator=g).to(torch.bfloat16)
        s2 = torch.empty((S, H, I // 128), device=dev).uniform_(0.005, 0.02, generator=g).to(torch.bfloat16)
        out.append((w13, s13, w2, s2))
    return out


# ---------------------------------------------------------------------------
# the W4A4 (MXFP4) variant
# ---------------------------------------------------------------------------

FP4_MFMA_PEAK_TFLOPS = 10100.0


def mx_weight_bytes_per_expert(H: int, I: int):
    """E2M1 codes + E8M0 scales (one byte per 32 along K) of one expert: (w13, w2)."""
    return 2 * I * H // 2 + 2 * I * (H // 32), H * I // 2 + H * (I // 32)


def make_mx_weights(ops, wl, L, torch, seed_base):
    """L replicas of the layer's MXFP4 weights, codes in the tiled layout
    (moe_mxfp4_pack_weights), so that a wave's code load covers whole lines."""
    from w4a16_grouped_gemm_amd.inputs import MX_SCALE_RANGE, make_mxfp4_layer_inputs
    dev = torch.device("cuda")
    H, I, El = wl.hidden, wl.inter, wl.num_local_experts
    inp = make_mxfp4_layer_inputs(wl, 1)
    reps = [dict(w13=torch.from_numpy(inp.w13_q).to(dev), s13=torch.from_numpy(inp.w13_s).to(dev),
                 w2=torch.from_numpy(inp.w2_q).to(dev), s2=torch.from_numpy(inp.w2_s).to(dev))]
    g = torch.Generator(device=dev)
    lo, hi = MX_SCALE_RANGE
    for i in range(1, L):
        g.manual_seed(seed_base * 1000 + i)
        reps.append(dict(
            w13=torch.randint(0, 256, (El, 2 * I, H // 2), generator=g, device=dev, dtype=torch.uint8),
            s13=torch.randint(lo, hi + 1, (El, 2 * I, H // 32), generator=g, device=dev, dtype=torch.uint8),
            w2=torch.randint(0, 256, (El, H, I // 2), generator=g, device=dev, dtype=torch.uint8),
            s2=torch.randint(lo, hi + 1, (El, H, I // 32), generator=g, device=dev, dtype=torch.uint8)))
    for r in reps:
        r["w13"] = ops.mxfp4_pack_weights(ops.W13_SWIGLU, r["w13"])
        r["w2"] = ops.mxfp4_pack_weights(ops.W2, r["w2"])
    torch.cuda.synchronize()
    return reps


def w4a4_point(ops, wl, weights, T, torch, seed, prefill=False):
    """The W4A4 layer at T tokens: median per call; weight bytes of the
    active experts (decode) or flops against the dense FP4 MFMA peak (prefill)."""
    import ctypes
    probe = make_batches(wl, T, 4, torch, seed)
    w13b, w2b = mx_weight_bytes_per_expert(wl.hidden, wl.inter)
    act0 = sum(s["active"] for s in routing_stats(ops, wl, probe, torch)) / len(probe)
    calls = 8 if prefill else n_calls_for(act0 * (w13b + w2b))
    batches = make_batches(wl, T, calls, torch, seed)
    st = routing_stats(ops, wl, batches, torch)
    act = sum(s["active"] for s in st) / calls
    shape = ops.make_shape(T, wl.hidden, wl.inter, wl.num_experts, wl.num_local_experts, wl.top_k,
                           wl.expert_begin, group_size=32)
    ws = torch.empty(max(int(ops.load_library().moe_w4a4_workspace_size(ctypes.byref(shape))), 256),
                     dtype=torch.uint8, device="cuda")
    outs = [torch.empty((T, wl.hidden), dtype=torch.bfloat16, device="cuda") for _ in range(calls)]

    def fwd(i):
        w, b = weights[i % len(weights)], batches[i]
        ops.moe_w4a4_forward(b["x"], b["logits"], w["w13"], w["s13"], w["w2"], w["s2"], wl.top_k, out=outs[i],
                             expert_begin=wl.expert_begin, workspace=ws, weight_layout=ops.WEIGHTS_TILED)
    g = capture(torch, [lambda i=i: fwd(i) for i in range(calls)])
    r = replay_stats(torch, g, calls)
    del g
    us = r["median_us"]
    rec = {"tokens": T, "us_per_layer": us, "tokens_per_s": round(T / (us * 1e-6), 1), "active_experts": act,
           "timing": r}
    if prefill:
        flops = 6.0 * wl.inter * wl.hidden * T * wl.top_k
        tf = flops / (us * 1e-6) / 1e12
        rec.update(routing="zipf(1.1)", tflops=round(tf, 1), fp4_mfma_frac=round(tf / FP4_MFMA_PEAK_TFLOPS, 4),
                   bf16_mfma_frac=round(tf / MFMA_PEAK_TFLOPS, 4))
    else:
        gbps = act * (w13b + w2b) / (us * 1e-6) / 1e9
        rec.update(weight_bytes=round(act * (w13b + w2b)), weight_GBps=round(gbps, 1),
                   hbm_frac=round(gbps / HBM_PEAK_GBPS, 4))
    return rec


# ---------------------------------------------------------------------------
# the GEMMs alone (roofline of the dominant kernel)
# ---------------------------------------------------------------------------

def gemm_alone(ops, wl, weights, batches, torch, layout, kind):
    """Average duration of one grouped-GEMM launch (GEMM1 with SwiGLU, or
    GEMM2), HIP events on the replaying stream over the timed replays, and
    its algorithmic bytes: active experts' weights and scales, the activation
    rows read, the output rows written, offsets and row index."""
    T = batches[0]["x"].shape[0]
    k, H, I = wl.top_k, wl.hidden, wl.inter
    calls = len(batches)
    pre = []
    for i, b in enumerate(batches):
        ids, _ = ops.route(b["logits"], k)
        counts, offsets, perm, _, _ = ops.permute(ids, wl.num_local_experts, num_experts=wl.num_experts,
                                                  expert_begin=wl.expert_begin)
        pre.append((counts, offsets, perm))
    hs = [torch.randn((T * k, I), device="cuda").to(torch.bfloat16) * 0.05 for _ in range(calls)]
    outs = [torch.empty((T * k, I if kind == ops.W13_SWIGLU else H), dtype=torch.bfloat16, device="cuda")
            for _ in range(calls)]

    def call(i):
        w, b = weights[i % len(weights)], batches[i]
        _, offsets, perm = pre[i]
        if kind == ops.W13_SWIGLU:
            ops.grouped_gemm_w4a16(ops.W13_SWIGLU, b["x"], offsets, w["w13"], w["s13"], num_tokens=T, top_k=k,
                                   a_row_index=perm, num_experts=wl.num_experts, out=outs[i], weight_layout=layout)
        else:
            ops.grouped_gemm_w4a16(ops.W2, hs[i], offsets, w["w2"], w["s2"], num_tokens=T, top_k=k,
                                   num_experts=wl.num_experts, out=outs[i], weight_layout=layout)

    g = capture(torch, [lambda i=i: call(i) for i in range(calls)])
    r = replay_stats(torch, g, calls)
    del g
    torch.cuda.synchronize()
    w13b, w2b = weight_bytes_per_expert(H, I)
    nb = 0.0
    for counts, offsets, _ in pre:
        act = int((counts > 0).sum().item())
        rows = int(offsets[-1].item())
        if kind == ops.W13_SWIGLU:
            nb += act * w13b + T * H * 2 + rows * I * 2 + (wl.num_local_experts + 1) * 4 + rows * 4
        else:
            nb += act * w2b + rows * I * 2 + rows * H * 2 + (wl.num_local_experts + 1) * 4
    nb /= calls
    return r["mean_us"], nb, r


def load_traffic(name, expected_hash):
    """HBM bytes per dispatch from a committed counter summary, scaled by the
    same counters read on a device copy of known size; None once the kernel
    source has changed since the counters were taken."""
    path = os.path.join(PROFILE_DIR, name)
    if not os.path.exists(path):
        return None, f"no counter summary {name}"
    with open(path) as f:
        c = json.load(f)
    if c.get("kernel_source_sha256") != expected_hash:
        return None, "kernel changed since the counters were taken"
    ff = c["copy_bytes"] / (c["copy_fetch_kib"] * 1024.0)
    fw = c["copy_bytes"] / (c["copy_write_kib"] * 1024.0)
    return (c["fetch_kib_per_dispatch"] * ff + c["write_kib_per_dispatch"] * fw) * 1024.0, \
        f"FETCH_SIZE x {ff:.4f} + WRITE_SIZE x {fw:.4f} (copy-kernel scale), {name}"


# ---------------------------------------------------------------------------
# the CPU oracle on the host (reported baseline)
# ---------------------------------------------------------------------------

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _time_runs(fn, max_runs=3, long_s=0.5):
    """Median wall time of up to `max_runs` runs; a single run once one takes
    longer than long_s (keeps the leg near 30 s of host time)."""
    ts = []
    for _ in range(max_runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
        if ts[-1] > long_s:
            break
    return statistics.median(ts), len(ts)


def cpu_baseline():
    """The oracle (fp64 C, OpenMP) on every workload, on the host cores.
    Each workload's weights are drawn once (its largest token count) and
    reused with the seeded activations and logits of the other token counts;
    long layers run on a seeded sample of tokens (tokens are independent, so
    a sample's tokens/s is the layer's); the finalize stress on 512 of its
    4096 tokens. Headline: the 256-token decode layer."""
    import dataclasses
    import numpy as np
    import oracle
    from w4a16_grouped_gemm_amd.inputs import make_finalize_stress, make_layer_inputs
    oracle.build(force=False)
    cores = len(os.sched_getaffinity(0))
    env_threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(cores, env_threads) if env_threads > 0 else cores
    per = []

    def layer_case(inp, n_sample=None):
        w, T = inp.workload, inp.tokens
        sel, n = None, T
        if n_sample is not None and n_sample < T:
            sel = np.zeros(T, np.uint8)
            sel[np.unique(np.linspace(0, T - 1, n_sample).astype(int))] = 1
            n = int(sel.sum())
        sec, runs = _time_runs(lambda: oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2,
                                                    top_k=w.top_k, expert_begin=w.expert_begin, tok_sel=sel))
        per.append({"workload": w.name, "tokens": T, "tokens_computed": n, "seconds": round(sec, 4), "runs": runs,
                    "tokens_per_s": round(n / sec, 2), "threads": oracle.get_threads()})
        return per[-1]

    def with_batch(base, wl, T):
        b = make_layer_inputs(wl, T, weights=False)
        return dataclasses.replace(base, workload=b.workload, tokens=T, x=b.x, logits=b.logits)

    tiny = make_layer_inputs("tiny", 16)
    oracle.set_threads(1)
    c0_single = layer_case(tiny)
    oracle.set_threads(threads)
    layer_case(tiny)
    q = make_layer_inputs("qwen3_decode", 256)
    for T in (1, 16, 64):
        layer_case(with_batch(q, "qwen3_decode", T))
    head = layer_case(q)
    layer_case(with_batch(q, "qwen3_prefill", 2048), n_sample=128)
    ep = make_layer_inputs("ep_shard_decode", 16)
    for T in (1, 16, 64, 256):
        layer_case(ep if T == 16 else with_batch(ep, "ep_shard_decode", T), n_sample=16)
    del q, ep
    fs = make_finalize_stress(tokens=512)
    ids, w = oracle.route(fs.logits, 8)
    w = np.where(fs.zero_mask, np.float32(0.0), w).astype(np.float32)
    _, _, _, inv = oracle.permute(ids, 128, 0)
    sec, runs = _time_runs(lambda: oracle.finalize(fs.y, w, inv, out_f32=True))
    nbytes = fs.y.nbytes + 512 * 8 * 8 + 512 * 4096 * 4
    per.append({"workload": "finalize_stress", "tokens": 512, "seconds": round(sec, 4), "runs": runs,
                "tokens_per_s": round(512 / sec, 1), "GBps": round(nbytes / sec / 1e9, 3),
                "threads": oracle.get_threads()})
    return {"value": head["tokens_per_s"], "unit": "tokens/s", "cores": oracle.get_threads(), "kind": "oracle",
            "sample": "the oracle's full 256-token decode layer (fp64 C, OpenMP) on the seeded batch, "
                      f"{head['runs']} run(s), median",
            "cpu_model": cpu_model(), "host_cpus": cores,
            "c0_single_thread": {"seconds": c0_single["seconds"], "tokens_per_s": c0_single["tokens_per_s"]},
            "per_workload": per}


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--tokens", type=int, default=256)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", help="comma list of extra workloads to time "
                    "(decode,prefill,ep,shared,finalize,dense,w4a4); default all")
    ap.add_argument("--decode-tokens", default="1,16,64,256",
                    help="token counts of the decode sweep (comma list)")
    ap.add_argument("--weights", choices=["tiled", "plain"], default="tiled",
                    help="int4 code layout the layer reads (tiled: packed once before timing)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 1 GiB device copy (scale reference for the HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path here (an expert-parallel "
              "layer would shard its experts across GPUs, each running this layer on its share)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from w4a16_grouped_gemm_amd import ops
    from w4a16_grouped_gemm_amd.inputs import WORKLOADS

    ops.load_library()
    only = set(filter(None, args.only.split(","))) or {"decode", "prefill", "ep", "shared", "finalize", "dense",
                                                        "w4a4"}
    if args.no_sweep:
        only = set()
    layout = ops.WEIGHTS_TILED if args.weights == "tiled" else ops.WEIGHTS_PLAIN
    wl = WORKLOADS["qwen3_decode"]
    T, L = args.tokens, args.replicas
    log(f"generating {L} weight replicas of {wl.name}")
    weights = make_weights(wl, L, torch, ops, layout, seed_base=7)
    batches = make_batches(wl, T, L, torch, seed=T)
    w13b, w2b = weight_bytes_per_expert(wl.hidden, wl.inter)

    # ---- the headline: exactly --steps steps after --warmup, one step = one layer call
    # (replica i % L); the warm-up steps and the timed steps are one HIP graph
    # each, so a step pays no launch of its own
    log(f"timing {args.steps} steps at T={T}")
    fns = layer_fns(ops, wl, weights, batches, L, torch, layout)
    graph_warm = capture(torch, [fns[i % L] for i in range(args.warmup)]) if args.warmup > 0 else None
    graph_steps = capture(torch, [fns[i % L] for i in range(args.steps)])
    if graph_warm is not None:
        graph_warm.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph_steps.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    del graph_warm, graph_steps
    ms = dt / args.steps * 1e3
    tok_s = T * args.steps / dt
    st = routing_stats(ops, wl, batches, torch)
    mean_active = sum(s["active"] for s in st) / L
    layer_gbps = mean_active * (w13b + w2b) / (ms * 1e-3) / 1e9

    log("timing GEMM1 and GEMM2 alone")
    g1_us, g1_bytes, g1_r = gemm_alone(ops, wl, weights, batches, torch, layout, ops.W13_SWIGLU)
    g2_us, g2_bytes, g2_r = gemm_alone(ops, wl, weights, batches, torch, layout, ops.W2)
    src = kernel_source_hash()
    traffic, traffic_note = load_traffic("gemm1_swiglu_qwen3_decode_t256_counters.json", src)
    traffic2, traffic2_note = load_traffic("gemm2_down_qwen3_decode_t256_counters.json", src)

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    sweep, prefill, ep, shared, fin, dense = [], None, [], None, None, None
    if "decode" in only:
        for ts in [int(v) for v in args.decode_tokens.split(",") if v]:
            log(f"decode T={ts}")
            sweep.append(decode_point(ops, wl, weights, ts, torch, layout, seed=ts))
    if "prefill" in only:
        log("prefill T=2048 (Zipf routing)")
        prefill = prefill_point(ops, WORKLOADS["qwen3_prefill"], weights, torch, layout)
    if "shared" in only:
        log("decode T=256 with one shared expert")
        sh = shared_weights(ops, wl, L, torch, layout)
        shared = decode_point(ops, wl, weights, 256, torch, layout, seed=256, shared=sh)
        del sh
    del weights
    torch.cuda.empty_cache()
    if "ep" in only:
        wle = WORKLOADS["ep_shard_decode"]
        log("EP shard: generating 8 weight replicas (726 MB each)")
        we = make_weights(wle, 8, torch, ops, layout, seed_base=11)
        for ts in (1, 16, 64, 256):
            log(f"EP shard T={ts}")
            ep.append(decode_point(ops, wle, we, ts, torch, layout, seed=ts + 7))
        del we
        torch.cuda.empty_cache()
    if "finalize" in only:
        log("finalize stream")
        fin = finalize_point(ops, torch)
    if "dense" in only:
        log("dense W4A16 GEMM")
        dense = dense_points(ops, torch, layout)

    w4a4 = None
    if "w4a4" in only:
        log("W4A4 (MXFP4) layer: decode 1/16/64/256 and prefill 2048")
        wm = make_mx_weights(ops, wl, 8, torch, seed_base=13)
        w4a4 = {"workload": "qwen3_decode / qwen3_prefill shapes, MXFP4 weights (tiled codes) and activations",
                "decode": [w4a4_point(ops, wl, wm, ts, torch, seed=ts + 3) for ts in (1, 16, 64, 256)],
                "prefill": w4a4_point(ops, WORKLOADS["qwen3_prefill"], wm, 2048, torch, seed=2049, prefill=True)}
        del wm
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline()

    rec = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name} (Qwen3-30B-A3B MoE layer, decode)", "tokens": T,
                   "experts": wl.num_experts, "top_k": wl.top_k, "hidden": wl.hidden, "inter": wl.inter,
                   "weights": f"int4 group-128 ({args.weights} code layout), bf16 scales",
                   "activations": "bf16", "replicas": L, "parallelism": "single GPU"},
        "layer_weight_GBps": round(layer_gbps, 1), "layer_hbm_frac": round(layer_gbps / HBM_PEAK_GBPS, 4),
        "roofline": {"kernel": "grouped GEMM1 (w13 + SwiGLU)", "bound": "hbm",
                     "achieved": round(g1_bytes / (g1_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(g1_bytes / (g1_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "algorithmic_bytes": round(g1_bytes), "avg_launch_us": round(g1_us, 3),
                     "median_launch_us": g1_r["median_us"], "traffic_note": traffic_note},
        "roofline_gemm2": {"kernel": "grouped GEMM2 (w2)", "bound": "hbm",
                           "achieved": round(g2_bytes / (g2_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                           "unit": "GB/s", "frac": round(g2_bytes / (g2_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                           "traffic": None if traffic2 is None else round(traffic2),
                           "algorithmic_bytes": round(g2_bytes), "avg_launch_us": round(g2_us, 3),
                           "median_launch_us": g2_r["median_us"], "traffic_note": traffic2_note},
        "cpu_baseline": cpu,
        "decode_sweep": sweep,
        "prefill": prefill,
        "shared_expert": shared,
        "ep_shard": ep,
        "finalize_stream": fin,
        "dense_gemm": dense,
        "w4a4_mxfp4": w4a4,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
