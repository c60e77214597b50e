#!/usr/bin/env python3
"""Benchmark of the W4A16 MoE expert layer on one MI355X.

Workload: the Qwen3-30B-A3B MoE layer (128 experts, top-8, hidden 2048,
expert intermediate 768, int4 group-128 weights, bf16 activations) in
decode at 256 tokens. One step = one full layer forward (route, permute,
GEMM1 + SwiGLU, GEMM2, finalize) on one batch. Steps rotate over L layer
replicas with distinct weights and logits (L * 311 MB of weights), so the
256 MB Infinity Cache cannot serve the weights from one step to the next.
Replica 0 is the seeded workload of the parity tests; replicas 1..L-1 are
drawn on the GPU. All inputs are resident in HBM before timing starts; the
steps are replayed from HIP graphs (one graph per L steps).

Prints ONE JSON line (rank 0) with the layer throughput, the roofline of the
dominant kernel (GEMM1, bound by HBM weight bytes), a decode-size sweep and
the CPU oracle timed on the host as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; weight HBM GB/s % peak (decode), MFMA % (prefill)"
HBM_PEAK_GBPS = 8000.0
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "gemm1_swiglu_qwen3_decode_t256_counters.json")
KERNEL_SOURCES = ["w4a16_grouped_gemm_amd/csrc/gemm_w4a16.hip", "w4a16_grouped_gemm_amd/csrc/common.hpp"]


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


MFMA_PEAK_TFLOPS = 2500.0


def time_prefill(ops, reps, torch, layout, steps, warmup):
    """The same layer shape in prefill: 2048 tokens whose routing follows Zipf(1.1)
    expert popularity, weights of the decode replicas. Reported against the
    dense bf16 MFMA peak (algorithmic flops 6 * I * H per routed row)."""
    from w4a16_grouped_gemm_amd.inputs import WORKLOADS, make_layer_inputs
    wl = WORKLOADS["qwen3_prefill"]
    T = 2048
    inp = make_layer_inputs(wl, T, weights=False)
    dev = torch.device("cuda")
    x = torch.from_numpy(inp.x).to(dev).view(torch.bfloat16)
    lg = torch.from_numpy(inp.logits).to(dev)
    reps_p = [dict(r, x=x, logits=lg) for r in reps]
    dt, _ = time_layer(ops, wl, reps_p, steps, warmup, torch, layout)
    us = dt / steps * 1e6
    flops = 6.0 * wl.inter * wl.hidden * T * wl.top_k
    return {"tokens": T, "routing": "zipf(1.1)", "us_per_layer": round(us, 1), "tokens_per_s": round(T / (us * 1e-6), 1),
            "tflops": round(flops / (us * 1e-6) / 1e12, 1), "mfma_frac": round(flops / (us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS, 4)}


def _graph_time(torch, fns, reps_n):
    """Seconds per call of the launches `fns` (one each per replay), replayed
    from a HIP graph, HIP events on the replaying stream."""
    for f in fns:
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
    stream = torch.cuda.current_stream()
    graph.replay()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps_n):
        graph.replay()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / 1000.0 / (reps_n * len(fns))


def time_ep_shard(ops, torch, layout, steps, warmup, T=256, L=3):
    """One GPU's shard of an expert-parallel layer (32 local of 256 experts,
    hidden 7168, intermediate 2048) in decode: the layer on its local slots,
    L replicas of 726 MB of weights."""
    from w4a16_grouped_gemm_amd.inputs import WORKLOADS
    wl = WORKLOADS["ep_shard_decode"]
    _, reps = make_replicas(wl, T, L, torch, seed_base=11)
    if layout == ops.WEIGHTS_TILED:
        pack_replicas(reps, ops)
    stats = routing_stats(ops, wl, reps, torch)
    dt, _ = time_layer(ops, wl, reps, steps, warmup, torch, layout)
    us = dt / steps * 1e6
    w13b, w2b = weight_bytes_per_expert(wl.hidden, wl.inter)
    act = sum(st["active"] for st in stats) / L
    gbps = act * (w13b + w2b) / (us * 1e-6) / 1e9
    del reps
    torch.cuda.empty_cache()
    return {"workload": "ep_shard_decode (32 of 256 experts, hidden 7168, inter 2048, top-8)", "tokens": T,
            "us_per_layer": round(us, 2), "tokens_per_s": round(T / (us * 1e-6), 1), "active_experts": act,
            "local_rows": sum(st["rows"] for st in stats) / L, "weight_GBps": round(gbps, 1),
            "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}


def time_shared(ops, wl, reps, torch, layout, steps, warmup, S=1):
    """The decode layer with S shared experts of the routed shape (every token
    through each; DeepSeek-style), on the same replicas."""
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    H, I = wl.hidden, wl.inter
    reps_s = []
    for i, r in enumerate(reps):
        g.manual_seed(31000 + i)
        w13 = torch.randint(0, 256, (S, 2 * I, H // 2), generator=g, device=dev, dtype=torch.uint8)
        w2 = torch.randint(0, 256, (S, H, I // 2), generator=g, device=dev, dtype=torch.uint8)
        if layout == ops.WEIGHTS_TILED:
            w13, w2 = ops.pack_weights(ops.W13_SWIGLU, w13), ops.pack_weights(ops.W2, w2)
        s13 = torch.empty((S, 2 * I, H // 128), device=dev).uniform_(0.005, 0.02, generator=g).to(torch.bfloat16)
        s2 = torch.empty((S, H, I // 128), device=dev).uniform_(0.005, 0.02, generator=g).to(torch.bfloat16)
        reps_s.append(dict(r, shared=(w13, s13, w2, s2)))
    T = reps[0]["x"].shape[0]
    dt, _ = time_layer(ops, wl, reps_s, steps, warmup, torch, layout)
    us = dt / steps * 1e6
    w13b, w2b = weight_bytes_per_expert(H, I)
    stats = routing_stats(ops, wl, reps, torch)
    act = sum(st["active"] for st in stats) / len(reps) + S
    gbps = act * (w13b + w2b) / (us * 1e-6) / 1e9
    return {"shared_experts": S, "tokens": T, "us_per_layer": round(us, 2), "tokens_per_s": round(T / (us * 1e-6), 1),
            "experts_streamed": act, "weight_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}


def time_finalize_stream(ops, torch, T=4096, k=8, H=4096, E=128, reps_n=20):
    """The finalize on its stress shape: fp32 y [T*k, H] (512 MiB, two buffers
    alternate so the Infinity Cache cannot hold them), bf16 out [T, H]."""
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    logits = torch.randn((T, E), generator=g, device=dev)
    ids, w = ops.route(logits, k)
    _, _, _, inv, _ = ops.permute(ids, E)
    ys = [torch.randn((T * k, H), generator=g, device=dev) for _ in range(2)]
    outs = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    sec = _graph_time(torch, [lambda i=i: ops.finalize(ys[i], w, inv, out=outs[i]) for i in range(2)], reps_n)
    nbytes = T * k * H * 4 + T * k * 8 + T * H * 2
    del ys, outs
    torch.cuda.empty_cache()
    return {"shape": f"T={T} k={k} H={H}, fp32 y, bf16 out", "us": round(sec * 1e6, 2), "bytes": nbytes,
            "GBps": round(nbytes / sec / 1e9, 1), "hbm_frac": round(nbytes / sec / 1e9 / HBM_PEAK_GBPS, 4)}


def time_dense(ops, torch, layout, Ms=(1, 16, 256), N=14336, K=4096, L=16, reps_n=20):
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
        fns = [lambda i=i: ops.dense_gemm_w4a16(a, ws[i][0], ws[i][1], out=outs[i], weight_layout=layout)
               for i in range(L)]
        sec = _graph_time(torch, fns, reps_n)
        res.append({"M": M, "N": N, "K": K, "us": round(sec * 1e6, 2),
                    "weight_GBps": round(wbytes / sec / 1e9, 1), "hbm_frac": round(wbytes / sec / 1e9 / HBM_PEAK_GBPS, 4),
                    "tflops": round(2.0 * M * N * K / sec / 1e12, 2)})
    del ws
    torch.cuda.empty_cache()
    return res


def gemm1_algorithmic_bytes(wl, T, active, rows):
    """Bytes GEMM1 must move at least once: the weights and scales of every
    active expert, the T input rows, the rows x I SwiGLU outputs, the offsets
    and the row index."""
    w13b, _ = weight_bytes_per_expert(wl.hidden, wl.inter)
    return (active * w13b + T * wl.hidden * 2 + rows * wl.inter * 2 + (wl.num_local_experts + 1) * 4
            + rows * 4)


def make_replicas(wl, T, L, torch, seed_base=7):
    """Replica 0 from the seeded numpy generator, the rest drawn on the GPU."""
    from w4a16_grouped_gemm_amd.inputs import make_layer_inputs
    dev = torch.device("cuda")
    H, I, E, El = wl.hidden, wl.inter, wl.num_experts, wl.num_local_experts
    inp = make_layer_inputs(wl, T)

    def d(a, dtype=None):
        t = torch.from_numpy(a).to(dev)
        return t.view(dtype) if dtype is not None else t

    reps = [dict(x=d(inp.x, torch.bfloat16), logits=d(inp.logits), w13=d(inp.w13_q), s13=d(inp.s13, torch.bfloat16),
                 w2=d(inp.w2_q), s2=d(inp.s2, torch.bfloat16))]
    g = torch.Generator(device=dev)
    for i in range(1, L):
        g.manual_seed(seed_base * 1000 + i)
        reps.append(dict(
            x=torch.randn((T, H), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16),
            logits=torch.randn((T, E), generator=g, device=dev, dtype=torch.float32),
            w13=torch.randint(0, 256, (El, 2 * I, H // 2), generator=g, device=dev, dtype=torch.uint8),
            s13=torch.empty((El, 2 * I, H // 128), device=dev).uniform_(0.005, 0.02, generator=g).to(torch.bfloat16),
            w2=torch.randint(0, 256, (El, H, I // 2), generator=g, device=dev, dtype=torch.uint8),
            s2=torch.empty((El, H, I // 128), device=dev).uniform_(0.005, 0.02, generator=g).to(torch.bfloat16)))
    return inp, reps


def pack_replicas(reps, ops):
    """Reorder every replica's codes into the tiled layout (a once-per-model step, untimed)."""
    for r in reps:
        r["w13"] = ops.pack_weights(ops.W13_SWIGLU, r["w13"])
        r["w2"] = ops.pack_weights(ops.W2, r["w2"])


def new_batch(wl, T, reps, torch, seed):
    """Fresh activations / logits of T tokens for every replica (weights kept)."""
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    out = []
    for i, r in enumerate(reps):
        g.manual_seed(seed * 1000 + i)
        out.append(dict(r, x=torch.randn((T, wl.hidden), generator=g, device=dev).to(torch.bfloat16),
                        logits=torch.randn((T, wl.num_experts), generator=g, device=dev)))
    return out


def time_layer(ops, wl, reps, steps, warmup, torch, layout=0):
    """Capture L forwards in one graph; replay; return (seconds for `steps` steps, outs)."""
    L = len(reps)
    T = reps[0]["x"].shape[0]
    outs = [torch.empty((T, wl.hidden), dtype=torch.bfloat16, device="cuda") for _ in reps]
    shape = ops.make_shape(T, wl.hidden, wl.inter, wl.num_experts, wl.num_local_experts, wl.top_k,
                           wl.expert_begin, weight_layout=layout)
    nsh = reps[0]["shared"][0].shape[0] if reps[0].get("shared") is not None else 0
    wsz = ops.workspace_size(shape) if nsh == 0 else \
        int(ops.load_library().moe_w4a16_workspace_size_shared(__import__("ctypes").byref(shape), nsh))
    ws = torch.empty(max(wsz, 256), dtype=torch.uint8, device="cuda")

    def fwd(i):
        r = reps[i]
        ops.moe_w4a16_forward(r["x"], r["logits"], r["w13"], r["s13"], r["w2"], r["s2"], wl.top_k,
                              out=outs[i], expert_begin=wl.expert_begin, workspace=ws, weight_layout=layout,
                              shared=r.get("shared"))

    for i in range(L):          # eager pass (also loads kernels)
        fwd(i)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graphs_all = torch.cuda.CUDAGraph()
    singles = [torch.cuda.CUDAGraph() for _ in range(L)]
    with torch.cuda.stream(s):
        with torch.cuda.graph(graphs_all, stream=s):
            for i in range(L):
                fwd(i)
        for i in range(L):
            with torch.cuda.graph(singles[i], stream=s):
                fwd(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    def run(n):
        full, rem = divmod(n, L)
        for _ in range(full):
            graphs_all.replay()
        for i in range(rem):
            singles[i].replay()

    run(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    return dt, outs


def routing_stats(ops, wl, reps, torch):
    """Per replica: perm / offsets (for the kernel timing) and active experts."""
    res = []
    for r in reps:
        ids, w = ops.route(r["logits"], wl.top_k)
        counts, offsets, perm, inv, _ = ops.permute(ids, wl.num_local_experts, num_experts=wl.num_experts,
                                                    expert_begin=wl.expert_begin)
        res.append(dict(offsets=offsets, perm=perm, counts=counts))
    torch.cuda.synchronize()
    for d in res:
        d["active"] = int((d["counts"] > 0).sum().item())
        d["rows"] = int(d["offsets"][-1].item())
    return res


def time_gemm1(ops, wl, reps, stats, reps_n, torch, layout=0):
    """Average duration of one GEMM1 (w13 + SwiGLU) launch, HIP events on its stream."""
    L = len(reps)
    T = reps[0]["x"].shape[0]
    hs = [torch.empty((T * wl.top_k, wl.inter), dtype=torch.bfloat16, device="cuda") for _ in reps]

    def g1(i):
        ops.grouped_gemm_w4a16(ops.W13_SWIGLU, reps[i]["x"], stats[i]["offsets"], reps[i]["w13"],
                               reps[i]["s13"], num_tokens=T, top_k=wl.top_k, a_row_index=stats[i]["perm"],
                               num_experts=wl.num_experts, out=hs[i], weight_layout=layout)

    for i in range(L):
        g1(i)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for i in range(L):
                g1(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    graph.replay()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps_n):
        graph.replay()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / 1000.0 / (reps_n * L)


def load_traffic(expected_hash):
    if not os.path.exists(PROFILE_COUNTERS):
        return None, "no counter profile"
    with open(PROFILE_COUNTERS) as f:
        c = json.load(f)
    if c.get("kernel_source_sha256") != expected_hash:
        return None, "kernel changed since the counters were taken"
    ff = c["copy_bytes"] / (c["copy_fetch_kib"] * 1024.0)
    fw = c["copy_bytes"] / (c["copy_write_kib"] * 1024.0)
    return (c["fetch_kib_per_dispatch"] * ff + c["write_kib_per_dispatch"] * fw) * 1024.0, \
        f"FETCH_SIZE x {ff:.4f} + WRITE_SIZE x {fw:.4f} (copy-kernel scale)"


def cpu_baseline(inp, wl, budget_s=10.0, max_runs=64):
    """The oracle's full layer on the seeded batch, repeated until about
    `budget_s` seconds of host time are spent; tokens per second overall."""
    import oracle
    oracle.build(force=False)
    cores = len(os.sched_getaffinity(0))
    env_threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(cores, env_threads) if env_threads > 0 else cores
    oracle.set_threads(threads)
    runs, total = 0, 0.0
    while runs < max_runs and total < budget_s:
        t0 = time.perf_counter()
        oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=wl.top_k,
                     expert_begin=wl.expert_begin)
        total += time.perf_counter() - t0
        runs += 1
    return {"value": inp.tokens * runs / total, "unit": "tokens/s", "cores": oracle.get_threads(),
            "kind": "oracle",
            "sample": f"{runs} run(s) of the full layer (fp64) over the seeded {inp.tokens}-token batch of "
                      f"replica 0, {total:.1f} s in all"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--tokens", type=int, default=256)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    wl = WORKLOADS["qwen3_decode"]
    T, L = args.tokens, args.replicas
    log(f"generating {L} replicas of {wl.name} (T={T})")
    inp, reps = make_replicas(wl, T, L, torch)
    layout = ops.WEIGHTS_TILED if args.weights == "tiled" else ops.WEIGHTS_PLAIN
    if layout == ops.WEIGHTS_TILED:
        pack_replicas(reps, ops)
    stats = routing_stats(ops, wl, reps, torch)
    w13b, w2b = weight_bytes_per_expert(wl.hidden, wl.inter)
    log("timing the layer")
    dt, _ = time_layer(ops, wl, reps, args.steps, args.warmup, torch, layout)
    ms = dt / args.steps * 1e3
    tok_s = T * args.steps / dt
    mean_active = sum(s["active"] for s in stats) / L
    layer_bytes = mean_active * (w13b + w2b)
    layer_gbps = layer_bytes / (ms * 1e-3) / 1e9

    log("timing GEMM1 alone")
    g1 = time_gemm1(ops, wl, reps, stats, max(4, args.steps // L), torch, layout)
    g1_bytes = sum(gemm1_algorithmic_bytes(wl, T, s["active"], s["rows"]) for s in stats) / L
    achieved = g1_bytes / g1 / 1e9
    traffic, traffic_note = load_traffic(kernel_source_hash())

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    sweep = []
    if not args.no_sweep:
        for ts in (1, 16, 64):
            log(f"sweep T={ts}")
            reps_t = new_batch(wl, ts, reps, torch, seed=ts)
            st = routing_stats(ops, wl, reps_t, torch)
            n = max(args.steps, 200)
            dts, _ = time_layer(ops, wl, reps_t, n, args.warmup, torch, layout)
            act = sum(s["active"] for s in st) / L
            us = dts / n * 1e6
            sweep.append({"tokens": ts, "us_per_layer": round(us, 2), "tokens_per_s": round(ts * n / dts, 1),
                          "active_experts": act, "weight_GBps": round(act * (w13b + w2b) / (us * 1e-6) / 1e9, 1),
                          "hbm_frac": round(act * (w13b + w2b) / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)})
        sweep.append({"tokens": T, "us_per_layer": round(ms * 1e3, 2), "tokens_per_s": round(tok_s, 1),
                      "active_experts": mean_active, "weight_GBps": round(layer_gbps, 1),
                      "hbm_frac": round(layer_gbps / HBM_PEAK_GBPS, 4)})

    prefill = None
    if not args.no_sweep:
        log("prefill T=2048 (Zipf routing)")
        prefill = time_prefill(ops, reps, torch, layout, max(8, args.steps // 50), args.warmup // 10 + 1)

    ep_shard = finalize_stream = dense = shared = None
    if not args.no_sweep:
        log("layer with one shared expert T=256")
        shared = time_shared(ops, wl, reps, torch, layout, max(100, args.steps // 2), args.warmup)
        del reps
        torch.cuda.empty_cache()
        log("EP shard decode T=256")
        ep_shard = time_ep_shard(ops, torch, layout, max(60, args.steps // 4), max(6, args.warmup // 10))
        log("finalize stream")
        finalize_stream = time_finalize_stream(ops, torch)
        log("dense W4A16 GEMM")
        dense = time_dense(ops, torch, layout)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(inp, wl)

    rec = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name} (Qwen3-30B-A3B MoE layer, decode)", "tokens": T,
                   "experts": wl.num_experts, "top_k": wl.top_k, "hidden": wl.hidden, "inter": wl.inter,
                   "weights": f"int4 group-128 ({args.weights} code layout), bf16 scales",
                   "activations": "bf16", "replicas": L,
                   "parallelism": "single GPU"},
        "layer_weight_GBps": round(layer_gbps, 1), "layer_hbm_frac": round(layer_gbps / HBM_PEAK_GBPS, 4),
        "roofline": {"kernel": "gemm_stream_kernel<W13_SWIGLU> (GEMM1 + SwiGLU)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "algorithmic_bytes": round(g1_bytes), "avg_launch_us": round(g1 * 1e6, 3),
                     "traffic_note": traffic_note},
        "cpu_baseline": cpu,
        "sweep": sweep,
        "prefill": prefill,
        "shared_expert": shared,
        "ep_shard": ep_shard,
        "finalize_stream": finalize_stream,
        "dense_gemm": dense,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
