"""Seeded synthetic inputs for the W4A16 MoE expert layer.

Shared by the GPU path's tests and benchmark and by the CPU oracle's tests. It
holds none of the layer's arithmetic: it draws numbers, encodes them in the
storage formats (bf16 bit patterns, nibble-packed int4) and names the
workloads. Everything is numpy PCG64 with seed = 1000 * (workload index + 1)
+ tokens and a fixed draw order: x, logits, w13, s13, w2, s2.

Storage formats:
  bf16      uint16 bit pattern, round-to-nearest-even from binary32.
  int4      two's-complement codes in [-8, 7]; element k of a row lives in
            byte k // 2, even k in the low nibble; rows are K-contiguous.
  scales    bf16 [E, N, K // 128], one per (row, 128-wide K group).
  w13       [E, 2I, H/2]: rows [0, I) gate projection, [I, 2I) up projection.
  w2        [E, H, I/2].

Workloads (the MoE layers the pages discuss):
  tiny              8 experts, top-2, hidden 256, inter 512, 16 tokens
  qwen3_decode      Qwen3-30B-A3B MoE layer (128 experts, top-8, hidden 2048,
                    inter 768), decode at 1 / 16 / 64 / 256 tokens
  qwen3_prefill     same layer, 2048 tokens, Zipf(1.1) expert popularity
  ep_shard_decode   one GPU's shard of an expert-parallel layer: 32 local of
                    256 experts, top-8, hidden 7168, inter 2048, 1-256 tokens
  finalize_stress   combine only: 4096 tokens, top-8, hidden 4096, fp32 expert
                    outputs with exact zeros and subnormals, zero weights
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

GROUP = 128


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    num_experts: int          # E_g: columns of the router logits
    num_local_experts: int    # E_loc: experts whose weights this GPU holds
    expert_begin: int         # first local expert id
    top_k: int
    hidden: int
    inter: int
    tokens: tuple = field(default_factory=tuple)
    routing: str = "normal"   # "normal" | "zipf"


WORKLOADS = {
    "tiny": Workload("tiny", 0, 8, 8, 0, 2, 256, 512, (16,)),
    "qwen3_decode": Workload("qwen3_decode", 1, 128, 128, 0, 8, 2048, 768, (1, 16, 64, 256)),
    "qwen3_prefill": Workload("qwen3_prefill", 2, 128, 128, 0, 8, 2048, 768, (2048,), "zipf"),
    "ep_shard_decode": Workload("ep_shard_decode", 3, 256, 32, 0, 8, 7168, 2048, (1, 16, 64, 256)),
}
FINALIZE_STRESS = dict(name="finalize_stress", index=4, tokens=4096, top_k=8, hidden=4096,
                       num_experts=128)


def seed_for(index: int, tokens: int) -> int:
    return 1000 * (index + 1) + tokens


def bf16_bits(a) -> np.ndarray:
    """binary32 array -> bf16 bit patterns, round to nearest even (no NaNs drawn)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_values(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> binary32 values (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """int codes in [-8, 7], last axis K (even) -> uint8 [..., K/2], even k low nibble."""
    q = np.asarray(q)
    assert q.shape[-1] % 2 == 0
    assert q.min(initial=0) >= -8 and q.max(initial=0) <= 7
    lo = (q[..., 0::2].astype(np.int16) & 0xF).astype(np.uint8)
    hi = (q[..., 1::2].astype(np.int16) & 0xF).astype(np.uint8)
    return lo | (hi << 4)


def unpack_int4(p: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] -> int8 codes [..., K] (inverse of pack_int4)."""
    p = np.asarray(p, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int8)
    hi = (p >> 4).astype(np.int8)
    q = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.int8)
    q[..., 0::2] = np.where(lo >= 8, lo - 16, lo)
    q[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
    return q


def random_int4_packed(rng: np.random.Generator, shape_packed) -> np.ndarray:
    """Uniform int4 codes in [-8, 7], already packed: every byte holds two
    independent uniform nibbles, i.e. two independent uniform codes."""
    return rng.integers(0, 256, size=shape_packed, dtype=np.uint8)


def random_scales(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_bits(rng.uniform(0.005, 0.02, size=shape).astype(np.float32))


def zipf_logits(rng: np.random.Generator, tokens: int, experts: int, s: float = 1.1) -> np.ndarray:
    """Router logits whose top-k sets follow Zipf(s) expert popularity.

    Gumbel-top-k: l[t, e] = log p[pi(e)] + G[t, e], G ~ Gumbel(0, 1), p_r ~ r^-s
    for popularity rank r = 1..E and a seeded permutation pi. The top-k of
    such logits is an exact sample of k distinct experts without replacement
    with probabilities p (Plackett-Luce).
    """
    ranks = np.arange(1, experts + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    pi = rng.permutation(experts)
    g = rng.gumbel(size=(tokens, experts))
    return (np.log(p[pi])[None, :] + g).astype(np.float32)


@dataclass
class LayerInputs:
    workload: Workload
    tokens: int
    x: np.ndarray        # uint16 (bf16) [T, H]
    logits: np.ndarray   # float32 [T, E_g]
    w13_q: np.ndarray    # uint8 [E_loc, 2I, H/2]
    s13: np.ndarray      # uint16 (bf16) [E_loc, 2I, H/128]
    w2_q: np.ndarray     # uint8 [E_loc, H, I/2]
    s2: np.ndarray       # uint16 (bf16) [E_loc, H, I/128]


def make_layer_inputs(workload: str | Workload, tokens: int, seed: int | None = None,
                      weights: bool = True) -> LayerInputs:
    """Draw x, logits and (unless weights=False) the four weight arrays.

    Weights are drawn last, so skipping them leaves x and logits unchanged."""
    wl = WORKLOADS[workload] if isinstance(workload, str) else workload
    T, H, I, E, El = tokens, wl.hidden, wl.inter, wl.num_experts, wl.num_local_experts
    rng = np.random.Generator(np.random.PCG64(seed_for(wl.index, T) if seed is None else seed))
    x = bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    if wl.routing == "zipf":
        logits = zipf_logits(rng, T, E)
    else:
        logits = rng.standard_normal((T, E), dtype=np.float32)
    if not weights:
        return LayerInputs(wl, T, x, logits, None, None, None, None)
    w13_q = random_int4_packed(rng, (El, 2 * I, H // 2))
    s13 = random_scales(rng, (El, 2 * I, H // GROUP))
    w2_q = random_int4_packed(rng, (El, H, I // 2))
    s2 = random_scales(rng, (El, H, I // GROUP))
    return LayerInputs(wl, T, x, logits, w13_q, s13, w2_q, s2)


def make_shared_weights(workload: str | Workload, num_shared: int, seed: int | None = None):
    """Weights of `num_shared` always-on (shared) experts with the routed
    experts' shape and distributions: (w13_sh, s13_sh, w2_sh, s2_sh), leading
    axis num_shared. Seeded apart from the layer inputs (seed default:
    the workload's seed + 500000 + num_shared)."""
    wl = WORKLOADS[workload] if isinstance(workload, str) else workload
    H, I, S = wl.hidden, wl.inter, num_shared
    rng = np.random.Generator(np.random.PCG64(seed_for(wl.index, 0) + 500000 + S if seed is None else seed))
    return (random_int4_packed(rng, (S, 2 * I, H // 2)), random_scales(rng, (S, 2 * I, H // GROUP)),
            random_int4_packed(rng, (S, H, I // 2)), random_scales(rng, (S, H, I // GROUP)))


@dataclass
class Mxfp4LayerInputs:
    """The W4A4 variant's layer inputs: x and logits as in make_layer_inputs,
    weights as MXFP4 (E2M1 codes in the int4 byte layout, E8M0 scales per 32
    along K)."""
    workload: Workload
    tokens: int
    x: np.ndarray        # uint16 (bf16) [T, H]
    logits: np.ndarray   # float32 [T, E_g]
    w13_q: np.ndarray    # uint8 E2M1 codes [E_loc, 2I, H/2]
    w13_s: np.ndarray    # uint8 E8M0 [E_loc, 2I, H/32]
    w2_q: np.ndarray     # uint8 E2M1 codes [E_loc, H, I/2]
    w2_s: np.ndarray     # uint8 E8M0 [E_loc, H, I/32]


MX_BLOCK = 32
MX_SCALE_RANGE = (119, 121)   # E8M0 bytes: scales 2^-8 .. 2^-6, the W4A16 scales' magnitude


def make_mxfp4_layer_inputs(workload: str | Workload, tokens: int, seed: int | None = None) -> Mxfp4LayerInputs:
    """x and logits drawn exactly as make_layer_inputs draws them (same seed,
    same order), then w13 codes, w13 scales, w2 codes, w2 scales: every code
    byte uniform (two independent uniform E2M1 codes), every scale byte
    uniform over MX_SCALE_RANGE."""
    wl = WORKLOADS[workload] if isinstance(workload, str) else workload
    T, H, I, E, El = tokens, wl.hidden, wl.inter, wl.num_experts, wl.num_local_experts
    rng = np.random.Generator(np.random.PCG64(seed_for(wl.index, T) if seed is None else seed))
    x = bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    if wl.routing == "zipf":
        logits = zipf_logits(rng, T, E)
    else:
        logits = rng.standard_normal((T, E), dtype=np.float32)
    lo, hi = MX_SCALE_RANGE
    w13_q = rng.integers(0, 256, size=(El, 2 * I, H // 2), dtype=np.uint8)
    w13_s = rng.integers(lo, hi + 1, size=(El, 2 * I, H // MX_BLOCK), dtype=np.uint8)
    w2_q = rng.integers(0, 256, size=(El, H, I // 2), dtype=np.uint8)
    w2_s = rng.integers(lo, hi + 1, size=(El, H, I // MX_BLOCK), dtype=np.uint8)
    return Mxfp4LayerInputs(wl, T, x, logits, w13_q, w13_s, w2_q, w2_s)


@dataclass
class FinalizeStressInputs:
    logits: np.ndarray      # float32 [T, E]: route these with top_k to get ids / weights
    zero_mask: np.ndarray   # bool [T, k]: routing weights forced to +0.0
    y: np.ndarray           # float32 [T*k, H]


def make_finalize_stress(tokens: int | None = None, hidden: int | None = None,
                         seed: int | None = None) -> FinalizeStressInputs:
    """Expert outputs: each element independently 80% N(0,1), 10% exact +-0.0
    (sign 50/50), 10% subnormal with random sign and magnitude 10^U[-40, -38]
    (all below 2^-126). Logits N(0,1) over 128 experts; 10% of the routing
    weights are then set to +0.0 (zero_mask)."""
    fs = FINALIZE_STRESS
    T = fs["tokens"] if tokens is None else tokens
    H = fs["hidden"] if hidden is None else hidden
    k, E = fs["top_k"], fs["num_experts"]
    rng = np.random.Generator(np.random.PCG64(seed_for(fs["index"], T) if seed is None else seed))
    logits = rng.standard_normal((T, E), dtype=np.float32)
    zero_mask = rng.random((T, k)) < 0.1
    R = T * k
    kind = rng.random((R, H))
    sign = np.where(rng.random((R, H)) < 0.5, -1.0, 1.0)
    normal = rng.standard_normal((R, H))
    sub = 10.0 ** rng.uniform(-40.0, -38.0, size=(R, H))
    y64 = np.where(kind < 0.8, normal, np.where(kind < 0.9, sign * 0.0, sign * sub))
    y = y64.astype(np.float32)
    return FinalizeStressInputs(logits, zero_mask, y)
