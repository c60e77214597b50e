"""The layer and the dense GEMM at the size limits the boundary accepts, vs the oracle.

- E_g = E_loc = 1024 experts with k = 16: routing takes its whole-wave path
  (64 lanes per token), the GEMMs hold 1024-entry chunk tables, the finalize
  its 16-slot variant.
- An expert-parallel window at the top of 512 experts with k = 16.
- k = E: every token goes to every expert.
- H = 16384 (GEMM1 reduces over 128 groups; GEMM2 has 16384 weight rows) and
  I = 16384 (the reverse), with two experts.
- Many rows on few experts (5000 tokens on 2 experts, k = 2).
- A long prefill (8192 tokens, Zipf routing): 64 token ranges in the permutation and
  several thousand tile-kernel items.
- The dense GEMM at N = 65536 and at K = 65536.
All within the layer tolerance (or the dense GEMM's derived bound).
"""
import numpy as np
import pytest

import oracle
from helpers import assert_layer_close, bf16_dev, bf16_to_f64, say, to_dev, to_np_u16
from w4a16_grouped_gemm_amd.inputs import WORKLOADS, Workload, bf16_bits, make_layer_inputs, make_shared_weights, pack_int4

pytestmark = pytest.mark.gpu

LIMITS = [
    (Workload("e1024_k16", 11, 1024, 1024, 0, 16, 256, 256, (1, 40)), 1, None),
    (Workload("e1024_k16", 11, 1024, 1024, 0, 16, 256, 256, (1, 40)), 40, None),
    (Workload("e512_window", 12, 512, 64, 448, 16, 256, 256, (100,)), 100, None),
    (Workload("k_equals_e", 13, 16, 16, 0, 16, 256, 256, (24,)), 24, None),
    (Workload("hidden_16384", 14, 2, 2, 0, 1, 16384, 128, (3,)), 3, None),
    (Workload("inter_16384", 15, 2, 2, 0, 1, 128, 16384, (3,)), 3, None),
    (Workload("rows_5000", 16, 2, 2, 0, 2, 256, 256, (5000,)), 5000, 24),
    (WORKLOADS["qwen3_prefill"], 8192, 48),           # tiled codes (the tile kernel)
]


@pytest.mark.parametrize("wl,T,n", LIMITS, ids=lambda v: v.name if isinstance(v, Workload) else str(v))
def test_layer_at_limits(wl, T, n):
    import torch
    from w4a16_grouped_gemm_amd import ops
    say(f"limits {wl.name} T={T}")
    inp = make_layer_inputs(wl, T)
    w13, w2 = to_dev(inp.w13_q), to_dev(inp.w2_q)
    tiled = wl.name == "qwen3_prefill"
    if tiled:
        w13, w2 = ops.pack_weights(ops.W13_SWIGLU, w13), ops.pack_weights(ops.W2, w2)
    o = ops.moe_w4a16_forward(bf16_dev(inp.x), to_dev(inp.logits), w13, bf16_dev(inp.s13), w2, bf16_dev(inp.s2),
                              wl.top_k, expert_begin=wl.expert_begin,
                              weight_layout=ops.WEIGHTS_TILED if tiled else ops.WEIGHTS_PLAIN)
    torch.cuda.synchronize()
    got = to_np_u16(o)
    sel = None
    if n is not None and T > n:
        sel = np.zeros(T, np.uint8)
        sel[np.unique(np.linspace(0, T - 1, n).astype(int))] = 1
    ref = oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=wl.top_k,
                       expert_begin=wl.expert_begin, tok_sel=sel)
    rows = np.arange(T) if sel is None else np.flatnonzero(sel)
    local = (ref["topk_ids"] >= wl.expert_begin) & (ref["topk_ids"] < wl.expert_begin + wl.num_local_experts)
    none = ~local.any(axis=1)
    assert np.all(got[none] == 0)
    keep = rows[~none[rows]]
    if keep.size:
        assert_layer_close(got[keep], ref["out"][keep], wl.name)


@pytest.mark.parametrize("M,N,K", [(3, 65536, 128), (3, 128, 65536)])
def test_dense_at_limits(M, N, K):
    import torch
    from w4a16_grouped_gemm_amd import ops
    say(f"dense limits M={M} N={N} K={K}")
    rng = np.random.default_rng(N + K)
    q = rng.integers(-8, 8, size=(N, K), dtype=np.int8)
    a = bf16_bits(rng.integers(-2, 3, size=(M, K)).astype(np.float32))
    s = np.full((N, K // 128), bf16_bits(np.float32(2.0 ** -6)), np.uint16)
    out = ops.dense_gemm_w4a16(bf16_dev(a), to_dev(pack_int4(q)), bf16_dev(s), out_dtype=torch.float32)
    torch.cuda.synchronize()
    # integer activations and codes: every partial sum is a multiple of 2^-6 below
    # 65536 * 2 * 8 * 2^-6 = 2^14 in magnitude (20 significant bits), exact in fp32
    want = (bf16_to_f64(a).astype(np.int64) @ q.T.astype(np.int64)).astype(np.float64) * 2.0 ** -6
    assert np.array_equal(out.cpu().numpy().astype(np.float64), want)


def test_shared_at_limits():
    # four shared experts (the most one call takes) after 16 routed slots of
    # 1024 experts: the finalize's longest chain, 20 terms per output
    import torch
    from w4a16_grouped_gemm_amd import ops
    wl = LIMITS[1][0]
    T = 40
    say(f"limits shared S=4 {wl.name} T={T}")
    inp = make_layer_inputs(wl, T)
    w13s, s13s, w2s, s2s = make_shared_weights(wl, 4)
    o = ops.moe_w4a16_forward(bf16_dev(inp.x), to_dev(inp.logits), to_dev(inp.w13_q), bf16_dev(inp.s13),
                              to_dev(inp.w2_q), bf16_dev(inp.s2), wl.top_k,
                              shared=(to_dev(w13s), bf16_dev(s13s), to_dev(w2s), bf16_dev(s2s)))
    torch.cuda.synchronize()
    ref = oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=wl.top_k,
                       shared=(w13s, s13s, w2s, s2s))
    assert_layer_close(to_np_u16(o), ref["out"], "shared S=4")


@pytest.mark.parametrize("mode", [0, -1])
def test_shared_at_expert_limit_split_k(mode):
    # 1024 routed experts plus four shared ones: the grouped GEMMs see 1028
    # experts, so every kernel's chunk table must hold 1029 entries. One token
    # with the split-K kernel forced (and the automatic choice)
    import torch
    from w4a16_grouped_gemm_amd import ops
    wl = LIMITS[0][0]
    T = 1
    say(f"limits shared S=4 {wl.name} T={T} gemm_mode={mode}")
    inp = make_layer_inputs(wl, T)
    w13s, s13s, w2s, s2s = make_shared_weights(wl, 4)
    with ops.launch_override(gemm_mode=mode):
        o = ops.moe_w4a16_forward(bf16_dev(inp.x), to_dev(inp.logits), to_dev(inp.w13_q), bf16_dev(inp.s13),
                                  to_dev(inp.w2_q), bf16_dev(inp.s2), wl.top_k,
                                  shared=(to_dev(w13s), bf16_dev(s13s), to_dev(w2s), bf16_dev(s2s)))
        torch.cuda.synchronize()
    ref = oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=wl.top_k,
                       shared=(w13s, s13s, w2s, s2s))
    assert_layer_close(to_np_u16(o), ref["out"], "shared S=4, 1028 experts")


def test_shared_zero_tokens():
    import torch
    from w4a16_grouped_gemm_amd import ops
    say("shared layer T=0")
    inp = make_layer_inputs("tiny", 4)
    empty = make_layer_inputs("tiny", 0, weights=False)
    w13s, s13s, w2s, s2s = make_shared_weights("tiny", 2)
    o = ops.moe_w4a16_forward(bf16_dev(empty.x), to_dev(empty.logits), to_dev(inp.w13_q), bf16_dev(inp.s13),
                              to_dev(inp.w2_q), bf16_dev(inp.s2), 2,
                              shared=(to_dev(w13s), bf16_dev(s13s), to_dev(w2s), bf16_dev(s2s)))
    torch.cuda.synchronize()
    assert tuple(o.shape) == (0, 256)
