"""The layer with shared experts (moe_w4a16_forward_shared) on the GPU vs the oracle.

Reading of the GC-MoE abstract's optional shared experts: S always-on experts
with the routed experts' shape run on every token; each one's bf16 output is
added to the binary32 combine with weight 1 after the routed slots. The GPU
folds them into the routed launches (extra experts of the grouped GEMMs).

Tolerance as for the layer: max |gpu - ref| <= 2e-2 * max |ref| and
sum|gpu - ref| / sum|ref| <= 5e-3; full sizes on sampled tokens.
"""
import numpy as np
import pytest

import oracle
from helpers import assert_layer_close, bf16_dev, say, to_dev, to_np_u16
from w4a16_grouped_gemm_amd.inputs import make_layer_inputs, make_shared_weights

pytestmark = pytest.mark.gpu


def _forward(inp, shared, tiled=False):
    import torch
    from w4a16_grouped_gemm_amd import ops
    w13, w2 = to_dev(inp.w13_q), to_dev(inp.w2_q)
    sh = None
    if shared is not None:
        w13s, s13s, w2s, s2s = shared
        w13s, w2s = to_dev(w13s), to_dev(w2s)
        if tiled:
            w13s, w2s = ops.pack_weights(ops.W13_SWIGLU, w13s), ops.pack_weights(ops.W2, w2s)
        sh = (w13s, bf16_dev(s13s), w2s, bf16_dev(s2s))
    if tiled:
        w13, w2 = ops.pack_weights(ops.W13_SWIGLU, w13), ops.pack_weights(ops.W2, w2)
    o = ops.moe_w4a16_forward(bf16_dev(inp.x), to_dev(inp.logits), w13, bf16_dev(inp.s13), w2,
                              bf16_dev(inp.s2), inp.workload.top_k, expert_begin=inp.workload.expert_begin,
                              weight_layout=ops.WEIGHTS_TILED if tiled else ops.WEIGHTS_PLAIN, shared=sh)
    torch.cuda.synchronize()
    return to_np_u16(o)


CASES = [("tiny", 16, 1, 64), ("tiny", 16, 2, 64), ("qwen3_decode", 1, 1, 64), ("qwen3_decode", 64, 1, 16),
         ("qwen3_decode", 256, 2, 12), ("ep_shard_decode", 16, 1, 8)]


@pytest.mark.parametrize("wl,T,S,n", CASES)
def test_shared_layer_matches_oracle(wl, T, S, n):
    say(f"shared layer {wl} T={T} S={S} sample={n}")
    inp = make_layer_inputs(wl, T)
    sh = make_shared_weights(inp.workload, S)
    got = _forward(inp, sh)
    sel = None
    if T > n:
        sel = np.zeros(T, np.uint8)
        sel[np.unique(np.linspace(0, T - 1, n).astype(int))] = 1
    ref = oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=inp.workload.top_k,
                       expert_begin=inp.workload.expert_begin, tok_sel=sel, shared=sh)
    rows = np.arange(T) if sel is None else np.flatnonzero(sel)
    assert_layer_close(got[rows], ref["out"][rows], f"{wl} T={T} S={S}")


@pytest.mark.parametrize("wl,T", [("qwen3_decode", 64), ("ep_shard_decode", 64)])
def test_zero_shared_scales_give_the_routed_layer(wl, T):
    # shared experts with all-zero scales output exactly +0 (every group sum
    # is multiplied by 0; zero codes would not do: the 136-offset correction
    # and the main MFMA chain round differently), so adding them gives back
    # the routed layer bit for bit, with -0 turned into +0 by the addition
    say(f"shared zero scales {wl} T={T}")
    inp = make_layer_inputs(wl, T)
    w13s, s13s, w2s, s2s = make_shared_weights(inp.workload, 1)
    base = _forward(inp, None)
    got = _forward(inp, (w13s, np.zeros_like(s13s), w2s, np.zeros_like(s2s)))
    assert np.array_equal(got, np.where(base == 0x8000, 0, base))


def test_shared_tiled_equals_plain():
    say("shared layer tiled vs plain")
    inp = make_layer_inputs("qwen3_decode", 64)
    sh = make_shared_weights("qwen3_decode", 2)
    assert np.array_equal(_forward(inp, sh, tiled=True), _forward(inp, sh))


def test_shared_argument_errors():
    import ctypes
    import torch
    from w4a16_grouped_gemm_amd import ops
    say("shared argument errors")
    inp = make_layer_inputs("tiny", 4)
    w13s, s13s, w2s, s2s = make_shared_weights("tiny", 1)
    with pytest.raises(ValueError):                       # shared w2 of the wrong shape
        ops.moe_w4a16_forward(bf16_dev(inp.x), to_dev(inp.logits), to_dev(inp.w13_q), bf16_dev(inp.s13),
                              to_dev(inp.w2_q), bf16_dev(inp.s2), 2,
                              shared=(to_dev(w13s), bf16_dev(s13s), to_dev(w2s)[:, :128], bf16_dev(s2s)))
    lib = ops.load_library()
    sh = ops.make_shape(4, 256, 512, 8, 8, 2)
    assert lib.moe_w4a16_workspace_size_shared(ctypes.byref(sh), 0) == 0
    assert lib.moe_w4a16_workspace_size_shared(ctypes.byref(sh), 5) == 0
    assert lib.moe_w4a16_workspace_size_shared(ctypes.byref(sh), 1) > lib.moe_w4a16_workspace_size(ctypes.byref(sh))
    torch.cuda.synchronize()


@pytest.mark.parametrize("wl,T,S", [("qwen3_decode", 1024, 2), ("qwen3_prefill", 2048, 1)])
def test_shared_many_tokens_sampled(wl, T, S):
    # past 384 tokens the permutation runs over token ranges (the first
    # range writes the shared segments); at 2048 tokens both GEMMs take the tile kernel,
    # shared experts included. 64 sampled tokens against the oracle
    say(f"shared layer {wl} T={T} S={S} (sampled)")
    inp = make_layer_inputs(wl, T)
    sh = make_shared_weights(wl, S)
    got = _forward(inp, sh, tiled=True)
    sel = np.zeros(T, np.uint8)
    rows = np.unique(np.linspace(0, T - 1, 64).astype(int))
    sel[rows] = 1
    ref = oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=inp.workload.top_k,
                       expert_begin=inp.workload.expert_begin, tok_sel=sel, shared=sh)
    assert_layer_close(got[rows], ref["out"][rows], f"shared {wl} T={T}")


@pytest.mark.parametrize("wl,T,S", [("tiny", 40, 4), ("qwen3_decode", 64, 1), ("qwen3_decode", 256, 2),
                                    ("ep_shard_decode", 64, 1)])
def test_shared_permutation_in_gemm_equals_separate_permutation(wl, T, S):
    # the layer with shared experts, its permutation (routed rows, then one
    # T-row segment per shared expert) built inside the gate/up GEMM, against
    # the same layer with the separate permutation launch: bit for bit
    from w4a16_grouped_gemm_amd import ops
    say(f"shared layer, permutation in gemm {wl} T={T} S={S}")
    inp = make_layer_inputs(wl, T)
    sh = make_shared_weights(inp.workload, S)
    with ops.launch_override(perm_in_gemm_max_tokens=4096):
        fused = _forward(inp, sh)
    with ops.launch_override(perm_in_gemm_max_tokens=0):
        separate = _forward(inp, sh)
    assert np.array_equal(fused, separate)
    assert np.any(fused != 0)
