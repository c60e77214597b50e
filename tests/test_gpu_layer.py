"""The whole layer on the GPU (moe_w4a16_forward) vs the oracle.

Tolerance (floating point, bitwise parity is not expected for the layer):
max |gpu - ref| <= 2e-2 * max |ref| and sum|gpu - ref| / sum|ref| <= 5e-3.
At full sizes the oracle computes a seeded sample of tokens (rows are
independent, so the sample is exact for those tokens).
"""
import dataclasses

import numpy as np
import pytest

import oracle
from helpers import assert_layer_close, bf16_dev, bf16_to_f64, say, to_dev, to_np_u16
from w4a16_grouped_gemm_amd.inputs import make_layer_inputs

pytestmark = pytest.mark.gpu


def _forward(inp, out=None, tiled=False):
    import torch
    from w4a16_grouped_gemm_amd import ops
    w13, w2 = to_dev(inp.w13_q), to_dev(inp.w2_q)
    if tiled:
        w13, w2 = ops.pack_weights(ops.W13_SWIGLU, w13), ops.pack_weights(ops.W2, w2)
    o = ops.moe_w4a16_forward(bf16_dev(inp.x), to_dev(inp.logits), w13, bf16_dev(inp.s13),
                              w2, bf16_dev(inp.s2), inp.workload.top_k, out=out,
                              expert_begin=inp.workload.expert_begin,
                              weight_layout=ops.WEIGHTS_TILED if tiled else ops.WEIGHTS_PLAIN)
    torch.cuda.synchronize()
    return to_np_u16(o)


def _sample(T, n):
    if T <= n:
        return None
    idx = np.unique(np.linspace(0, T - 1, n).astype(int))
    sel = np.zeros(T, np.uint8)
    sel[idx] = 1
    return sel


CASES = [("tiny", 16, 64), ("qwen3_decode", 1, 64), ("qwen3_decode", 16, 64), ("qwen3_decode", 64, 64),
         ("qwen3_decode", 256, 24), ("qwen3_prefill", 2048, 16), ("ep_shard_decode", 1, 64),
         ("ep_shard_decode", 16, 16), ("ep_shard_decode", 64, 12), ("ep_shard_decode", 256, 12)]


# the code layout each workload is timed with (tiled codes) as well as the
# plain one; the tiled prefill layer takes the tile kernel in both GEMMs
TILED_CASES = [("qwen3_prefill", 2048, 16), ("ep_shard_decode", 1, 64), ("ep_shard_decode", 16, 16),
               ("ep_shard_decode", 64, 12), ("ep_shard_decode", 256, 12), ("qwen3_decode", 1, 64),
               ("qwen3_decode", 16, 64), ("qwen3_decode", 64, 64), ("qwen3_decode", 256, 24)]


@pytest.mark.parametrize("wl,T,n", CASES)
def test_layer_matches_oracle(wl, T, n):
    _layer_vs_oracle(wl, T, n, tiled=False)


@pytest.mark.parametrize("wl,T,n", TILED_CASES)
def test_tiled_layer_matches_oracle(wl, T, n):
    _layer_vs_oracle(wl, T, n, tiled=True)


def _layer_vs_oracle(wl, T, n, tiled):
    say(f"layer {wl} T={T} sample={n} tiled={tiled}")
    inp = make_layer_inputs(wl, T)
    got = _forward(inp, tiled=tiled)
    sel = _sample(T, n)
    ref = oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=inp.workload.top_k,
                       expert_begin=inp.workload.expert_begin, tok_sel=sel)
    rows = np.arange(T) if sel is None else np.flatnonzero(sel)
    local = (ref["topk_ids"] >= inp.workload.expert_begin) & \
            (ref["topk_ids"] < inp.workload.expert_begin + inp.workload.num_local_experts)
    none = ~local.any(axis=1)
    assert np.all(got[none] == 0), "tokens with no local slot must be +0.0"
    if (~none[rows]).any():
        assert_layer_close(got[rows], ref["out"][rows], f"{wl} T={T}")


def test_layer_deterministic():
    say("layer determinism qwen3_decode T=64")
    inp = make_layer_inputs("qwen3_decode", 64)
    a = _forward(inp)
    b = _forward(inp)
    assert np.array_equal(a, b)


def test_zero_tokens_is_noop_and_errors_touch_nothing():
    import torch
    from w4a16_grouped_gemm_amd import ops
    say("layer T=0 and error paths")
    inp = make_layer_inputs("tiny", 4)
    empty = make_layer_inputs("tiny", 0)
    out = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    ops.moe_w4a16_forward(bf16_dev(empty.x), to_dev(empty.logits), to_dev(inp.w13_q), bf16_dev(inp.s13),
                          to_dev(inp.w2_q), bf16_dev(inp.s2), 2, out=out)
    sentinel = torch.full((4, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        ops.moe_w4a16_forward(bf16_dev(inp.x), to_dev(inp.logits), to_dev(inp.w13_q), bf16_dev(inp.s13),
                              to_dev(inp.w2_q), bf16_dev(inp.s2), 9, out=sentinel)    # k > E
    with pytest.raises(ValueError):
        ops.moe_w4a16_forward(bf16_dev(inp.x), to_dev(inp.logits), to_dev(inp.w13_q), bf16_dev(inp.s13),
                              to_dev(inp.w2_q), bf16_dev(inp.s2), 2, out=sentinel,
                              workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())


@pytest.mark.parametrize("wl,T", [("tiny", 16), ("qwen3_decode", 1), ("qwen3_decode", 256),
                                  ("ep_shard_decode", 64)])
def test_tiled_layout_gives_identical_layer(wl, T):
    # the tiled codes feed the same MFMA sequence in the same order: the
    # layer output must match the plain-layout run bit for bit
    say(f"layer tiled vs plain {wl} T={T}")
    inp = make_layer_inputs(wl, T)
    assert np.array_equal(_forward(inp, tiled=True), _forward(inp))


@pytest.mark.parametrize("wl,T", [("tiny", 16), ("tiny", 3), ("qwen3_decode", 1), ("qwen3_decode", 4),
                                  ("qwen3_decode", 5), ("qwen3_decode", 16), ("qwen3_decode", 17),
                                  ("qwen3_decode", 64), ("qwen3_decode", 256), ("qwen3_decode", 300),
                                  ("ep_shard_decode", 1), ("ep_shard_decode", 4), ("ep_shard_decode", 16),
                                  ("ep_shard_decode", 256)])
def test_forward_equals_the_entry_points_composed(wl, T):
    # forward routes and permutes in one workgroup while the tokens are few
    # and in two launches otherwise; either way it must give, bit for bit,
    # what moe_route -> moe_permute -> two grouped GEMMs -> moe_finalize give
    import torch
    from w4a16_grouped_gemm_amd import ops
    say(f"layer forward vs composed entry points {wl} T={T}")
    inp = make_layer_inputs(wl, T)
    w = inp.workload
    x, logits = bf16_dev(inp.x), to_dev(inp.logits)
    w13, s13, w2, s2 = to_dev(inp.w13_q), bf16_dev(inp.s13), to_dev(inp.w2_q), bf16_dev(inp.s2)
    ids, wt = ops.route(logits, w.top_k)
    _, offsets, perm, inv, _ = ops.permute(ids, w.num_local_experts, num_experts=w.num_experts,
                                           expert_begin=w.expert_begin)
    h = ops.grouped_gemm_w4a16(ops.W13_SWIGLU, x, offsets, w13, s13, num_tokens=T, top_k=w.top_k,
                               a_row_index=perm, num_experts=w.num_experts)
    y = ops.grouped_gemm_w4a16(ops.W2, h, offsets, w2, s2, num_tokens=T, top_k=w.top_k,
                               num_experts=w.num_experts)
    composed = ops.finalize(y, wt, inv)
    torch.cuda.synchronize()
    assert np.array_equal(_forward(inp), to_np_u16(composed))


# (workload, T): the general path where the gate/up GEMM builds the
# permutation from the routing ids itself, against the permutation launch
# (routing inside it up to 32 tokens, T = 20 and 24 here): the largest T it
# takes, token counts that are not a multiple of 32 (partial bitmap words),
# slots of non-local experts (EP shard), top-2 of 8 experts (one and two
# tiles per wave), top-16 (k16_e64), two subtiles per chunk (256 and 512)
PERM_IN_GEMM = [("qwen3_decode", 20), ("qwen3_decode", 33), ("qwen3_decode", 100), ("qwen3_decode", 256),
                ("qwen3_decode", 512), ("ep_shard_decode", 24), ("ep_shard_decode", 64), ("ep_shard_decode", 256),
                ("tiny", 200), ("k16_e64", 40)]


@pytest.mark.parametrize("wl,T", PERM_IN_GEMM)
def test_permutation_in_gemm_equals_separate_permutation(wl, T):
    # the layer with the permutation built inside the gate/up GEMM against
    # the layer with the separate permutation launch: bit for bit (the down
    # GEMM and the finalize read the tables the GEMM stored)
    from w4a16_grouped_gemm_amd import ops
    say(f"permutation in gemm {wl} T={T}")
    inp = _small_inputs(wl, T)
    with ops.launch_override(perm_in_gemm_max_tokens=4096):
        fused = _forward(inp)
    with ops.launch_override(perm_in_gemm_max_tokens=0):
        separate = _forward(inp)
    assert np.array_equal(fused, separate)
    assert np.any(fused != 0)


@pytest.mark.parametrize("wl,T", [("tiny", 16), ("qwen3_decode", 16), ("qwen3_decode", 64)])
def test_masked_experts(wl, T):
    # router logits of -inf (masked experts), and tokens with fewer finite
    # logits than slots: the selected masked experts get weight exactly 0, so
    # every output is finite and matches the oracle
    say(f"layer masked experts {wl} T={T}")
    inp = make_layer_inputs(wl, T)
    rng = np.random.default_rng(T)
    lg = inp.logits.copy()
    E, k = lg.shape[1], inp.workload.top_k
    lg[:, rng.permutation(E)[: E // 4]] = -np.inf               # a quarter of the experts masked for all
    for t in range(0, T, 3):                                     # fewer finite logits than slots
        keep = rng.permutation(E)[: max(1, k // 2)]
        row = np.full(E, -np.inf, np.float32)
        row[keep] = lg[t, keep]
        row[keep[~np.isfinite(row[keep])]] = 0.25
        lg[t] = row
    inp = dataclasses.replace(inp, logits=lg)
    got = _forward(inp)
    ref = oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=k)
    assert np.all(np.isfinite(bf16_to_f64(got)))
    assert_layer_close(got, ref["out"], f"masked {wl} T={T}")


def test_two_streams_default_workspaces():
    # two forwards in flight on two streams, each with the binding's default
    # workspace: the workspaces are per stream, so neither run disturbs the other
    import torch
    from w4a16_grouped_gemm_amd import ops
    say("layer on two streams")
    a = make_layer_inputs("qwen3_decode", 64)
    b = make_layer_inputs("qwen3_decode", 16)
    dev = {}
    for name, inp in (("a", a), ("b", b)):
        dev[name] = (bf16_dev(inp.x), to_dev(inp.logits), to_dev(inp.w13_q), bf16_dev(inp.s13),
                     to_dev(inp.w2_q), bf16_dev(inp.s2))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = {"a": [], "b": []}
    for _ in range(4):
        with torch.cuda.stream(s1):
            outs["a"].append(ops.moe_w4a16_forward(*dev["a"], 8))
        with torch.cuda.stream(s2):
            outs["b"].append(ops.moe_w4a16_forward(*dev["b"], 8))
    torch.cuda.synchronize()
    for name, inp in (("a", a), ("b", b)):
        ref = oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=8)["out"]
        first = to_np_u16(outs[name][0])
        assert_layer_close(first, ref, f"stream {name}")
        for o in outs[name][1:]:
            assert np.array_equal(to_np_u16(o), first)


# (workload, T): the small-batch path's regimes -- down GEMM with the combine
# (T <= 2; forced up to 16 below), down GEMM then the finalize, both kernel
# families (split-K on the EP shard at 1 token and on the tiny layer,
# streaming elsewhere), and the edges: 128 slots
# (T = 8 at k = 16), a token with no local slot (EP shard), 2 tokens sharing
# experts (tiny: 8 experts, top-2)
SMALL = [("qwen3_decode", 1), ("qwen3_decode", 2), ("qwen3_decode", 4), ("qwen3_decode", 5),
         ("qwen3_decode", 8), ("qwen3_decode", 16), ("ep_shard_decode", 1), ("ep_shard_decode", 3),
         ("ep_shard_decode", 16), ("tiny", 2), ("tiny", 7), ("k16_e64", 8), ("k16_e64", 3)]


def _small_inputs(wl, T):
    from w4a16_grouped_gemm_amd.inputs import Workload
    if wl == "k16_e64":
        wl = Workload("k16_e64", 21, 64, 64, 0, 16, 256, 256, (3, 8))
    return make_layer_inputs(wl, T)


@pytest.mark.parametrize("wl,T", SMALL)
def test_small_batch_path_equals_general_path(wl, T):
    # the small-batch path (routing inside the gate/up GEMM, no permutation)
    # against the general path (route, permute, grouped GEMMs, finalize) with
    # the small-batch path switched off, with and without the fused combine:
    # bit for bit, and within the tolerance of the oracle
    from w4a16_grouped_gemm_amd import ops
    say(f"small-batch path {wl} T={T}")
    inp = _small_inputs(wl, T)
    fast = _forward(inp)
    with ops.launch_override(decode_combine_max_tokens=0):
        no_combine = _forward(inp)
    with ops.launch_override(decode_combine_max_tokens=16):
        combine = _forward(inp)                          # the fused combine wherever it fits
    with ops.launch_override(decode_max_tokens=0):
        general = _forward(inp)
    assert np.array_equal(fast, general)
    assert np.array_equal(no_combine, general)
    assert np.array_equal(combine, general)
    ref = oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=inp.workload.top_k,
                       expert_begin=inp.workload.expert_begin)
    local = (ref["topk_ids"] >= inp.workload.expert_begin) & \
            (ref["topk_ids"] < inp.workload.expert_begin + inp.workload.num_local_experts)
    none = ~local.any(axis=1)
    assert np.all(fast[none] == 0)
    if (~none).any():
        assert_layer_close(fast[~none], ref["out"][~none], f"small {wl} T={T}")


@pytest.mark.parametrize("T", [1, 3])
def test_small_batch_masked_experts(T):
    # -inf logits on the small-batch path (routing inside the GEMM): masked
    # experts selected with weight 0 must not disturb the output
    say(f"small-batch masked experts T={T}")
    inp = make_layer_inputs("qwen3_decode", T)
    lg = np.full_like(inp.logits, -np.inf)
    lg[:, :3] = inp.logits[:, :3]                        # 3 finite logits, 8 slots
    inp = dataclasses.replace(inp, logits=lg)
    got = _forward(inp)
    ref = oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=8)
    assert np.all(np.isfinite(bf16_to_f64(got)))
    assert_layer_close(got, ref["out"], f"small masked T={T}")


def test_small_batch_tiled_equals_plain():
    say("small-batch path tiled vs plain")
    for wl, T in (("qwen3_decode", 1), ("qwen3_decode", 12), ("ep_shard_decode", 4)):
        inp = make_layer_inputs(wl, T)
        assert np.array_equal(_forward(inp, tiled=True), _forward(inp)), (wl, T)
