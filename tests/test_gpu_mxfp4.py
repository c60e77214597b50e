"""The W4A4 (MXFP4) variant on the GPU against the MXFP4 oracle.

- moe_mxfp4_quantize: bit-exact against the oracle's quantization (codes and
  scales), on random blocks across wide magnitudes with planted grid
  midpoints, signed zeros, all-zero blocks and subnormal maxima; and on
  every finite bf16 bit pattern under block maxima from the largest finite
  value down to the smallest subnormal (non-finite activations are outside
  the quantizer's contract: the two sides give such blocks different scales).
- moe_grouped_gemm_mxfp4: exact products and power-of-two block scales keep
  every sum exact in binary32 at these magnitudes, so RAW / W2 with f32
  output equal the oracle bit for bit (ragged experts, a gather through a
  permutation); SwiGLU and bf16 outputs within a bf16 rounding bound.
- moe_w4a4_forward: within the layer tolerance of the oracle's W4A4 layer
  (max |d| <= 2e-2 max |ref|, sum |d| / sum |ref| <= 5e-3), and equal to its
  entry points composed.
- The tiled MXFP4 code layout: moe_mxfp4_pack_weights equals the layout's
  definition (a byte permutation written out in numpy); the GEMMs on tiled
  codes equal the oracle exactly like the plain ones, and the layer on tiled
  codes equals the layer on plain codes bit for bit.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from helpers import assert_layer_close, bf16_dev, bf16_to_f64, say, tiled_runs, to_dev, to_np_u16
from w4a16_grouped_gemm_amd.inputs import bf16_bits, make_mxfp4_layer_inputs

pytestmark = pytest.mark.gpu


def _blocks(rng, rows, K):
    x = rng.standard_normal((rows, K)) * np.ldexp(1.0, rng.integers(-30, 31, size=(rows, K // 32)).repeat(32, 1))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for r in range(0, rows, 3):
        e = rng.integers(-20, 20)
        x[r, 0] = 4.0 * 2.0 ** e
        x[r, 1:8] = mids * 2.0 ** e * rng.choice([-1, 1], size=7)
    xb = bf16_bits(x.astype(np.float32))
    xb[1, :32] = 0                                         # an all-zero block
    xb[2, 32:64] = 0x8000                                  # a block of -0.0
    xb[4, :32] = rng.integers(0, 0x80, size=32)            # bf16 subnormals only
    return xb


@pytest.mark.parametrize("rows,K", [(7, 256), (300, 2048), (33, 7168)])
def test_quantize_bit_exact(rows, K):
    from w4a16_grouped_gemm_amd import ops
    import torch
    say(f"mxfp4 quantize rows={rows} K={K}")
    rng = np.random.default_rng(rows + K)
    xb = _blocks(rng, rows, K)
    codes, scales = ops.mxfp4_quantize(bf16_dev(xb))
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quantize(xb)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("amax_bits", [0x7F7F, 0x4730, 0x3FC0, 0x0080, 0x0041, 0x0001])
def test_quantize_every_bf16_value(amax_bits):
    # every bf16 bit pattern whose magnitude does not exceed the block maximum
    # (a finite value), 31 to a block after that maximum, so each block
    # exponent sees the whole range below it
    from w4a16_grouped_gemm_amd import ops
    import torch
    say(f"mxfp4 quantize every bf16 value, block maximum 0x{amax_bits:04x}")
    allv = np.arange(65536, dtype=np.uint32)
    vals = allv[(allv & 0x7FFF) <= amax_bits]
    nblk = -(-len(vals) // 31)
    body = np.zeros(nblk * 31, np.uint16)
    body[:len(vals)] = vals
    blocks = np.concatenate([np.full((nblk, 1), amax_bits, np.uint16), body.reshape(nblk, 31)], axis=1)
    K = 2048
    rows = -(-nblk // (K // 32))
    xb = np.zeros((rows * (K // 32), 32), np.uint16)
    xb[:nblk] = blocks
    xb = xb.reshape(rows, K)
    codes, scales = ops.mxfp4_quantize(bf16_dev(xb))
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quantize(xb)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def _mx(rng, shape, smin, smax):
    E, N, K = shape
    return (rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8),
            rng.integers(smin, smax + 1, size=(E, N, K // 32), dtype=np.uint8))


RAGGED = np.array([0, 1, 17, 40, 3, 0, 70, 16, 33, 128])


@pytest.mark.parametrize("kind,H,I", [(2, 2048, 768), (1, 2048, 768), (2, 256, 512), (1, 7168, 2048)])
@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("tiled", [False, True])
def test_gemm_exact(kind, H, I, gather, tiled):
    import torch
    from w4a16_grouped_gemm_amd import ops
    say(f"mxfp4 gemm exact kind={kind} H={H} I={I} gather={gather} tiled={tiled}")
    rng = np.random.default_rng(H + I + kind + gather)
    counts = RAGGED
    E = len(counts)
    N, K = (2 * I, H) if kind == ops.W13_RAW else (H, I)
    # scales 2^-1..2^0 (weights) and 2^0..2^1 (activations): products are
    # multiples of 2^-3 and |sums| <= 7168 * 36 * 2 < 2^21 units of 2^-3,
    # so every partial sum is exact in binary32 under any order
    wq, ws = _mx(rng, (E, N, K), 126, 127)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    k = 4
    T = (R + k - 1) // k + 1
    rows = T if gather else T * k
    aq, as_ = _mx(rng, (1, rows, K), 127, 128)
    aq, as_ = aq[0], as_[0]
    idx = None
    if gather:
        idx = np.full(T * k, -1, np.int32)
        idx[:R] = rng.permutation(T * k)[:R].astype(np.int32)
    wdev = to_dev(wq)
    if tiled:
        wdev = ops.mxfp4_pack_weights(kind, wdev)
    got = ops.grouped_gemm_mxfp4(kind, to_dev(aq), to_dev(as_), to_dev(offsets), wdev, to_dev(ws),
                                 num_tokens=T, top_k=k, a_row_index=None if idx is None else to_dev(idx),
                                 out_dtype=torch.float32,
                                 weight_layout=ops.WEIGHTS_TILED if tiled else ops.WEIGHTS_PLAIN)
    torch.cuda.synchronize()
    ref = oracle.grouped_gemm_mxfp4(oracle.RAW, aq, as_, offsets, wq, ws, rows=T * k, a_row_index=idx, top_k=k,
                                    out_f32=True)
    assert np.array_equal(got.cpu().numpy()[:R].view(np.uint32), ref[:R].view(np.uint32))


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("T", [16, 256, 2048])
def test_gemm_bf16_outputs(kind, T):
    # SwiGLU / down GEMM in bf16 against the oracle: within one bf16 rounding
    # of the exact value plus the transcendental's error
    import torch
    from w4a16_grouped_gemm_amd import ops
    say(f"mxfp4 gemm bf16 kind={kind} T={T}")
    inp = make_mxfp4_layer_inputs("qwen3_prefill" if T == 2048 else "qwen3_decode", T)
    k = inp.workload.top_k
    ids, _ = oracle.route(inp.logits, k)
    _, offsets, perm, _ = oracle.permute(ids, inp.workload.num_local_experts, 0)
    R = int(offsets[-1])
    sel_rows = np.unique(np.linspace(0, R - 1, min(R, 96)).astype(int))
    sel = np.zeros(T * k, np.uint8)
    sel[sel_rows] = 1
    if kind == 0:
        xq, xs = oracle.mx_quantize(inp.x)
        ref = oracle.grouped_gemm_mxfp4(0, xq, xs, offsets, inp.w13_q, inp.w13_s, rows=T * k, a_row_index=perm,
                                        top_k=k, row_sel=sel)
        got = ops.grouped_gemm_mxfp4(0, to_dev(xq), to_dev(xs), to_dev(offsets), to_dev(inp.w13_q),
                                     to_dev(inp.w13_s), num_tokens=T, top_k=k, a_row_index=to_dev(perm))
    else:
        rng = np.random.default_rng(T)
        h = bf16_bits((rng.standard_normal((T * k, inp.workload.inter)) * 0.05).astype(np.float32))
        hq, hs = oracle.mx_quantize(h)
        ref = oracle.grouped_gemm_mxfp4(1, hq, hs, offsets, inp.w2_q, inp.w2_s, rows=T * k, row_sel=sel)
        got = ops.grouped_gemm_mxfp4(1, to_dev(hq), to_dev(hs), to_dev(offsets), to_dev(inp.w2_q),
                                     to_dev(inp.w2_s), num_tokens=T, top_k=k)
    torch.cuda.synchronize()
    g = bf16_to_f64(to_np_u16(got)[sel_rows])
    r = bf16_to_f64(ref[sel_rows])
    bound = 2.0 ** -7 * np.abs(r) + 1e-3 * np.abs(r).max()
    assert np.all(np.abs(g - r) <= bound)


CASES = [("tiny", 16, None), ("qwen3_decode", 1, None), ("qwen3_decode", 16, None), ("qwen3_decode", 64, 32),
         ("qwen3_decode", 256, 24), ("qwen3_prefill", 2048, 16), ("ep_shard_decode", 16, 8),
         ("ep_shard_decode", 256, 8)]


def _w4a4_forward(inp):
    import torch
    from w4a16_grouped_gemm_amd import ops
    o = ops.moe_w4a4_forward(bf16_dev(inp.x), to_dev(inp.logits), to_dev(inp.w13_q), to_dev(inp.w13_s),
                             to_dev(inp.w2_q), to_dev(inp.w2_s), inp.workload.top_k,
                             expert_begin=inp.workload.expert_begin)
    torch.cuda.synchronize()
    return to_np_u16(o)


@pytest.mark.parametrize("wl,T,n", CASES)
def test_w4a4_layer_matches_oracle(wl, T, n):
    say(f"w4a4 layer {wl} T={T}")
    inp = make_mxfp4_layer_inputs(wl, T)
    got = _w4a4_forward(inp)
    sel = None
    rows = np.arange(T)
    if n is not None and T > n:
        rows = np.unique(np.linspace(0, T - 1, n).astype(int))
        sel = np.zeros(T, np.uint8)
        sel[rows] = 1
    w = inp.workload
    ref = oracle.layer_w4a4(inp.x, inp.logits, inp.w13_q, inp.w13_s, inp.w2_q, inp.w2_s, top_k=w.top_k,
                            expert_begin=w.expert_begin, tok_sel=sel)
    local = (ref["topk_ids"] >= w.expert_begin) & (ref["topk_ids"] < w.expert_begin + w.num_local_experts)
    none = ~local.any(axis=1)
    assert np.all(got[none] == 0)
    keep = rows[~none[rows]]
    if keep.size:
        assert_layer_close(got[keep], ref["out"][keep], f"w4a4 {wl} T={T}")


# the forward quantizes x inside its routing launch (the fused route +
# permutation up to 32 tokens, the routing kernel past that) and h inside the
# gate/up GEMM's epilogue where that GEMM stages activations in LDS (K <=
# 2048), else with the quantize kernel after it (the EP shard's K = 7168)
@pytest.mark.parametrize("wl,T", [("qwen3_decode", 1), ("qwen3_decode", 16), ("qwen3_decode", 256), ("tiny", 40),
                                  ("ep_shard_decode", 16), ("ep_shard_decode", 64)])
def test_w4a4_forward_equals_entry_points_composed(wl, T):
    import torch
    from w4a16_grouped_gemm_amd import ops
    say(f"w4a4 forward vs composed {wl} T={T}")
    inp = make_mxfp4_layer_inputs(wl, T)
    w = inp.workload
    ids, wt = ops.route(to_dev(inp.logits), w.top_k)
    _, offsets, perm, inv, _ = ops.permute(ids, w.num_local_experts, num_experts=w.num_experts,
                                           expert_begin=w.expert_begin)
    xq, xs = ops.mxfp4_quantize(bf16_dev(inp.x))
    h = ops.grouped_gemm_mxfp4(ops.W13_SWIGLU, xq, xs, offsets, to_dev(inp.w13_q), to_dev(inp.w13_s), num_tokens=T,
                               top_k=w.top_k, a_row_index=perm, num_experts=w.num_experts)
    torch.cuda.synchronize()
    R = int(offsets[-1].item())
    hq, hs = ops.mxfp4_quantize(h)
    y = ops.grouped_gemm_mxfp4(ops.W2, hq, hs, offsets, to_dev(inp.w2_q), to_dev(inp.w2_s), num_tokens=T,
                               top_k=w.top_k, num_experts=w.num_experts)
    composed = ops.finalize(y, wt, inv)
    torch.cuda.synchronize()
    assert R > 0
    assert np.array_equal(_w4a4_forward(inp), to_np_u16(composed))


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_mxfp4_pack_matches_layout_definition(kind):
    from w4a16_grouped_gemm_amd import ops
    say(f"mxfp4 pack layout kind={kind}")
    rng = np.random.default_rng(40 + kind)
    E, H, I = 3, 256, 384
    N, K = (H, I) if kind == ops.W2 else (2 * I, H)
    wq = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    got = ops.mxfp4_pack_weights(kind, to_dev(wq)).cpu().numpy()
    ref = tiled_runs(wq, 0 if kind == ops.W13_SWIGLU else 1, I)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("wl,T", [("qwen3_decode", 16), ("qwen3_decode", 256), ("ep_shard_decode", 64)])
def test_w4a4_forward_tiled_equals_plain(wl, T):
    import torch
    from w4a16_grouped_gemm_amd import ops
    say(f"w4a4 forward tiled vs plain {wl} T={T}")
    inp = make_mxfp4_layer_inputs(wl, T)
    w = inp.workload
    w13t = ops.mxfp4_pack_weights(ops.W13_SWIGLU, to_dev(inp.w13_q))
    w2t = ops.mxfp4_pack_weights(ops.W2, to_dev(inp.w2_q))
    o = ops.moe_w4a4_forward(bf16_dev(inp.x), to_dev(inp.logits), w13t, to_dev(inp.w13_s), w2t, to_dev(inp.w2_s),
                             w.top_k, expert_begin=w.expert_begin, weight_layout=ops.WEIGHTS_TILED)
    torch.cuda.synchronize()
    assert np.array_equal(to_np_u16(o), _w4a4_forward(inp))


# the W4A4 gate/up GEMM builds the permutation from the routing ids where it
# stages activations in LDS (K <= 2048): against the separate permutation
# launch (routing inside it up to 32 tokens), bit for bit; the EP shard (K =
# 7168) keeps the permutation launch either way
@pytest.mark.parametrize("wl,T", [("qwen3_decode", 20), ("qwen3_decode", 33), ("qwen3_decode", 256),
                                  ("qwen3_decode", 512), ("tiny", 200), ("ep_shard_decode", 64)])
def test_w4a4_permutation_in_gemm_equals_separate_permutation(wl, T):
    from w4a16_grouped_gemm_amd import ops
    say(f"w4a4 permutation in gemm {wl} T={T}")
    inp = make_mxfp4_layer_inputs(wl, T)
    with ops.launch_override(perm_in_gemm_max_tokens=4096):
        fused = _w4a4_forward(inp)
    with ops.launch_override(perm_in_gemm_max_tokens=0):
        separate = _w4a4_forward(inp)
    assert np.array_equal(fused, separate)
    assert np.any(fused != 0)


# (workload, T): the W4A4 small-batch path (routing and the quantization of x
# inside the gate/up GEMM, slot-ordered h and y, no permutation): one and
# two tokens, a token count between, the largest T, 8 experts of top-2 (two
# tokens sharing experts), 128 slots at top-16 (k16_e64), and the EP shard,
# whose K = 7168 keeps the general path either way
def _mx_small_inputs(wl, T):
    from w4a16_grouped_gemm_amd.inputs import Workload
    if wl == "k16_e64":
        wl = Workload("k16_e64", 21, 64, 64, 0, 16, 256, 256, (3, 8))
    return make_mxfp4_layer_inputs(wl, T)


@pytest.mark.parametrize("wl,T", [("qwen3_decode", 1), ("qwen3_decode", 2), ("qwen3_decode", 5),
                                  ("qwen3_decode", 16), ("tiny", 2), ("tiny", 7), ("k16_e64", 8),
                                  ("ep_shard_decode", 3)])
def test_w4a4_small_batch_path_equals_general_path(wl, T):
    from w4a16_grouped_gemm_amd import ops
    say(f"w4a4 small-batch path {wl} T={T}")
    inp = _mx_small_inputs(wl, T)
    fast = _w4a4_forward(inp)
    with ops.launch_override(decode_max_tokens=0):
        general = _w4a4_forward(inp)
    assert np.array_equal(fast, general)
    w = inp.workload
    ref = oracle.layer_w4a4(inp.x, inp.logits, inp.w13_q, inp.w13_s, inp.w2_q, inp.w2_s, top_k=w.top_k,
                            expert_begin=w.expert_begin)
    local = (ref["topk_ids"] >= w.expert_begin) & (ref["topk_ids"] < w.expert_begin + w.num_local_experts)
    none = ~local.any(axis=1)
    assert np.all(fast[none] == 0)
    if (~none).any():
        assert_layer_close(fast[~none], ref["out"][~none], f"w4a4 small {wl} T={T}")


@pytest.mark.parametrize("T", [1, 3])
def test_w4a4_small_batch_masked_experts(T):
    # -inf logits (masked experts) on the small-batch path: the experts
    # selected with weight 0 must not disturb the output
    say(f"w4a4 small-batch masked experts T={T}")
    inp = make_mxfp4_layer_inputs("qwen3_decode", T)
    lg = np.full_like(inp.logits, -np.inf)
    lg[:, :3] = inp.logits[:, :3]                        # 3 finite logits, 8 slots
    inp = dataclasses.replace(inp, logits=lg)
    got = _w4a4_forward(inp)
    ref = oracle.layer_w4a4(inp.x, inp.logits, inp.w13_q, inp.w13_s, inp.w2_q, inp.w2_s, top_k=8)
    assert np.all(np.isfinite(bf16_to_f64(got)))
    assert_layer_close(got, ref["out"], f"w4a4 small masked T={T}")
