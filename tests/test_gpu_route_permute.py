"""GPU routing and permutation vs the oracle: ids, counts, offsets, perm, inv_perm bit-exact.

Routing weights are not in the bit-exact set (fp32 exp vs the oracle's fp64
softmax); they must lie within the forward error bound derived below and
sum to 1.
"""
import numpy as np
import pytest

import oracle
from helpers import bf16_dev, say, to_dev, to_np_u16
from w4a16_grouped_gemm_amd.inputs import WORKLOADS, make_layer_inputs

pytestmark = pytest.mark.gpu

CASES = [("tiny", 16), ("qwen3_decode", 1), ("qwen3_decode", 16), ("qwen3_decode", 64),
         ("qwen3_decode", 256), ("qwen3_prefill", 2048), ("ep_shard_decode", 1),
         ("ep_shard_decode", 16), ("ep_shard_decode", 64), ("ep_shard_decode", 256)]


def _logits(wl, T):
    return make_layer_inputs(wl, T, weights=False).logits


@pytest.mark.parametrize("wl,T", CASES)
def test_route_matches_oracle(wl, T):
    import torch
    from w4a16_grouped_gemm_amd import ops
    say(f"route {wl} T={T}")
    w = WORKLOADS[wl]
    logits = _logits(wl, T)
    ref_ids, ref_w = oracle.route(logits, w.top_k)
    ids, wt = ops.route(to_dev(logits), w.top_k)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    got_w = wt.cpu().numpy()
    # Forward error of the fp32 path against the exact weight, with u = 2^-24:
    # each exp term carries <= 2u (1 ulp of expf) + u (the residual fma);
    # the k-term sum adds (k-1)u; the divide adds u; the oracle's single
    # rounding adds u. Relative error <= 2*3u + (k-1)u + u + u = (k+7)u, and
    # one ulp of a binary32 value is at least u relative, so <= k+7 ulp.
    ulps = np.abs(got_w.astype(np.float64) - ref_w) / np.spacing(ref_w).astype(np.float64)
    say(f"  max weight error {ulps.max():.1f} ulp")
    assert ulps.max() <= w.top_k + 7
    assert np.all(np.abs(got_w.astype(np.float64).sum(axis=1) - 1.0) <= w.top_k * 2.0 ** -23)


def test_route_ties_and_signed_zeros():
    import torch
    from w4a16_grouped_gemm_amd import ops
    say("route ties")
    rng = np.random.default_rng(9)
    for E, k in [(8, 2), (128, 8), (256, 8), (1024, 16), (64, 1)]:
        logits = rng.standard_normal((64, E)).astype(np.float32)
        logits[0] = 0.5                                  # all equal
        logits[1] = 0.0
        logits[1, ::2] = -0.0                            # mixed signed zeros
        logits[2, : E // 2] = 3.0                        # many equal maxima
        logits[3] = np.round(logits[3])                  # many exact duplicates
        logits[4] = -np.inf
        logits[4, E - 1] = 1.0
        # fewer finite logits than slots: the rest are masked experts (-inf)
        logits[5] = -np.inf
        logits[5, rng.permutation(E)[: max(1, k // 2)]] = rng.standard_normal(max(1, k // 2))
        # l_q - l_0 overflows binary32 (to -inf) for the negative slots
        logits[6] = rng.choice(np.float32([-3e38, 3e38, -2.5e38]), size=E)
        ref_ids, ref_w = oracle.route(logits, k)
        ids, wt = ops.route(to_dev(logits), k)
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), ref_ids), (E, k)
        # weights: finite everywhere, exactly 0 where the exact weight is 0
        # (exp of a -inf difference), else within the k+7 ulp bound below
        got_w = wt.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got_w)), (E, k)
        zero = ref_w == 0
        assert np.all(got_w[zero] == 0.0), (E, k)
        ulps = np.abs(got_w[~zero] - ref_w[~zero]) / np.spacing(ref_w[~zero]).astype(np.float64)
        assert ulps.max() <= k + 7, (E, k, ulps.max())
        assert np.all(np.abs(got_w[4] - np.eye(k)[0]) == 0.0), (E, k)


@pytest.mark.parametrize("wl,T", CASES)
def test_permute_matches_oracle(wl, T):
    import torch
    from w4a16_grouped_gemm_amd import ops
    say(f"permute {wl} T={T}")
    w = WORKLOADS[wl]
    inp = make_layer_inputs(wl, T, weights=False)
    logits = inp.logits
    ids, _ = oracle.route(logits, w.top_k)
    c, o, p, inv = oracle.permute(ids, w.num_local_experts, w.expert_begin)
    x = bf16_dev(inp.x)
    gc, go, gp, ginv, xp = ops.permute(to_dev(ids), w.num_local_experts, num_experts=w.num_experts,
                                       expert_begin=w.expert_begin, x=x)
    torch.cuda.synchronize()
    assert np.array_equal(gc.cpu().numpy(), c)
    assert np.array_equal(go.cpu().numpy(), o)
    assert np.array_equal(gp.cpu().numpy(), p)
    assert np.array_equal(ginv.cpu().numpy(), inv)
    R = int(o[-1])
    assert np.array_equal(to_np_u16(xp)[:R], inp.x[p[:R] // w.top_k])


@pytest.mark.parametrize("begin,E_loc,E_g", [(0, 8, 8), (100, 32, 256), (224, 32, 256), (5, 1, 16)])
def test_permute_local_window_and_chunks(begin, E_loc, E_g):
    import torch
    from w4a16_grouped_gemm_amd import ops
    say(f"permute window begin={begin} E_loc={E_loc}")
    rng = np.random.default_rng(begin + E_loc)
    T, k = 3000, min(8, E_g)       # several 1024-token scatter chunks
    logits = rng.standard_normal((T, E_g)).astype(np.float32)
    ids, _ = oracle.route(logits, k)
    c, o, p, inv = oracle.permute(ids, E_loc, begin)
    gc, go, gp, ginv, _ = ops.permute(to_dev(ids), E_loc, num_experts=E_g, expert_begin=begin)
    torch.cuda.synchronize()
    assert np.array_equal(gc.cpu().numpy(), c) and np.array_equal(go.cpu().numpy(), o)
    assert np.array_equal(gp.cpu().numpy(), p) and np.array_equal(ginv.cpu().numpy(), inv)


# (T, E_g, E_loc, expert_begin, k): one workgroup over two bitmap chunks
# (1024 experts leave 128-token chunks); just past the token count where the
# permutation splits into ranges; one local expert; ranges over a window of
# 1024 experts; and the 64-range cap with ranges too long to stage their ids
# in LDS.
RANGES = [(200, 1024, 1024, 0, 16), (385, 128, 128, 0, 8), (513, 128, 128, 0, 8), (1000, 16, 1, 5, 2),
          (5000, 1024, 512, 256, 16),
          (160000, 64, 32, 16, 16)]


@pytest.mark.parametrize("T,E_g,E_loc,begin,k", RANGES)
def test_permute_token_ranges(T, E_g, E_loc, begin, k):
    import torch
    from w4a16_grouped_gemm_amd import ops
    say(f"permute ranges T={T} E_g={E_g} E_loc={E_loc} begin={begin} k={k}")
    rng = np.random.default_rng(T + E_g)
    # k distinct experts per token, skewed so some experts get far more slots
    keys = rng.random((T, E_g)) * np.linspace(1.0, 3.0, E_g)
    ids = np.argsort(keys, axis=1)[:, :k].astype(np.int32)
    c, o, p, inv = oracle.permute(ids, E_loc, begin)
    gc, go, gp, ginv, _ = ops.permute(to_dev(ids), E_loc, num_experts=E_g, expert_begin=begin)
    torch.cuda.synchronize()
    assert np.array_equal(gc.cpu().numpy(), c) and np.array_equal(go.cpu().numpy(), o)
    assert np.array_equal(gp.cpu().numpy(), p) and np.array_equal(ginv.cpu().numpy(), inv)
