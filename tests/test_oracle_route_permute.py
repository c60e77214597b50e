"""Pins of the oracle's routing and permutation (no GPU).

Routing (workload definition: softmax over all experts, keep the top-k,
renormalise; slot order = selection order, ties to the lower expert index) is
checked against a full stable sort per token, against closed forms and against
scipy's softmax. The permutation (InfiniLM PR #500 report, section 2.2: bucket
the routing ids into per-expert counts and a permutation; stable by token) is
checked against a brute-force stable sort of (expert, token) pairs and its
invariants.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
from w4a16_grouped_gemm_amd.inputs import make_layer_inputs, zipf_logits


def brute_topk(row, k):
    return sorted(range(len(row)), key=lambda e: (-float(row[e]), e))[:k]


@pytest.mark.parametrize("T,E,k", [(40, 8, 2), (30, 128, 8), (10, 256, 8), (5, 16, 16), (3, 4, 1)])
def test_route_ids_match_stable_sort(T, E, k):
    rng = np.random.default_rng(T * E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    # inject ties, duplicate maxima and signed zeros
    logits[0, : E // 2] = logits[0, 0]
    logits[1, :] = 0.0
    logits[1, ::3] = -0.0
    if T > 2:
        logits[2, 1] = logits[2, 3] = logits[2].max() + 1
    ids, w = oracle.route(logits, k)
    for t in range(T):
        assert list(ids[t]) == brute_topk(logits[t], k)
        assert len(set(ids[t])) == k
        keys = logits[t, ids[t]]
        assert np.all(keys[:-1] >= keys[1:])


def test_route_equal_logits_closed_form():
    for k in (1, 2, 4, 8):
        ids, w = oracle.route(np.full((3, 64), 0.75, np.float32), k)
        assert np.array_equal(ids, np.tile(np.arange(k), (3, 1)))
        assert np.all(w == np.float32(1.0 / k))


def test_route_top2_closed_form():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((200, 8)).astype(np.float32)
    ids, w = oracle.route(logits, 2)
    for t in range(200):
        d = float(logits[t, ids[t, 0]]) - float(logits[t, ids[t, 1]])
        w0 = 1.0 / (1.0 + np.exp(-d))
        assert abs(float(w[t, 0]) - w0) <= 2.0 ** -24 * w0 * 1.01
        assert abs(float(w[t, 1]) - (1 - w0)) <= 2.0 ** -24 * max(1 - w0, 1e-30) * 1.01 + 1e-300


def test_route_weights_match_scipy_softmax_renormalised():
    rng = np.random.default_rng(6)
    for E, k in [(128, 8), (256, 8), (8, 2)]:
        logits = rng.standard_normal((50, E)).astype(np.float32)
        ids, w = oracle.route(logits, k)
        p = softmax(logits.astype(np.float64), axis=1)
        for t in range(50):
            sel = p[t, ids[t]]
            ref = sel / sel.sum()
            assert np.all(np.abs(w[t] - ref) <= 2.0 ** -24 * ref * 1.01)
            assert abs(float(w[t].astype(np.float64).sum()) - 1.0) <= k * 2.0 ** -24


def brute_permute(ids, E_loc, begin):
    T, k = ids.shape
    pairs = [(int(ids[t, j]) - begin, t, j) for t in range(T) for j in range(k)
             if 0 <= ids[t, j] - begin < E_loc]
    pairs.sort(key=lambda p: (p[0], p[1]))
    return [t * k + j for (_, t, j) in pairs]


def check_permutation(ids, E_loc, begin, counts, offsets, perm, inv):
    T, k = ids.shape
    local = (ids >= begin) & (ids < begin + E_loc)
    R = int(local.sum())
    assert counts.sum() == R
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    for e in range(E_loc):
        assert counts[e] == int((ids == begin + e).sum())
    assert sorted(perm[:R].tolist()) == sorted((np.flatnonzero(local.reshape(-1))).tolist())
    assert np.all(perm[R:] == -1)
    flat_inv = inv.reshape(-1)
    for r in range(R):
        assert flat_inv[perm[r]] == r
    assert np.all(flat_inv[~local.reshape(-1)] == -1)
    for e in range(E_loc):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(ids.reshape(-1)[seg] == begin + e)
        assert np.all(np.diff(seg // k) > 0)   # tokens strictly ascending (experts distinct per token)
    assert perm[:R].tolist() == brute_permute(ids, E_loc, begin)


@pytest.mark.parametrize("wl,T,begin,E_loc", [("tiny", 16, 0, 8), ("qwen3_decode", 64, 0, 128),
                                               ("ep_shard_decode", 64, 0, 32),
                                               ("ep_shard_decode", 16, 100, 32)])
def test_permute_invariants_and_brute_force(wl, T, begin, E_loc):
    inp = make_layer_inputs(wl, T)
    ids, _ = oracle.route(inp.logits, inp.workload.top_k)
    c, o, p, inv = oracle.permute(ids, E_loc, begin)
    check_permutation(ids, E_loc, begin, c, o, p, inv)


def test_permute_zipf_skew():
    rng = np.random.default_rng(1)
    ids, _ = oracle.route(zipf_logits(rng, 512, 128), 8)
    c, o, p, inv = oracle.permute(ids, 128, 0)
    check_permutation(ids, 128, 0, c, o, p, inv)
    assert c.max() > 8 * c.mean()       # skewed load
    assert c.max() <= 512               # one slot per token per expert


def test_permute_empty_and_no_local():
    ids = np.zeros((0, 4), np.int32)
    c, o, p, inv = oracle.permute(ids, 8, 0)
    assert c.sum() == 0 and o[-1] == 0
    ids = np.array([[40, 41], [42, 43]], np.int32)
    c, o, p, inv = oracle.permute(ids, 8, 0)
    assert c.sum() == 0 and np.all(p == -1) and np.all(inv == -1)
