"""Pins of the oracle's grouped GEMM, SwiGLU and whole layer (no GPU).

- The int4 decode against a hand-decoded golden byte string.
- One-hot activations read single dequantised weight columns back exactly
  (pins nibble order, scale-group index, the gate/up split, expert offsets
  and the gather through the permutation).
- Integer-valued activations with power-of-two scales make every partial sum
  exact, so the result must equal numpy's int64 matmul exactly.
- One expert is a dense W4A16 GEMM: fp64 numpy matmul on dequantised weights.
- SwiGLU against scipy.special.expit at known gate/up values.
- The permuted layer against the naive per-(token, slot) loop, bit for bit
  (InfiniLM PR #500 report, section 2.2 vs its naive per-token MoE baseline).
"""
import json
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle import exact
from w4a16_grouped_gemm_amd.inputs import (bf16_bits, bf16_values, make_layer_inputs, pack_int4,
                                           unpack_int4)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_int4_golden_decode():
    g = json.load(open(os.path.join(GOLD, "int4_decode.json")))
    K = 2 * len(g["bytes"])
    Kp = 128
    wq = np.zeros((1, 1, Kp // 2), np.uint8)
    wq[0, 0, : len(g["bytes"])] = g["bytes"]
    s = np.full((1, 1, 1), 0x3F80, np.uint16)             # scale 1.0
    x = bf16_bits(np.eye(Kp, dtype=np.float32))          # row k = e_k
    offsets = np.array([0, Kp], np.int32)
    c = oracle.grouped_gemm(oracle.RAW, x, offsets, wq, s, rows=Kp, out_f32=True)
    assert c[:K, 0].astype(int).tolist() == g["codes"]
    assert np.array_equal(unpack_int4(wq)[0, 0, :K], np.array(g["codes"], np.int8))
    assert np.array_equal(pack_int4(np.array(g["codes"]))[None, None, :], wq[..., : len(g["bytes"])])


def test_one_hot_reads_weight_columns():
    rng = np.random.default_rng(21)
    E, N, K = 3, 48, 384
    q = rng.integers(-8, 8, size=(E, N, K)).astype(np.int8)
    sexp = rng.integers(-9, -3, size=(E, N, K // 128))
    s = bf16_bits((2.0 ** sexp).astype(np.float32))
    wq = pack_int4(q)
    # tokens: each probes one k; rows grouped by expert through a gather
    ks = rng.integers(0, K, size=20)
    x = bf16_bits(np.eye(K, dtype=np.float32)[ks])
    counts = np.array([7, 0, 13])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    top_k = 2
    perm = (rng.permutation(20) * top_k + 1).astype(np.int32)   # token = perm // top_k
    c = oracle.grouped_gemm(oracle.RAW, x, offsets, wq, s, rows=20, a_row_index=perm, top_k=top_k,
                            out_f32=True)
    for e in range(E):
        for r in range(offsets[e], offsets[e + 1]):
            k = ks[perm[r] // top_k]
            want = q[e, :, k].astype(np.float64) * 2.0 ** sexp[e, :, k // 128]
            assert np.array_equal(c[r].astype(np.float64), want)


@pytest.mark.parametrize("E,N,K", [(2, 64, 2048), (1, 32, 768), (4, 16, 7168)])
def test_integer_exact(E, N, K):
    rng = np.random.default_rng(E * N + K)
    q = rng.integers(-8, 8, size=(E, N, K)).astype(np.int8)
    s = np.full((E, N, K // 128), bf16_bits(np.float32(2.0 ** -6)), np.uint16)
    rows_per = rng.integers(0, 9, size=E)
    offsets = np.concatenate([[0], np.cumsum(rows_per)]).astype(np.int32)
    R = int(offsets[-1])
    xi = rng.integers(-2, 3, size=(R, K))
    x = bf16_bits(xi.astype(np.float32))
    c = oracle.grouped_gemm(oracle.RAW, x, offsets, pack_int4(q), s, rows=R, out_f32=True)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        want = (xi[r0:r1].astype(np.int64) @ q[e].T.astype(np.int64)).astype(np.float64) * 2.0 ** -6
        assert np.array_equal(c[r0:r1].astype(np.float64), want)


def test_single_expert_is_dense_gemm():
    rng = np.random.default_rng(31)
    N, K, R = 96, 1024, 24
    wq = rng.integers(0, 256, size=(1, N, K // 2), dtype=np.uint8)
    s = bf16_bits(rng.uniform(0.005, 0.02, size=(1, N, K // 128)).astype(np.float32))
    x = bf16_bits(rng.standard_normal((R, K)).astype(np.float32))
    W = unpack_int4(wq)[0].astype(np.float64) * np.repeat(bf16_values(s[0]).astype(np.float64), 128, axis=1)
    ref = bf16_values(x).astype(np.float64) @ W.T
    c = oracle.grouped_gemm(oracle.RAW, x, np.array([0, R], np.int32), wq, s, rows=R, out_f32=True)
    assert np.all(np.abs(c - ref) <= np.abs(ref) * 2.0 ** -23 + 1e-30)
    cb = oracle.grouped_gemm(oracle.W2, x, np.array([0, R], np.int32), wq, s, rows=R)
    assert np.all(np.abs(bf16_values(cb) - ref) <= np.abs(ref) * 2.0 ** -8)


def test_swiglu_at_known_points():
    # one expert, I features; token r probes k = 0 with value 1.0 so that
    # g_n = q_g[n] * s_g, u_n = q_u[n] * s_u exactly.
    rng = np.random.default_rng(41)
    I, H = 128, 128
    q = rng.integers(-8, 8, size=(1, 2 * I, H)).astype(np.int8)
    s = bf16_bits(rng.uniform(0.05, 1.5, size=(1, 2 * I, 1)).astype(np.float32))
    x = bf16_bits(np.eye(H, dtype=np.float32)[:1])
    h = oracle.grouped_gemm(oracle.W13_SWIGLU, x, np.array([0, 1], np.int32), pack_int4(q), s, rows=1)
    sv = bf16_values(s[0, :, 0]).astype(np.float64)
    g = q[0, :I, 0] * sv[:I]
    u = q[0, I:, 0] * sv[I:]
    ref = g * expit(g) * u
    got = bf16_values(h[0]).astype(np.float64)
    for n in range(I):
        want = bf16_values(np.array([exact.bf16_bits(float(ref[n]))], np.uint16))[0]
        # one bf16 rounding of the same real number; exp implementations may
        # differ in the last fp64 bit, which can only matter at a tie
        assert got[n] == want or abs(got[n] - want) <= abs(want) * 2.0 ** -7
        if g[n] == 0:
            assert got[n] == 0


@pytest.mark.parametrize("wl,T,begin,E_loc", [("tiny", 16, 0, 8), ("tiny", 16, 2, 4), ("tiny", 5, 6, 2)])
def test_layer_equals_per_token_loop(wl, T, begin, E_loc):
    inp = make_layer_inputs(wl, T)
    w13, s13 = inp.w13_q[:E_loc], inp.s13[:E_loc]
    w2, s2 = inp.w2_q[:E_loc], inp.s2[:E_loc]
    r = oracle.layer(inp.x, inp.logits, w13, s13, w2, s2, top_k=inp.workload.top_k, expert_begin=begin)
    bf = oracle.layer_bruteforce(inp.x, r["topk_ids"], r["topk_w"], w13, s13, w2, s2, expert_begin=begin)
    assert np.array_equal(r["out"], bf)
    local = (r["topk_ids"] >= begin) & (r["topk_ids"] < begin + E_loc)
    none = ~local.any(axis=1)
    assert np.all(r["out"][none] == 0)      # no local slot -> +0.0


def test_token_selection_matches_full_run():
    inp = make_layer_inputs("tiny", 16)
    full = oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=2)
    sel = np.zeros(16, np.uint8)
    sel[[0, 5, 11]] = 1
    part = oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=2, tok_sel=sel)
    assert np.array_equal(part["out"][sel == 1], full["out"][sel == 1])
    assert np.all(part["out"][sel == 0] == 0)
