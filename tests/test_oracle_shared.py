"""Pins of the oracle's shared experts (no GPU).

Reading (GC-MoE abstract names "optional shared experts" without defining
them): S always-on experts with the routed experts' shape run on every token;
each one's bf16 output joins the binary32 combine with weight 1 after the
routed slots (acc = acc + v, or acc = v when it is the token's first term).

- The per-token brute force (no permutation) equals the permuted path bit for
  bit, with an expert-parallel window (non-local slots, tokens with no local
  slot) included.
- All-zero routed codes leave only the shared experts: the output is then an
  fp64 numpy SwiGLU FFN of x through them (a separate arithmetic path).
- All-zero shared codes give back the routed-only layer.
- The finalize's shared terms against exact-rational rounding.
"""
import numpy as np
import pytest

import oracle
from oracle import exact
from w4a16_grouped_gemm_amd.inputs import (Workload, bf16_bits, bf16_values, make_layer_inputs,
                                           make_shared_weights)

EP_SMALL = Workload("ep_small", 7, 16, 4, 6, 4, 256, 256, (8,))


def _zero_codes(w):
    return np.zeros_like(w)                               # byte 0 = two zero codes


@pytest.mark.parametrize("wl,T,S", [("tiny", 16, 1), ("tiny", 16, 2), (EP_SMALL, 24, 1)])
def test_shared_bruteforce_equals_permuted(wl, T, S):
    inp = make_layer_inputs(wl, T)
    sh = make_shared_weights(inp.workload, S)
    r = oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=inp.workload.top_k,
                     expert_begin=inp.workload.expert_begin, shared=sh)
    bf = oracle.layer_bruteforce(inp.x, r["topk_ids"], r["topk_w"], inp.w13_q, inp.s13, inp.w2_q, inp.s2,
                                 expert_begin=inp.workload.expert_begin, shared=sh)
    assert np.array_equal(r["out"], bf)
    if wl is EP_SMALL:
        local = (r["topk_ids"] >= 6) & (r["topk_ids"] < 10)
        assert (~local.any(axis=1)).any(), "the window must leave some token without a local slot"


def _np_ffn(x_u16, w13_q, s13, w2_q, s2, e):
    """fp64 numpy SwiGLU FFN of expert e, bf16 RNE at h and y (one rounding each)."""
    def deq(wq, s):
        lo = (wq & 0xF).astype(np.int16)
        hi = (wq >> 4).astype(np.int16)
        q = np.empty(wq.shape[:-1] + (wq.shape[-1] * 2,), np.int16)
        q[..., 0::2], q[..., 1::2] = lo, hi
        q = np.where(q >= 8, q - 16, q).astype(np.float64)
        return q * np.repeat(bf16_values(s).astype(np.float64), 128, axis=-1)
    x = bf16_values(x_u16).astype(np.float64)
    W13, W2 = deq(w13_q[e], s13[e]), deq(w2_q[e], s2[e])
    I = W13.shape[0] // 2
    g, u = x @ W13[:I].T, x @ W13[I:].T
    a = g / (1.0 + np.exp(-g)) * u
    h = np.array([[exact.bf16_bits(v) for v in row] for row in a], np.uint16)
    d = bf16_values(h).astype(np.float64) @ W2.T
    return np.array([[exact.bf16_bits(v) for v in row] for row in d], np.uint16)


def test_zero_routed_codes_leave_the_dense_shared_ffn():
    inp = make_layer_inputs("tiny", 8)
    sh = make_shared_weights("tiny", 1)
    r = oracle.layer(inp.x, inp.logits, _zero_codes(inp.w13_q), inp.s13, _zero_codes(inp.w2_q), inp.s2,
                     top_k=inp.workload.top_k, shared=sh)
    want = _np_ffn(inp.x, *sh, 0)
    want = np.where(want == 0x8000, 0, want)              # +0 (routed) + (-0) = +0
    assert np.array_equal(r["out"], want)


def test_zero_shared_codes_give_the_routed_layer():
    inp = make_layer_inputs("tiny", 16)
    w13s, s13s, w2s, s2s = make_shared_weights("tiny", 2)
    base = oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=inp.workload.top_k)
    r = oracle.layer(inp.x, inp.logits, inp.w13_q, inp.s13, inp.w2_q, inp.s2, top_k=inp.workload.top_k,
                     shared=(_zero_codes(w13s), s13s, _zero_codes(w2s), s2s))
    want = np.where(base["out"] == 0x8000, 0, base["out"])    # acc + (+0): -0 becomes +0
    assert np.array_equal(r["out"], want)
    assert not r["ys"].any()


def test_finalize_shared_terms_are_exact_adds():
    rng = np.random.default_rng(5)
    T, k, H, S = 64, 3, 4, 2
    y = (rng.standard_normal((T * k, H)) * 2.0 ** rng.integers(-30, 30, (T * k, H))).astype(np.float32)
    ys = (rng.standard_normal((S, T, H)) * 2.0 ** rng.integers(-30, 30, (S, T, H))).astype(np.float32)
    ys[0, 0, 0] = -0.0
    w = rng.random((T, k)).astype(np.float32)
    inv = np.arange(T * k, dtype=np.int32).reshape(T, k)
    inv[rng.random((T, k)) < 0.3] = -1
    inv[1] = -1                                           # a token with no routed slot
    got = oracle.finalize(y, w, inv, out_f32=True, ys=ys)
    for t in range(T):
        for c in range(H):
            present = inv[t] >= 0
            acc = None
            for j in range(k):
                if present[j]:
                    v, wj = float(y[inv[t, j], c]), float(w[t, j])
                    acc = exact.mul_f32(v, wj) if acc is None else exact.fma_f32(v, wj, acc)
            for s in range(S):
                v = float(ys[s, t, c])
                acc = v if acc is None else exact.fma_f32(v, 1.0, acc)
            assert np.float32(got[t, c]).tobytes() == np.float32(acc).tobytes(), (t, c)
