"""The seeded generators: reproducible bytes and the stated distributions (no GPU)."""
import hashlib

import numpy as np

from w4a16_grouped_gemm_amd.inputs import (WORKLOADS, bf16_values, make_finalize_stress,
                                           make_layer_inputs, unpack_int4)


def digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_reproducible():
    a = make_layer_inputs("tiny", 16)
    b = make_layer_inputs("tiny", 16)
    assert digest(a.x, a.logits, a.w13_q, a.s13, a.w2_q, a.s2) == digest(b.x, b.logits, b.w13_q, b.s13, b.w2_q, b.s2)
    c = make_layer_inputs("tiny", 15)
    assert digest(a.x) != digest(c.x[:1])


def test_shapes_and_distributions():
    inp = make_layer_inputs("tiny", 16)
    wl = WORKLOADS["tiny"]
    assert inp.x.shape == (16, 256) and inp.logits.shape == (16, 8)
    assert inp.w13_q.shape == (8, 1024, 128) and inp.s13.shape == (8, 1024, 2)
    assert inp.w2_q.shape == (8, 256, 256) and inp.s2.shape == (8, 256, 4)
    q = unpack_int4(inp.w13_q)
    assert q.min() == -8 and q.max() == 7
    hist = np.bincount((q.astype(int) + 8).reshape(-1), minlength=16) / q.size
    assert np.all(np.abs(hist - 1 / 16) < 0.01)
    s = bf16_values(inp.s13)
    assert s.min() >= 0.0049 and s.max() <= 0.0201
    x = bf16_values(inp.x)
    assert abs(float(x.mean())) < 0.1 and abs(float(x.std()) - 1) < 0.1
    assert wl.hidden % 128 == 0 and wl.inter % 128 == 0


def test_zipf_routing_is_skewed():
    import oracle
    inp = make_layer_inputs("qwen3_prefill", 2048)
    ids, _ = oracle.route(inp.logits, 8)
    counts = np.bincount(ids.reshape(-1), minlength=128)
    assert counts.sum() == 2048 * 8
    assert counts.max() > 1000 and np.median(counts) < 128


def test_finalize_stress_mix():
    fs = make_finalize_stress(tokens=64, hidden=256)
    y = fs.y
    zeros = y == 0
    sub = (y != 0) & (np.abs(y) < np.float32(2.0 ** -126))
    assert abs(zeros.mean() - 0.1) < 0.02 and abs(sub.mean() - 0.1) < 0.02
    assert np.signbit(y[zeros]).mean() > 0.3
    assert abs(fs.zero_mask.mean() - 0.1) < 0.05
