"""GPU finalize vs the oracle: bit-exact (IEEE binary32 mul-then-FMA in slot order, no FTZ).

Inputs come from the seeded generators and the oracle's own routing and
permutation; no input or expected value comes from the GPU path.
"""
import json
import os
import struct

import numpy as np
import pytest

import oracle
from helpers import say, to_dev, to_np_u16
from w4a16_grouped_gemm_amd.inputs import bf16_bits, make_finalize_stress

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gpu_finalize(y, w, inv, out_f32):
    import torch
    from w4a16_grouped_gemm_amd import ops
    yd = to_dev(y) if y.dtype == np.float32 else to_dev(y).view(torch.bfloat16)
    out = ops.finalize(yd, to_dev(w), to_dev(inv), out_dtype=torch.float32 if out_f32 else torch.bfloat16)
    torch.cuda.synchronize()
    return out.cpu().numpy() if out_f32 else to_np_u16(out)


def test_golden_cases_on_gpu():
    cases = json.load(open(os.path.join(GOLD, "finalize_cases.json")))["cases"]
    H = 128
    for c in cases:
        say("finalize golden:", c["name"])
        ys = np.array([int(v, 16) for v in c["y"]], np.uint32).view(np.float32)
        ws = np.array([int(v, 16) for v in c["w"]], np.uint32).view(np.float32)
        k = len(ys)
        y = np.repeat(ys[:, None], H, axis=1).astype(np.float32)
        w = ws.reshape(1, k)
        inv = np.arange(k, dtype=np.int32).reshape(1, k)
        got = gpu_finalize(y, w, inv, True)
        assert np.all(got.view(np.uint32) == int(c["out"], 16)), c["name"]


@pytest.mark.parametrize("out_f32", [True, False])
def test_finalize_stress_full_size(out_f32):
    say("finalize_stress T=4096 k=8 H=4096 fp32 y, out_f32=", out_f32)
    fs = make_finalize_stress()
    ids, w = oracle.route(fs.logits, 8)
    w[fs.zero_mask] = 0.0
    _, _, _, inv = oracle.permute(ids, 128, 0)
    ref = oracle.finalize(fs.y, w, inv, out_f32=out_f32)
    got = gpu_finalize(fs.y, w, inv, out_f32)
    view = np.uint32 if out_f32 else np.uint16
    mism = int((got.view(view) != ref.view(view)).sum())
    assert mism == 0, f"{mism} mismatching elements"
    # the workload really exercises the edge cases
    assert (fs.y == 0).mean() > 0.05 and (np.abs(fs.y[fs.y != 0]) < 2 ** -126).mean() > 0.05


@pytest.mark.parametrize("T,k,H", [(7, 3, 256), (33, 8, 1024), (1, 1, 128)])
def test_finalize_bf16_y_absent_slots(T, k, H):
    say(f"finalize bf16 y T={T} k={k} H={H}")
    rng = np.random.default_rng(T * 100 + k)
    R = T * k
    yv = rng.standard_normal((R, H)).astype(np.float32)
    yv[rng.random((R, H)) < 0.1] = -0.0
    y = bf16_bits(yv)
    w = rng.standard_normal((T, k)).astype(np.float32)
    inv = rng.permutation(R).astype(np.int32).reshape(T, k)
    inv[rng.random((T, k)) < 0.3] = -1
    inv[0, :] = -1                              # a token with no local slot -> +0
    for out_f32 in (True, False):
        ref = oracle.finalize(y, w, inv, out_f32=out_f32)
        got = gpu_finalize(y, w, inv, out_f32)
        view = np.uint32 if out_f32 else np.uint16
        assert np.array_equal(got.view(view), ref.view(view))
    assert np.all(got[0] == 0)
