"""moe_w4a16_forward_noalloc (the layer with no caller workspace) vs moe_w4a16_forward.

The entry point keeps the layer's intermediates in the library's fixed
per-GPU scratch array. Through the C ABI, two calls in a row (the second with
fewer tokens, so the array holds the first call's intermediates when it
starts) must each equal moe_w4a16_forward bit for bit; a shape whose
workspace exceeds the array is refused before any launch.
"""
import numpy as np
import pytest

from helpers import bf16_dev, say, to_dev, to_np_u16
from w4a16_grouped_gemm_amd.inputs import make_layer_inputs

pytestmark = pytest.mark.gpu


def _dev(inp):
    return (bf16_dev(inp.x), to_dev(inp.logits), to_dev(inp.w13_q), bf16_dev(inp.s13), to_dev(inp.w2_q),
            bf16_dev(inp.s2))


@pytest.mark.parametrize("wl,T1,T2", [("qwen3_decode", 256, 16), ("ep_shard_decode", 64, 1), ("tiny", 16, 3)])
def test_noalloc_equals_forward(wl, T1, T2):
    import torch
    from w4a16_grouped_gemm_amd import ops
    say(f"noalloc {wl} T={T1} then T={T2}")
    for T in (T1, T2):
        inp = make_layer_inputs(wl, T)
        args = _dev(inp)
        w = inp.workload
        want = ops.moe_w4a16_forward(*args, w.top_k, expert_begin=w.expert_begin)
        out = torch.full((T, w.hidden), 3.0, dtype=torch.bfloat16, device="cuda")
        ops.moe_w4a16_forward_noalloc(*args, w.top_k, out, expert_begin=w.expert_begin)
        torch.cuda.synchronize()
        assert np.array_equal(to_np_u16(out), to_np_u16(want)), (wl, T)


def test_noalloc_refuses_oversized_shapes():
    import ctypes
    import torch
    from w4a16_grouped_gemm_amd import ops
    say("noalloc size limit")
    lib = ops.load_library()
    T = 4096                                              # Qwen3-30B-A3B shape: ~185 MB of workspace
    sh = ops.make_shape(T, 2048, 768, 128, 128, 8)
    assert lib.moe_w4a16_workspace_size(ctypes.byref(sh)) > ops.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, 2048), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((T, 128), dtype=torch.float32, device="cuda")
    w13 = torch.zeros((128, 1536, 1024), dtype=torch.uint8, device="cuda")
    s13 = torch.zeros((128, 1536, 16), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((128, 2048, 384), dtype=torch.uint8, device="cuda")
    s2 = torch.zeros((128, 2048, 6), dtype=torch.bfloat16, device="cuda")
    out = torch.full((T, 2048), 5.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ops.MoeError) as ei:
        ops.moe_w4a16_forward_noalloc(x, lg, w13, s13, w2, s2, 8, out)
    assert ei.value.code == 5                             # MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())                       # untouched
