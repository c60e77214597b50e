"""The C-ABI library loads and exports every symbol include/moe_w4a16.h declares (no GPU, no compute)."""
import ctypes
import os
import re

import pytest

from w4a16_grouped_gemm_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        pytest.fail("libmoe_w4a16.so is not built; run __graft_entry__.build()")
    return ctypes.CDLL(ops.LIB_PATH)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(ops.EXPORTED)


def test_shape_queries_without_gpu():
    # pure host-side validation: no device needed
    ok = ops.make_shape(16, 256, 512, 8, 8, 2)
    assert ops.is_supported(ok) and ops.check_shape(ok) == 0
    assert ops.workspace_size(ok) > 0
    bad = [ops.make_shape(16, 200, 512, 8, 8, 2),          # H % 128
           ops.make_shape(16, 256, 512, 8, 8, 9),          # k > E
           ops.make_shape(16, 256, 512, 8, 8, 17),         # k > 16
           ops.make_shape(-1, 256, 512, 8, 8, 2),
           ops.make_shape(16, 256, 512, 8, 4, 2, expert_begin=6),
           ops.make_shape(16, 256, 512, 2000, 8, 2)]
    for b in bad:
        assert not ops.is_supported(b)
        assert ops.check_shape(b) == 2
        assert ops.workspace_size(b) == 0
    g64 = ops.make_shape(16, 256, 512, 8, 8, 2, group_size=64)
    assert ops.check_shape(g64) == 3
    assert ops.status_str(0) == "MOE_OK"


def test_layout_validation_without_gpu():
    # an unknown weight layout is rejected on the host
    bad = ops.make_shape(16, 256, 512, 8, 8, 2, weight_layout=2)
    assert ops.check_shape(bad) == 3
    assert not ops.is_supported(bad)
    tiled = ops.make_shape(16, 256, 512, 8, 8, 2, weight_layout=ops.WEIGHTS_TILED)
    assert ops.check_shape(tiled) == 0
    # packing in place is refused before any launch (host-side check only)
    lib = ops.load_library()
    sh = ops.make_shape(0, 256, 512, 8, 8, 1)
    p = ctypes.c_void_p(1 << 20)
    assert lib.moe_w4a16_pack_weights(ctypes.byref(sh), 0, p, p, None) == 3
    assert lib.moe_w4a16_pack_weights(ctypes.byref(sh), 7, p, p, None) == 3
    assert lib.moe_w4a16_pack_weights(ctypes.byref(sh), 0, None, p, None) == 1


def test_dense_validation_without_gpu():
    # every case below is refused (or is the M = 0 no-op) on the host, before any launch
    lib = ops.load_library()
    p = ctypes.c_void_p(1 << 20)
    f = lib.moe_w4a16_dense_gemm
    assert f(4, 200, 256, p, p, p, p, 0, 0, None) == 2          # N % 128
    assert f(4, 256, 64, p, p, p, p, 0, 0, None) == 2           # K < 128
    assert f(-1, 256, 256, p, p, p, p, 0, 0, None) == 2         # M < 0
    assert f(4, 131072, 256, p, p, p, p, 0, 0, None) == 2       # N > 65536
    assert f(4, 65536, 65536, p, p, p, p, 0, 0, None) == 3      # weights beyond one descriptor
    assert f(4, 256, 256, p, p, p, p, 7, 0, None) == 3          # output dtype
    assert f(4, 256, 256, p, p, p, p, 0, 2, None) == 3          # weight layout
    assert f(4, 256, 256, None, p, p, p, 0, 0, None) == 1       # NULL activations
    assert f(4, 256, 256, ctypes.c_void_p((1 << 20) + 2), p, p, p, 0, 0, None) == 4   # misaligned
    assert f(0, 256, 256, None, None, None, None, 0, 0, None) == 0    # M = 0: nothing to do


def test_shared_validation_without_gpu():
    # refused on the host before any launch
    lib = ops.load_library()
    sh = ops.make_shape(4, 256, 512, 8, 8, 2)
    p = ctypes.c_void_p(1 << 20)
    f = lib.moe_w4a16_forward_shared
    assert f(ctypes.byref(sh), 0, p, p, p, p, p, p, p, p, p, p, p, p, 1 << 30, None) == 3    # no shared expert
    assert f(ctypes.byref(sh), 5, p, p, p, p, p, p, p, p, p, p, p, p, 1 << 30, None) == 3    # more than 4
    assert f(ctypes.byref(sh), 1, p, p, p, p, p, p, None, p, p, p, p, p, 1 << 30, None) == 1  # NULL shared w13
    assert f(ctypes.byref(sh), 1, p, p, p, p, p, p, p, p, p, p, p, p, 16, None) == 5        # workspace too small
    assert lib.moe_w4a16_workspace_size_shared(ctypes.byref(sh), 2) > lib.moe_w4a16_workspace_size_shared(
        ctypes.byref(sh), 1)


def test_permute_workspace_without_gpu(lib):
    # 0 bytes while one workgroup permutes (up to 384 tokens), else int32
    # counts per (token range, local expert); a short or missing workspace is
    # refused before anything reaches the device
    S = ops.MoeShape
    lib.moe_permute_workspace_size.argtypes = [ctypes.POINTER(S)]
    lib.moe_permute_workspace_size.restype = ctypes.c_size_t
    small = ops.make_shape(384, 256, 512, 128, 128, 8)
    assert lib.moe_permute_workspace_size(ctypes.byref(small)) == 0
    for T, E in [(385, 128), (2048, 128), (100000, 32)]:
        sh = ops.make_shape(T, 256, 512, E, E, 8)
        ranges = min(64, (T + 127) // 128)
        assert lib.moe_permute_workspace_size(ctypes.byref(sh)) == ranges * E * 4
    sh = ops.make_shape(2048, 256, 512, 128, 128, 8)
    need = lib.moe_permute_workspace_size(ctypes.byref(sh))
    fake = ctypes.c_void_p(1 << 20)                       # never dereferenced: validation fails first
    args = [ctypes.byref(sh), fake, None, fake, fake, fake, fake, None]
    lib.moe_permute.restype = ctypes.c_int
    MOE_ERR_NULL, MOE_ERR_WORKSPACE = 1, 5
    assert lib.moe_permute(*args, fake, ctypes.c_size_t(need - 4), None) == MOE_ERR_WORKSPACE
    assert lib.moe_permute(*args, None, ctypes.c_size_t(need), None) == MOE_ERR_NULL


def test_launch_override_without_gpu():
    # the override is host state only: setting, resetting and rejecting an
    # unknown field need no device
    ops.set_launch_override(gemm_mode=1, gemm_tiles_per_wave=2)
    ops.set_launch_override()
    with ops.launch_override(route_fuse_max_tokens=0):
        pass
    with pytest.raises(ValueError):
        ops.set_launch_override(no_such_field=1)
