"""ctypes binding of libmoe_w4a16.so (argument marshalling only).

Every function takes torch tensors on a gfx950 device, checks dtypes and
shapes, and passes data pointers plus the current (or given) HIP stream to the
C ABI declared in include/moe_w4a16.h. All arithmetic runs in the library's
HIP kernels; nothing here computes on the host. If the library is missing the
first call raises; there is no fallback path.

Status codes map to exceptions: NULL / SHAPE / UNSUPPORTED / ALIGN / WORKSPACE
raise ValueError, a failed launch raises RuntimeError.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_w4a16.so")

MOE_BF16, MOE_F32 = 0, 1
W13_SWIGLU, W2, W13_RAW = 0, 1, 2
WEIGHTS_PLAIN, WEIGHTS_TILED = 0, 1
_STATUS = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_UNSUPPORTED",
           4: "MOE_ERR_ALIGN", 5: "MOE_ERR_WORKSPACE", 6: "MOE_ERR_HIP"}
EXPORTED = ["moe_status_str", "moe_w4a16_check_shape", "moe_w4a16_is_supported",
            "moe_w4a16_workspace_size", "moe_w4a16_forward", "moe_route", "moe_permute_workspace_size",
            "moe_permute", "moe_grouped_gemm_w4a16", "moe_finalize", "moe_w4a16_pack_weights",
            "moe_w4a16_dense_gemm", "moe_w4a16_workspace_size_shared", "moe_w4a16_forward_shared",
            "moe_w4a16_set_launch_override", "moe_w4a16_forward_noalloc", "moe_mxfp4_quantize",
            "moe_grouped_gemm_mxfp4", "moe_w4a4_workspace_size", "moe_w4a4_forward",
            "moe_mxfp4_pack_weights"]


class MoeShape(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("expert_begin", ctypes.c_int32),
                ("num_local_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("weight_layout", ctypes.c_int32)]


class LaunchOverride(ctypes.Structure):
    _fields_ = [("gemm_mode", ctypes.c_int32), ("gemm_tiles_per_wave", ctypes.c_int32),
                ("gemm_subtiles", ctypes.c_int32), ("gemm_kseg", ctypes.c_int32), ("gemm_ring", ctypes.c_int32),
                ("gemm_nontemporal", ctypes.c_int32), ("permute_parallel_min_tokens", ctypes.c_int32),
                ("route_fuse_max_tokens", ctypes.c_int32), ("decode_max_tokens", ctypes.c_int32),
                ("decode_combine_max_tokens", ctypes.c_int32), ("perm_in_gemm_max_tokens", ctypes.c_int32)]


class MoeError(ValueError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH):
    """Load the C ABI library (once). Raises RuntimeError if it is not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} not found: build it first (python -m w4a16_grouped_gemm_amd.build "
                               "or __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        P, I, S, Z = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(MoeShape), ctypes.c_size_t
        lib.moe_status_str.argtypes = [I]
        lib.moe_status_str.restype = ctypes.c_char_p
        lib.moe_w4a16_check_shape.argtypes = [S]
        lib.moe_w4a16_check_shape.restype = I
        lib.moe_w4a16_is_supported.argtypes = [S]
        lib.moe_w4a16_is_supported.restype = I
        lib.moe_w4a16_workspace_size.argtypes = [S]
        lib.moe_w4a16_workspace_size.restype = Z
        lib.moe_permute_workspace_size.argtypes = [S]
        lib.moe_permute_workspace_size.restype = Z
        lib.moe_w4a16_forward.argtypes = [S, P, P, P, P, P, P, P, P, Z, P]
        lib.moe_w4a16_forward.restype = I
        lib.moe_route.argtypes = [S, P, P, P, P]
        lib.moe_route.restype = I
        lib.moe_permute.argtypes = [S, P, P, P, P, P, P, P, P, Z, P]
        lib.moe_permute.restype = I
        lib.moe_grouped_gemm_w4a16.argtypes = [S, I, P, P, P, P, P, P, I, P]
        lib.moe_grouped_gemm_w4a16.restype = I
        lib.moe_finalize.argtypes = [S, P, I, P, P, P, I, P]
        lib.moe_finalize.restype = I
        lib.moe_w4a16_pack_weights.argtypes = [S, I, P, P, P]
        lib.moe_w4a16_pack_weights.restype = I
        lib.moe_w4a16_dense_gemm.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P, P, I,
                                             ctypes.c_int32, P]
        lib.moe_w4a16_dense_gemm.restype = I
        lib.moe_w4a16_workspace_size_shared.argtypes = [S, ctypes.c_int32]
        lib.moe_w4a16_workspace_size_shared.restype = Z
        lib.moe_w4a16_forward_shared.argtypes = [S, ctypes.c_int32] + [P] * 12 + [Z, P]
        lib.moe_w4a16_forward_shared.restype = I
        lib.moe_w4a16_set_launch_override.argtypes = [ctypes.POINTER(LaunchOverride)]
        lib.moe_w4a16_set_launch_override.restype = I
        lib.moe_w4a16_forward_noalloc.argtypes = [S, P, P, P, P, P, P, P, P]
        lib.moe_w4a16_forward_noalloc.restype = I
        lib.moe_mxfp4_quantize.argtypes = [ctypes.c_int64, ctypes.c_int32, P, P, P, P]
        lib.moe_mxfp4_quantize.restype = I
        lib.moe_grouped_gemm_mxfp4.argtypes = [S, I, P, P, P, P, P, P, P, I, P]
        lib.moe_grouped_gemm_mxfp4.restype = I
        lib.moe_w4a4_workspace_size.argtypes = [S]
        lib.moe_w4a4_workspace_size.restype = Z
        lib.moe_w4a4_forward.argtypes = [S, P, P, P, P, P, P, P, P, Z, P]
        lib.moe_w4a4_forward.restype = I
        lib.moe_mxfp4_pack_weights.argtypes = [S, I, P, P, P]
        lib.moe_mxfp4_pack_weights.restype = I
        _lib = lib
        return lib


def make_shape(num_tokens, hidden, inter, num_experts, num_local_experts, top_k, expert_begin=0,
               group_size=128, weight_layout=WEIGHTS_PLAIN) -> MoeShape:
    return MoeShape(int(num_tokens), int(hidden), int(inter), int(num_experts), int(expert_begin),
                    int(num_local_experts), int(top_k), int(group_size), int(weight_layout))


def status_str(code: int) -> str:
    return load_library().moe_status_str(int(code)).decode()


def _check(code: int):
    if code == 0:
        return
    msg = status_str(code)
    if code == 6:
        raise RuntimeError(msg)
    raise MoeError(code, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t, dtype, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def set_launch_override(**fields) -> None:
    """Force launch-shape choices (see moe_launch_override in the C header);
    fields not given stay automatic (-1). No fields: back to automatic."""
    ov = LaunchOverride(*([-1] * len(LaunchOverride._fields_)))
    for k, v in fields.items():
        if k not in dict(LaunchOverride._fields_):
            raise ValueError(f"unknown launch override field {k}")
        setattr(ov, k, int(v))
    _check(load_library().moe_w4a16_set_launch_override(ctypes.byref(ov) if fields else None))


class launch_override:
    """Context manager: set_launch_override(**fields) inside, automatic after."""

    def __init__(self, **fields):
        self.fields = fields

    def __enter__(self):
        set_launch_override(**self.fields)
        return self

    def __exit__(self, *exc):
        set_launch_override()
        return False


def check_shape(shape: MoeShape) -> int:
    return int(load_library().moe_w4a16_check_shape(ctypes.byref(shape)))


def is_supported(shape: MoeShape) -> bool:
    return bool(load_library().moe_w4a16_is_supported(ctypes.byref(shape)))


def workspace_size(shape: MoeShape) -> int:
    return int(load_library().moe_w4a16_workspace_size(ctypes.byref(shape)))


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def route(logits: torch.Tensor, top_k: int, *, stream=None):
    """Top-k routing -> (topk_ids int32 [T,k], topk_w float32 [T,k])."""
    _need(logits, torch.float32, "logits")
    T, E = logits.shape
    ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    sh = make_shape(T, 128, 128, E, E, top_k)
    _check(load_library().moe_route(ctypes.byref(sh), _ptr(logits), _ptr(ids), _ptr(w), _stream(stream)))
    return ids, w


def permute(topk_ids: torch.Tensor, num_local_experts: int, *, num_experts: int | None = None,
            expert_begin: int = 0, x: torch.Tensor | None = None, stream=None):
    """Stable expert permutation -> (counts, offsets, perm, inv_perm, x_perm or None)."""
    _need(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    dev = topk_ids.device
    E_g = num_experts if num_experts is not None else expert_begin + num_local_experts
    H = 128
    x_perm = None
    if x is not None:
        _need(x, torch.bfloat16, "x")
        H = x.shape[1]
        x_perm = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    sh = make_shape(T, H, 128, E_g, num_local_experts, k, expert_begin)
    counts = torch.empty(num_local_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(num_local_experts + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv_perm = torch.empty((T, k), dtype=torch.int32, device=dev)
    lib = load_library()
    nws = lib.moe_permute_workspace_size(ctypes.byref(sh))
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    _check(lib.moe_permute(ctypes.byref(sh), _ptr(topk_ids), _ptr(x), _ptr(counts), _ptr(offsets),
                           _ptr(perm), _ptr(inv_perm), _ptr(x_perm), _ptr(ws), nws, _stream(stream)))
    return counts, offsets, perm, inv_perm, x_perm


def pack_weights(kind: int, wq: torch.Tensor, *, stream=None) -> torch.Tensor:
    """Plain -> tiled int4 codes of one weight matrix (same shape and dtype).

    kind: W13_SWIGLU (w13 for the layer / SwiGLU GEMM), W13_RAW or W2."""
    _need(wq, torch.uint8, "wq")
    E_loc, N, K2 = wq.shape
    if kind == W2:
        H, I = N, 2 * K2
    else:
        H, I = 2 * K2, N // 2
    out = torch.empty_like(wq)
    sh = make_shape(0, H, I, E_loc, E_loc, 1)
    _check(load_library().moe_w4a16_pack_weights(ctypes.byref(sh), int(kind), _ptr(wq), _ptr(out),
                                                 _stream(stream)))
    return out


def grouped_gemm_w4a16(kind: int, a: torch.Tensor, offsets: torch.Tensor, wq: torch.Tensor,
                       s: torch.Tensor, *, num_tokens: int, top_k: int,
                       a_row_index: torch.Tensor | None = None, out_dtype=torch.bfloat16,
                       num_experts: int | None = None, out: torch.Tensor | None = None, stream=None,
                       weight_layout: int = WEIGHTS_PLAIN):
    """Grouped W4A16 GEMM over expert slabs; returns c [num_tokens*top_k, cols]."""
    _need(a, torch.bfloat16, "a")
    _need(offsets, torch.int32, "offsets")
    _need(wq, torch.uint8, "wq")
    _need(s, torch.bfloat16, "s")
    if a_row_index is not None:
        _need(a_row_index, torch.int32, "a_row_index")
    E_loc, N, K2 = wq.shape
    K = 2 * K2
    if kind == W2:
        H, I = N, K
        cols = N
    else:
        H, I = K, N // 2
        cols = I if kind == W13_SWIGLU else N
    if a.shape[-1] != K:
        raise ValueError(f"a has {a.shape[-1]} columns, weights expect K={K}")
    if s.shape != (E_loc, N, K // 128):
        raise ValueError(f"scales shape {tuple(s.shape)} != {(E_loc, N, K // 128)}")
    rows = num_tokens * top_k
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype, device=a.device)
    dt = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}.get(out.dtype)
    if dt is None:
        raise ValueError("out dtype must be bfloat16 or float32")
    sh = make_shape(num_tokens, H, I, num_experts or E_loc, E_loc, top_k, weight_layout=weight_layout)
    _check(load_library().moe_grouped_gemm_w4a16(ctypes.byref(sh), int(kind), _ptr(a), _ptr(a_row_index),
                                                 _ptr(offsets), _ptr(wq), _ptr(s), _ptr(out), dt,
                                                 _stream(stream)))
    return out


def pack_dense_weights(wq: torch.Tensor, *, stream=None) -> torch.Tensor:
    """Plain -> tiled int4 codes of one dense weight matrix [N, K/2]."""
    return pack_weights(W2, wq.unsqueeze(0), stream=stream)[0]


def dense_gemm_w4a16(a: torch.Tensor, wq: torch.Tensor, s: torch.Tensor, *, out_dtype=torch.bfloat16,
                     out: torch.Tensor | None = None, weight_layout: int = WEIGHTS_PLAIN, stream=None):
    """Dense W4A16 GEMM: c [M, N] = a [M, K] . W^T, W[n, k] = q[n, k] * s[n, k // 128]."""
    _need(a, torch.bfloat16, "a")
    _need(wq, torch.uint8, "wq")
    _need(s, torch.bfloat16, "s")
    M, K = a.shape
    N = wq.shape[0]
    if wq.shape != (N, K // 2) or s.shape != (N, K // 128):
        raise ValueError(f"weight shapes {tuple(wq.shape)}, {tuple(s.shape)} do not match K={K}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    dt = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}.get(out.dtype)
    if dt is None:
        raise ValueError("out dtype must be bfloat16 or float32")
    _check(load_library().moe_w4a16_dense_gemm(M, N, K, _ptr(a), _ptr(wq), _ptr(s), _ptr(out), dt,
                                               int(weight_layout), _stream(stream)))
    return out


def finalize(y: torch.Tensor, topk_w: torch.Tensor, inv_perm: torch.Tensor, *,
             out_dtype=torch.bfloat16, out: torch.Tensor | None = None, stream=None):
    """Slot-ordered combine -> out [T, H] (float32 accumulator or its bf16 RNE)."""
    _need(topk_w, torch.float32, "topk_w")
    _need(inv_perm, torch.int32, "inv_perm")
    if y.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("y must be bfloat16 or float32")
    _need(y, y.dtype, "y")
    T, k = topk_w.shape
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=y.device)
    sh = make_shape(T, H, 128, k, k, k)
    ydt = MOE_F32 if y.dtype == torch.float32 else MOE_BF16
    odt = MOE_F32 if out.dtype == torch.float32 else MOE_BF16
    _check(load_library().moe_finalize(ctypes.byref(sh), _ptr(y), ydt, _ptr(topk_w), _ptr(inv_perm),
                                       _ptr(out), odt, _stream(stream)))
    return out


_ws_cache: dict = {}
_ws_lock = threading.Lock()


def _workspace(nbytes: int, device, stream) -> torch.Tensor:
    """Default layer workspace, one per (device, stream): forwards in flight on
    different streams never share one. It is allocated while its stream is
    current, so when it grows the caching allocator reuses the old block only
    for work ordered after everything already queued on that stream."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    dev = device.index if device.index is not None else torch.cuda.current_device()
    key = (dev, handle)
    with _ws_lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            if isinstance(stream, torch.cuda.Stream):
                with torch.cuda.stream(stream):
                    buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            else:
                buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
                buf.record_stream(torch.cuda.ExternalStream(handle, device=device))
            _ws_cache[key] = buf
    return buf


def moe_w4a16_forward(x: torch.Tensor, router_logits: torch.Tensor, w13_q: torch.Tensor,
                      s13: torch.Tensor, w2_q: torch.Tensor, s2: torch.Tensor, top_k: int,
                      out: torch.Tensor | None = None, stream=None, *, expert_begin: int = 0,
                      workspace: torch.Tensor | None = None,
                      weight_layout: int = WEIGHTS_PLAIN, shared=None) -> torch.Tensor:
    """The whole quantized MoE expert layer (route, permute, GEMM1+SwiGLU, GEMM2, finalize).

    weight_layout=WEIGHTS_TILED takes codes from pack_weights (w13 packed
    with W13_SWIGLU, w2 with W2). shared: optional (w13_sh [S, 2I, H/2],
    s13_sh, w2_sh [S, H, I/2], s2_sh) always-on experts, added after the
    routed slots."""
    _need(x, torch.bfloat16, "x")
    _need(router_logits, torch.float32, "router_logits")
    _need(w13_q, torch.uint8, "w13_q")
    _need(s13, torch.bfloat16, "s13")
    _need(w2_q, torch.uint8, "w2_q")
    _need(s2, torch.bfloat16, "s2")
    T, H = x.shape
    E_g = router_logits.shape[1]
    E_loc, N13, H2 = w13_q.shape
    I = N13 // 2
    if H2 * 2 != H or w2_q.shape != (E_loc, H, I // 2):
        raise ValueError("weight shapes do not match x")
    if s13.shape != (E_loc, 2 * I, H // 128) or s2.shape != (E_loc, H, I // 128):
        raise ValueError("scale shapes do not match the weights")
    if router_logits.shape[0] != T:
        raise ValueError("router_logits rows != tokens")
    sh = make_shape(T, H, I, E_g, E_loc, top_k, expert_begin, weight_layout=weight_layout)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    lib = load_library()
    if shared is not None:
        w13s, s13s, w2s, s2s = shared
        for t, d, n in ((w13s, torch.uint8, "w13_sh"), (s13s, torch.bfloat16, "s13_sh"),
                        (w2s, torch.uint8, "w2_sh"), (s2s, torch.bfloat16, "s2_sh")):
            _need(t, d, n)
        nsh = w13s.shape[0]
        if (w13s.shape != (nsh, 2 * I, H // 2) or w2s.shape != (nsh, H, I // 2)
                or s13s.shape != (nsh, 2 * I, H // 128) or s2s.shape != (nsh, H, I // 128)):
            raise ValueError("shared expert shapes do not match the routed experts")
        nbytes = int(lib.moe_w4a16_workspace_size_shared(ctypes.byref(sh), nsh))
        if nbytes == 0:
            _check(int(lib.moe_w4a16_check_shape(ctypes.byref(sh))) or 3)
        if workspace is None:
            workspace = _workspace(nbytes, x.device, stream)
        _check(lib.moe_w4a16_forward_shared(ctypes.byref(sh), nsh, _ptr(x), _ptr(router_logits), _ptr(w13_q),
                                            _ptr(s13), _ptr(w2_q), _ptr(s2), _ptr(w13s), _ptr(s13s), _ptr(w2s),
                                            _ptr(s2s), _ptr(out), _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), _stream(stream)))
        return out
    nbytes = int(lib.moe_w4a16_workspace_size(ctypes.byref(sh)))
    if nbytes == 0:
        _check(int(lib.moe_w4a16_check_shape(ctypes.byref(sh))) or 2)
    if workspace is None:
        workspace = _workspace(nbytes, x.device, stream)
    _check(lib.moe_w4a16_forward(ctypes.byref(sh), _ptr(x), _ptr(router_logits), _ptr(w13_q), _ptr(s13),
                                 _ptr(w2_q), _ptr(s2), _ptr(out), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES of the C header


def moe_w4a16_forward_noalloc(x: torch.Tensor, router_logits: torch.Tensor, w13_q: torch.Tensor,
                              s13: torch.Tensor, w2_q: torch.Tensor, s2: torch.Tensor, top_k: int,
                              out: torch.Tensor, stream=None, *, expert_begin: int = 0,
                              weight_layout: int = WEIGHTS_PLAIN) -> torch.Tensor:
    """The layer through moe_w4a16_forward_noalloc: no workspace, nothing
    allocated (the caller passes `out`); the library's fixed per-GPU scratch
    array holds the intermediates. Calls that overlap on one GPU race."""
    for t, d, n in ((x, torch.bfloat16, "x"), (router_logits, torch.float32, "router_logits"),
                    (w13_q, torch.uint8, "w13_q"), (s13, torch.bfloat16, "s13"), (w2_q, torch.uint8, "w2_q"),
                    (s2, torch.bfloat16, "s2"), (out, torch.bfloat16, "out")):
        _need(t, d, n)
    T, H = x.shape
    E_loc, N13, _ = w13_q.shape
    sh = make_shape(T, H, N13 // 2, router_logits.shape[1], E_loc, top_k, expert_begin,
                    weight_layout=weight_layout)
    if tuple(out.shape) != (T, H):
        raise ValueError("out must be [T, H]")
    _check(load_library().moe_w4a16_forward_noalloc(ctypes.byref(sh), _ptr(x), _ptr(router_logits), _ptr(w13_q),
                                                    _ptr(s13), _ptr(w2_q), _ptr(s2), _ptr(out), _stream(stream)))
    return out


# ---------------------------------------------------------------------------
# the W4A4 (MXFP4) variant
# ---------------------------------------------------------------------------

def mxfp4_quantize(x: torch.Tensor, *, stream=None):
    """bf16 [R, K] -> (codes uint8 [R, K/2], scales uint8 [R, K/32]), MXFP4."""
    _need(x, torch.bfloat16, "x")
    R, K = x.shape
    codes = torch.empty((R, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((R, K // 32), dtype=torch.uint8, device=x.device)
    _check(load_library().moe_mxfp4_quantize(int(R), int(K), _ptr(x), _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def mxfp4_pack_weights(kind: int, wq: torch.Tensor, *, stream=None) -> torch.Tensor:
    """Plain -> tiled MXFP4 codes of one weight matrix (same shape and dtype).

    kind: W13_SWIGLU (w13 for the layer / SwiGLU GEMM), W13_RAW or W2."""
    _need(wq, torch.uint8, "wq")
    E_loc, N, K2 = wq.shape
    if kind == W2:
        H, I = N, 2 * K2
    else:
        H, I = 2 * K2, N // 2
    out = torch.empty_like(wq)
    sh = make_shape(0, H, I, E_loc, E_loc, 1, group_size=32)
    _check(load_library().moe_mxfp4_pack_weights(ctypes.byref(sh), int(kind), _ptr(wq), _ptr(out),
                                                 _stream(stream)))
    return out


def grouped_gemm_mxfp4(kind: int, a_codes: torch.Tensor, a_scales: torch.Tensor, offsets: torch.Tensor,
                       wq: torch.Tensor, ws: torch.Tensor, *, num_tokens: int, top_k: int,
                       a_row_index: torch.Tensor | None = None, out_dtype=torch.bfloat16,
                       num_experts: int | None = None, out: torch.Tensor | None = None, stream=None,
                       weight_layout: int = WEIGHTS_PLAIN):
    """Grouped GEMM on MXFP4 activations and weights; returns c [num_tokens*top_k, cols]."""
    _need(a_codes, torch.uint8, "a_codes")
    _need(a_scales, torch.uint8, "a_scales")
    _need(offsets, torch.int32, "offsets")
    _need(wq, torch.uint8, "wq")
    _need(ws, torch.uint8, "ws")
    E_loc, N, K2 = wq.shape
    K = 2 * K2
    if ws.shape != (E_loc, N, K // 32) or a_codes.shape[-1] != K // 2 or a_scales.shape[-1] != K // 32:
        raise ValueError("MXFP4 operand shapes do not match")
    if kind == W2:
        H, I, cols = N, K, N
    else:
        H, I = K, N // 2
        cols = I if kind == W13_SWIGLU else N
    if out is None:
        out = torch.empty((num_tokens * top_k, cols), dtype=out_dtype, device=a_codes.device)
    dt = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}.get(out.dtype)
    if dt is None:
        raise ValueError("out dtype must be bfloat16 or float32")
    if a_row_index is not None:
        _need(a_row_index, torch.int32, "a_row_index")
    sh = make_shape(num_tokens, H, I, num_experts or E_loc, E_loc, top_k, group_size=32,
                    weight_layout=weight_layout)
    _check(load_library().moe_grouped_gemm_mxfp4(ctypes.byref(sh), int(kind), _ptr(a_codes), _ptr(a_scales),
                                                 _ptr(a_row_index), _ptr(offsets), _ptr(wq), _ptr(ws), _ptr(out),
                                                 dt, _stream(stream)))
    return out


def moe_w4a4_forward(x: torch.Tensor, router_logits: torch.Tensor, w13_q: torch.Tensor, w13_s: torch.Tensor,
                     w2_q: torch.Tensor, w2_s: torch.Tensor, top_k: int, out: torch.Tensor | None = None,
                     stream=None, *, expert_begin: int = 0, workspace: torch.Tensor | None = None,
                     weight_layout: int = WEIGHTS_PLAIN) -> torch.Tensor:
    """The W4A4 (MXFP4) MoE expert layer: MXFP4 weights, activations quantized on the fly.
    weight_layout WEIGHTS_TILED: w13_q and w2_q from mxfp4_pack_weights (W13_SWIGLU / W2)."""
    _need(x, torch.bfloat16, "x")
    _need(router_logits, torch.float32, "router_logits")
    for t, n in ((w13_q, "w13_q"), (w13_s, "w13_s"), (w2_q, "w2_q"), (w2_s, "w2_s")):
        _need(t, torch.uint8, n)
    T, H = x.shape
    E_loc, N13, H2 = w13_q.shape
    I = N13 // 2
    if (H2 * 2 != H or w2_q.shape != (E_loc, H, I // 2) or w13_s.shape != (E_loc, 2 * I, H // 32)
            or w2_s.shape != (E_loc, H, I // 32)):
        raise ValueError("MXFP4 weight shapes do not match x")
    sh = make_shape(T, H, I, router_logits.shape[1], E_loc, top_k, expert_begin, group_size=32,
                    weight_layout=weight_layout)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    lib = load_library()
    nbytes = int(lib.moe_w4a4_workspace_size(ctypes.byref(sh)))
    if nbytes == 0 and T > 0:
        raise MoeError(2, "shape not supported by the W4A4 layer")
    if workspace is None:
        workspace = _workspace(nbytes, x.device, stream)
    _check(lib.moe_w4a4_forward(ctypes.byref(sh), _ptr(x), _ptr(router_logits), _ptr(w13_q), _ptr(w13_s),
                                _ptr(w2_q), _ptr(w2_s), _ptr(out), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)))
    return out
