"""CPU oracle for the W4A16 MoE expert layer (ctypes wrapper over moe_oracle.c).

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. It never imports the GPU package and
the GPU package never imports it; the two share only the seeded input
generators, which hold none of the layer's arithmetic.

bf16 tensors are passed as numpy uint16 bit patterns. Every function here is a
thin marshalling layer; the arithmetic lives in moe_oracle.c, whose header
cites the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_SRCS = [_SRC, os.path.join(_HERE, "mxfp4_oracle.c")]
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

W13_SWIGLU, W2, RAW = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", tmp, *_SRCS, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(os.path.getmtime(f) for f in _SRCS):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_bf16_from_double.argtypes = [ctypes.c_double]
    lib.oracle_bf16_from_double.restype = ctypes.c_uint16
    lib.oracle_set_threads.argtypes = [I]
    lib.oracle_get_threads.restype = I
    lib.oracle_route.argtypes = [I, I, I, P, P, P]
    lib.oracle_permute.argtypes = [I, I, I, I, P, P, P, P, P]
    lib.oracle_grouped_gemm.argtypes = [I, I, I, I, I, P, P, I, P, P, P, P, P, I]
    lib.oracle_finalize.argtypes = [I, I, I, P, I, P, P, I, P, P, P, I]
    lib.oracle_layer.argtypes = [I] * 8 + [P] * 6 + [I] + [P] * 4 + [P] + [P] * 10
    lib.oracle_layer_bruteforce.argtypes = [I] * 7 + [P] * 7 + [I] + [P] * 4 + [P] * 2
    lib.oracle_e2m1_value.argtypes = [I]
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e8m0_value.argtypes = [I]
    lib.oracle_e8m0_value.restype = ctypes.c_double
    lib.oracle_mx_quantize.argtypes = [ctypes.c_int64, I, P, P, P]
    lib.oracle_grouped_gemm_mxfp4.argtypes = [I, I, I, I, P, P, P, I, P, P, P, P, P, I]
    lib.oracle_layer_w4a4.argtypes = [I] * 7 + [P] * 7 + [P] * 13
    lib.oracle_layer_w4a4_bruteforce.argtypes = [I] * 6 + [P] * 7 + [P] * 2
    _lib = lib
    return lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def bf16_from_double(d: float) -> int:
    """Single round-to-nearest-even of a double to a bf16 bit pattern."""
    return int(_load().oracle_bf16_from_double(float(d)))


def route(logits: np.ndarray, top_k: int):
    """Top-k routing: returns (topk_ids int32 [T,k], topk_w float32 [T,k])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float32)
    _load().oracle_route(T, E, top_k, _ptr(logits), _ptr(ids), _ptr(w))
    return ids, w


def permute(topk_ids: np.ndarray, num_local_experts: int, expert_begin: int = 0):
    """Stable expert bucketing: returns counts, offsets, perm, inv_perm."""
    topk_ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    T, k = topk_ids.shape
    counts = np.empty(num_local_experts, np.int32)
    offsets = np.empty(num_local_experts + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv_perm = np.empty((T, k), np.int32)
    _load().oracle_permute(T, k, expert_begin, num_local_experts, _ptr(topk_ids), _ptr(counts),
                           _ptr(offsets), _ptr(perm), _ptr(inv_perm))
    return counts, offsets, perm, inv_perm


def grouped_gemm(kind: int, a: np.ndarray, offsets: np.ndarray, wq: np.ndarray, s: np.ndarray,
                 *, rows: int, a_row_index: np.ndarray | None = None, top_k: int = 1,
                 out_f32: bool = False, row_sel: np.ndarray | None = None, group: int = 128,
                 out: np.ndarray | None = None):
    """Grouped GEMM over expert slabs (see oracle_grouped_gemm in moe_oracle.c).

    wq: uint8 [E_loc, N, K/2]; s: uint16 (bf16) [E_loc, N, K/group]; a: uint16 [*, K].
    Returns c [rows, out_cols] as float32 or uint16 (bf16); rows not computed stay 0.
    """
    E_loc, N, K2 = wq.shape
    K = 2 * K2
    out_cols = N // 2 if kind == W13_SWIGLU else N
    if out is None:
        out = np.zeros((rows, out_cols), np.float32 if out_f32 else np.uint16)
    a = np.ascontiguousarray(a, dtype=np.uint16)
    assert a.shape[-1] == K
    idx = None if a_row_index is None else np.ascontiguousarray(a_row_index, dtype=np.int32)
    sel = None if row_sel is None else np.ascontiguousarray(row_sel, dtype=np.uint8)
    _load().oracle_grouped_gemm(kind, E_loc, N, K, group, _ptr(a), _ptr(idx), top_k,
                                _ptr(np.ascontiguousarray(offsets, dtype=np.int32)),
                                _ptr(np.ascontiguousarray(wq)), _ptr(np.ascontiguousarray(s)),
                                _ptr(sel), _ptr(out), 1 if out_f32 else 0)
    return out


def finalize(y: np.ndarray, topk_w: np.ndarray, inv_perm: np.ndarray, *, out_f32: bool,
             tok_sel: np.ndarray | None = None, ys: np.ndarray | None = None):
    """Slot-ordered combine. y: float32 or uint16 (bf16) [R, H]; ys: the shared
    experts' outputs [S, T, H] in y's dtype (added after the slots), or None."""
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    inv_perm = np.ascontiguousarray(inv_perm, dtype=np.int32)
    T, k = topk_w.shape
    H = y.shape[-1]
    y_f32 = y.dtype == np.float32
    assert y_f32 or y.dtype == np.uint16
    out = np.zeros((T, H), np.float32 if out_f32 else np.uint16)
    sel = None if tok_sel is None else np.ascontiguousarray(tok_sel, dtype=np.uint8)
    S = 0 if ys is None else ys.shape[0]
    if ys is not None:
        assert ys.dtype == y.dtype and ys.shape == (S, T, H)
    _load().oracle_finalize(T, k, H, _ptr(np.ascontiguousarray(y)), 1 if y_f32 else 0, _ptr(topk_w),
                            _ptr(inv_perm), S, _ptr(None if ys is None else np.ascontiguousarray(ys)), _ptr(sel),
                            _ptr(out), 1 if out_f32 else 0)
    return out


def _shared_args(shared):
    """(S, w13_sh, s13_sh, w2_sh, s2_sh) pointers for an optional shared-expert tuple."""
    if shared is None:
        return 0, None, None, None, None
    w13, s13, w2, s2 = (np.ascontiguousarray(a) for a in shared)
    return w13.shape[0], w13, s13, w2, s2


def layer(x, logits, w13_q, s13, w2_q, s2, *, top_k: int, expert_begin: int = 0,
          tok_sel: np.ndarray | None = None, group: int = 128, shared=None):
    """The whole layer through the permutation; returns a dict of every stage.

    shared: optional (w13_sh [S, 2I, H/2], s13_sh, w2_sh [S, H, I/2], s2_sh):
    S always-on experts added after the routed slots (hs, ys in the result)."""
    T, H = x.shape
    E_g = logits.shape[1]
    E_loc, N13, _ = w13_q.shape
    I = N13 // 2
    S = T * top_k
    r = dict(
        topk_ids=np.empty((T, top_k), np.int32), topk_w=np.empty((T, top_k), np.float32),
        counts=np.empty(E_loc, np.int32), offsets=np.empty(E_loc + 1, np.int32),
        perm=np.empty(S, np.int32), inv_perm=np.empty((T, top_k), np.int32),
        h=np.zeros((S, I), np.uint16), y=np.zeros((S, H), np.uint16), out=np.zeros((T, H), np.uint16))
    nsh, w13s, s13s, w2s, s2s = _shared_args(shared)
    r["hs"] = np.zeros((nsh, T, I), np.uint16)
    r["ys"] = np.zeros((nsh, T, H), np.uint16)
    sel = None if tok_sel is None else np.ascontiguousarray(tok_sel, dtype=np.uint8)
    _load().oracle_layer(T, E_g, top_k, expert_begin, E_loc, H, I, group,
                         _ptr(np.ascontiguousarray(x, dtype=np.uint16)),
                         _ptr(np.ascontiguousarray(logits, dtype=np.float32)),
                         _ptr(np.ascontiguousarray(w13_q)), _ptr(np.ascontiguousarray(s13)),
                         _ptr(np.ascontiguousarray(w2_q)), _ptr(np.ascontiguousarray(s2)),
                         nsh, _ptr(w13s), _ptr(s13s), _ptr(w2s), _ptr(s2s), _ptr(sel),
                         _ptr(r["topk_ids"]), _ptr(r["topk_w"]), _ptr(r["counts"]), _ptr(r["offsets"]),
                         _ptr(r["perm"]), _ptr(r["inv_perm"]), _ptr(r["h"]), _ptr(r["y"]),
                         _ptr(r["hs"] if nsh else None), _ptr(r["ys"] if nsh else None), _ptr(r["out"]))
    return r


def layer_bruteforce(x, topk_ids, topk_w, w13_q, s13, w2_q, s2, *, expert_begin: int = 0,
                     tok_sel: np.ndarray | None = None, group: int = 128, shared=None):
    """Naive per-(token, slot) expert MLPs + ordered combine; no permutation."""
    T, H = x.shape
    k = topk_ids.shape[1]
    E_loc, N13, _ = w13_q.shape
    I = N13 // 2
    out = np.zeros((T, H), np.uint16)
    sel = None if tok_sel is None else np.ascontiguousarray(tok_sel, dtype=np.uint8)
    _load().oracle_layer_bruteforce(T, k, expert_begin, E_loc, H, I, group,
                                    _ptr(np.ascontiguousarray(x, dtype=np.uint16)),
                                    _ptr(np.ascontiguousarray(topk_ids, dtype=np.int32)),
                                    _ptr(np.ascontiguousarray(topk_w, dtype=np.float32)),
                                    _ptr(np.ascontiguousarray(w13_q)), _ptr(np.ascontiguousarray(s13)),
                                    _ptr(np.ascontiguousarray(w2_q)), _ptr(np.ascontiguousarray(s2)),
                                    *_shared_ptrs(shared), _ptr(sel), _ptr(out))
    return out


def _shared_ptrs(shared):
    nsh, w13s, s13s, w2s, s2s = _shared_args(shared)
    return nsh, _ptr(w13s), _ptr(s13s), _ptr(w2s), _ptr(s2s)


# ---------------------------------------------------------------------------
# W4A4 (MXFP4) variant -- see mxfp4_oracle.c for the format reading
# ---------------------------------------------------------------------------

def e2m1_value(code: int) -> float:
    return float(_load().oracle_e2m1_value(int(code)))


def e8m0_value(s: int) -> float:
    return float(_load().oracle_e8m0_value(int(s)))


def mx_quantize(x: np.ndarray):
    """bf16 rows [R, K] (K % 32 == 0) -> (codes uint8 [R, K/2], scales uint8 [R, K/32])."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    R, K = x.shape
    codes = np.empty((R, K // 2), np.uint8)
    scales = np.empty((R, K // 32), np.uint8)
    _load().oracle_mx_quantize(R, K, _ptr(x), _ptr(codes), _ptr(scales))
    return codes, scales


def grouped_gemm_mxfp4(kind: int, a_codes, a_scales, offsets, wq, ws, *, rows: int, a_row_index=None,
                       top_k: int = 1, out_f32: bool = False, row_sel=None):
    """Grouped GEMM on MXFP4 activations and weights (oracle_grouped_gemm_mxfp4)."""
    E_loc, N, K2 = wq.shape
    K = 2 * K2
    out_cols = N // 2 if kind == W13_SWIGLU else N
    out = np.zeros((rows, out_cols), np.float32 if out_f32 else np.uint16)
    idx = None if a_row_index is None else np.ascontiguousarray(a_row_index, dtype=np.int32)
    sel = None if row_sel is None else np.ascontiguousarray(row_sel, dtype=np.uint8)
    _load().oracle_grouped_gemm_mxfp4(kind, E_loc, N, K, _ptr(np.ascontiguousarray(a_codes)),
                                      _ptr(np.ascontiguousarray(a_scales)), _ptr(idx), top_k,
                                      _ptr(np.ascontiguousarray(offsets, dtype=np.int32)),
                                      _ptr(np.ascontiguousarray(wq)), _ptr(np.ascontiguousarray(ws)), _ptr(sel),
                                      _ptr(out), 1 if out_f32 else 0)
    return out


def layer_w4a4(x, logits, w13_q, w13_s, w2_q, w2_s, *, top_k: int, expert_begin: int = 0, tok_sel=None):
    """The W4A4 (MXFP4) layer through the permutation; a dict of every stage."""
    T, H = x.shape
    E_g = logits.shape[1]
    E_loc, N13, _ = w13_q.shape
    I = N13 // 2
    S = T * top_k
    r = dict(topk_ids=np.empty((T, top_k), np.int32), topk_w=np.empty((T, top_k), np.float32),
             counts=np.empty(E_loc, np.int32), offsets=np.empty(E_loc + 1, np.int32),
             perm=np.empty(S, np.int32), inv_perm=np.empty((T, top_k), np.int32),
             xq=np.zeros((T, H // 2), np.uint8), xs=np.zeros((T, H // 32), np.uint8),
             h=np.zeros((S, I), np.uint16), hq=np.zeros((S, I // 2), np.uint8), hs=np.zeros((S, I // 32), np.uint8),
             y=np.zeros((S, H), np.uint16), out=np.zeros((T, H), np.uint16))
    sel = None if tok_sel is None else np.ascontiguousarray(tok_sel, dtype=np.uint8)
    _load().oracle_layer_w4a4(T, E_g, top_k, expert_begin, E_loc, H, I,
                              _ptr(np.ascontiguousarray(x, dtype=np.uint16)),
                              _ptr(np.ascontiguousarray(logits, dtype=np.float32)),
                              _ptr(np.ascontiguousarray(w13_q)), _ptr(np.ascontiguousarray(w13_s)),
                              _ptr(np.ascontiguousarray(w2_q)), _ptr(np.ascontiguousarray(w2_s)), _ptr(sel),
                              _ptr(r["topk_ids"]), _ptr(r["topk_w"]), _ptr(r["counts"]), _ptr(r["offsets"]),
                              _ptr(r["perm"]), _ptr(r["inv_perm"]), _ptr(r["xq"]), _ptr(r["xs"]), _ptr(r["h"]),
                              _ptr(r["hq"]), _ptr(r["hs"]), _ptr(r["y"]), _ptr(r["out"]))
    return r


def layer_w4a4_bruteforce(x, topk_ids, topk_w, w13_q, w13_s, w2_q, w2_s, *, expert_begin: int = 0,
                          tok_sel=None):
    """Per (token, slot) W4A4 expert FFNs + ordered combine; no permutation."""
    T, H = x.shape
    k = topk_ids.shape[1]
    E_loc, N13, _ = w13_q.shape
    I = N13 // 2
    out = np.zeros((T, H), np.uint16)
    sel = None if tok_sel is None else np.ascontiguousarray(tok_sel, dtype=np.uint8)
    _load().oracle_layer_w4a4_bruteforce(T, k, expert_begin, E_loc, H, I,
                                         _ptr(np.ascontiguousarray(x, dtype=np.uint16)),
                                         _ptr(np.ascontiguousarray(topk_ids, dtype=np.int32)),
                                         _ptr(np.ascontiguousarray(topk_w, dtype=np.float32)),
                                         _ptr(np.ascontiguousarray(w13_q)), _ptr(np.ascontiguousarray(w13_s)),
                                         _ptr(np.ascontiguousarray(w2_q)), _ptr(np.ascontiguousarray(w2_s)),
                                         _ptr(sel), _ptr(out))
    return out
