"""Dense W4A16 GEMM (moe_w4a16_dense_gemm) on the GPU vs the oracle.

The dense GEMM is the grouped GEMM with one expert holding every row, so the
oracle is oracle.grouped_gemm with E = 1 (itself pinned to a plain fp64
matmul on the dequantised weights).

- Integer-exact pin: activations in {-2..2}, codes in [-8, 7], scales 2^-6:
  every partial sum is exact in fp32, so the fp32 output is bit-exact.
- Random bf16 activations: within an error bound derived from the kernel's
  arithmetic (below), fp32 and bf16 outputs.
- The dense entry point equals the grouped GEMM with offsets {0, M} bit for
  bit, and the tiled code layout equals the plain one bit for bit through
  the same kernel (the prefill tile kernel, with its own summation order,
  is held to the bound instead).
"""
import numpy as np
import pytest

import oracle
from helpers import bf16_dev, bf16_to_f64, say, to_dev, to_np_u16
from w4a16_grouped_gemm_amd.inputs import bf16_bits, pack_int4

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _dense(a_u16, wq, s, *, out_f32, tiled=False):
    import torch
    from w4a16_grouped_gemm_amd import ops
    w = to_dev(wq)
    if tiled:
        w = ops.pack_dense_weights(w)
    out = ops.dense_gemm_w4a16(bf16_dev(a_u16), w, bf16_dev(s),
                               out_dtype=torch.float32 if out_f32 else torch.bfloat16,
                               weight_layout=ops.WEIGHTS_TILED if tiled else ops.WEIGHTS_PLAIN)
    torch.cuda.synchronize()
    return out.cpu().numpy() if out_f32 else to_np_u16(out)


def _inputs(M, N, K, seed, integer=False):
    rng = np.random.default_rng(seed)
    q = rng.integers(-8, 8, size=(N, K), dtype=np.int8)
    if integer:
        a = bf16_bits(rng.integers(-2, 3, size=(M, K)).astype(np.float32))
        s = np.full((N, K // 128), bf16_bits(np.float32(2.0 ** -6)), np.uint16)
    else:
        a = bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        s = bf16_bits(rng.uniform(0.005, 0.02, size=(N, K // 128)).astype(np.float32))
    return q, a, s


def _error_bound(q, a_u16, s_u16):
    # Per group g the kernel accumulates, in fp32 on the matrix unit, the
    # 2*128 exact products (-136)*x and (136+q)*x (|each| <= 144|x|), then
    # applies the scale with one fp32 FMA per group: tot = fma(s_g, acc_g, tot).
    # Bound: |err(acc_g)| <= 2*256*u*144*sum_{k in g}|x_k| (a conservative
    # sequential-summation bound over 256 terms, doubled for the intermediate
    # roundings of the MFMA chain), and the G FMAs add <= (G+2)*u*sum_g|s_g acc_g|
    # with sum_g |s_g acc_g| <= sum_k |s x q|.
    x = np.abs(bf16_to_f64(a_u16))
    sc = bf16_to_f64(s_u16)
    K = x.shape[1]
    G = K // 128
    sk = np.repeat(sc, 128, axis=1)                       # [N, K] scale of each column
    s1 = x @ sk.T                                         # sum_k |x_k| s_g(k)
    s2 = x @ (np.abs(q).astype(np.float64) * sk).T        # sum_k |x_k q_k| s_g(k)
    return U * (512 * 144 * s1 + (G + 2) * s2)


def _oracle(q, a_u16, s_u16, out_f32, row_sel=None):
    M = a_u16.shape[0]
    N = q.shape[0]
    offsets = np.array([0, M], np.int32)
    return oracle.grouped_gemm(oracle.W2, a_u16, offsets, pack_int4(q[None]), s_u16[None], rows=M,
                               out_f32=out_f32, row_sel=row_sel)


SHAPES = [(1, 128, 128), (17, 256, 512), (100, 2048, 768), (256, 1024, 2048), (1000, 512, 4096)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("tiled", [False, True])
def test_dense_integer_exact(M, N, K, tiled):
    say(f"dense integer-exact M={M} N={N} K={K} tiled={tiled}")
    q, a, s = _inputs(M, N, K, M + N + K, integer=True)
    got = _dense(a, pack_int4(q), s, out_f32=True, tiled=tiled)
    want = (bf16_to_f64(a).astype(np.int64) @ q.T.astype(np.int64)).astype(np.float64) * 2.0 ** -6
    assert np.array_equal(got.astype(np.float64), want)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_dense_vs_oracle_within_bound(M, N, K):
    say(f"dense vs oracle M={M} N={N} K={K}")
    q, a, s = _inputs(M, N, K, 7 * M + N + K)
    ref = _oracle(q, a, s, out_f32=True).astype(np.float64)   # fp32-rounded fp64 result
    bound = _error_bound(q, a, s) + np.abs(ref) * U           # + the oracle's own fp32 rounding
    got = _dense(a, pack_int4(q), s, out_f32=True)
    err = np.abs(got.astype(np.float64) - ref)
    say(f"  max err / bound {np.max(err / bound):.3e}")
    assert np.all(err <= bound)
    # bf16 output: the fp32 result v rounded once more, |RNE(v) - v| <= 2^-8 |v|
    # and |v| <= |ref| + bound
    got16 = bf16_to_f64(_dense(a, pack_int4(q), s, out_f32=False))
    assert np.all(np.abs(got16 - ref) <= bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref))


def test_dense_equals_one_expert_grouped_gemm():
    import torch
    from w4a16_grouped_gemm_amd import ops
    say("dense == grouped GEMM with one expert")
    M, N, K = 300, 2048, 2048
    q, a, s = _inputs(M, N, K, 5)
    wq = pack_int4(q)
    got = _dense(a, wq, s, out_f32=False)
    grouped = ops.grouped_gemm_w4a16(ops.W2, bf16_dev(a), to_dev(np.array([0, M], np.int32)), to_dev(wq[None]),
                                     bf16_dev(s[None]), num_tokens=M, top_k=1)
    torch.cuda.synchronize()
    assert np.array_equal(got, to_np_u16(grouped))
    # at 300 rows tiled codes with bf16 output take the tile kernel (its own
    # summation order): within the bound of the oracle
    ref = _oracle(q, a, s, out_f32=True).astype(np.float64)
    bound = _error_bound(q, a, s) + np.abs(ref) * U
    tile = bf16_to_f64(_dense(a, wq, s, out_f32=False, tiled=True))
    assert np.all(np.abs(tile - ref) <= bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref))
    # through the streaming kernel the tiled layout equals the plain one bit for bit
    with ops.launch_override(gemm_mode=1):
        assert np.array_equal(got, _dense(a, wq, s, out_f32=False, tiled=True))


def test_dense_zero_rows_and_errors():
    import torch
    from w4a16_grouped_gemm_amd import ops
    say("dense M=0 and argument errors")
    q, a, s = _inputs(4, 256, 256, 3)
    empty = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    out = ops.dense_gemm_w4a16(empty, to_dev(pack_int4(q)), bf16_dev(s))
    assert out.shape == (0, 256)
    with pytest.raises(ValueError):                       # weights do not match K
        ops.dense_gemm_w4a16(bf16_dev(a), to_dev(pack_int4(q))[:, :64], bf16_dev(s))
    torch.cuda.synchronize()


def test_dense_full_size_sampled_rows():
    # the measured shape (256 x 14336 x 4096): the oracle computes 16 sampled rows
    say("dense full size, sampled rows")
    M, N, K = 256, 14336, 4096
    q, a, s = _inputs(M, N, K, 11)
    sel = np.zeros(M, np.uint8)
    rows = np.unique(np.linspace(0, M - 1, 16).astype(int))
    sel[rows] = 1
    ref = _oracle(q, a, s, out_f32=True, row_sel=sel).astype(np.float64)[rows]
    bound = _error_bound(q, a[rows], s) + np.abs(ref) * U
    got = _dense(a, pack_int4(q), s, out_f32=True, tiled=True)[rows].astype(np.float64)
    assert np.all(np.abs(got - ref) <= bound)
