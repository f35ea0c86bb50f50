"""Pins of the oracle GEMM (double accumulation) against library routines and closed forms.

  * Special case that reduces to a library matmul: weights decoded here (OCP table + torch
    float8_e4m3fn, numpy nibble unpacking) and multiplied with numpy's float64 matmul; A against
    |X| @ |W|. Non-square shapes catch transposed operands and swapped indices.
  * Exact integer sums: scales in {0.5, 1, 2}, g = 1, integer X -> Y*4 equals an int64 matmul.
  * One-hot rows return the dequantised weights; sign, scaling and column-subset invariants.
  * The tolerance's closed form: recursive fp32 summation error (K-1) 2^-24 sum|x w| stays below
    the acceptance bound 2e-3 sum|x w| for every K of the workloads.
"""
import numpy as np
import torch

import oracle
from golden_data import e2m1_table
from skinny_gemm_nvfp4_amd import inputs

TABLE = e2m1_table()


def _decode_here(Wq, Ws, g):
    N, Kh = Wq.shape
    codes = np.empty((N, 2 * Kh), dtype=np.uint8)
    codes[:, 0::2] = Wq & 0x0F
    codes[:, 1::2] = Wq >> 4
    s = torch.from_numpy(np.ascontiguousarray(Ws)).view(torch.float8_e4m3fn)
    s = s.to(torch.float64).numpy()
    return (TABLE[codes] * np.repeat(s, 16, axis=1) * float(g)).T   # [K][N]


def test_matches_library_matmul():
    for seed, (M, N, K) in enumerate([(1, 7, 16), (3, 33, 96), (16, 40, 512), (5, 9, 1040)]):
        gen = inputs.generator(seed)
        Wq, Ws = inputs.random_packed(gen, N, K, scale_bytes=range(0x7F))
        X = inputs.activations(gen, M, K)
        g = 0.0123
        Y, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g)
        Wd = _decode_here(Wq.numpy(), Ws.numpy(), np.float32(g))
        Xd = X.to(torch.float64).numpy()
        Yl = Xd @ Wd
        Al = np.abs(Xd) @ np.abs(Wd)
        assert np.allclose(Y, Yl, rtol=0, atol=1e-12 * Al.max())
        assert np.allclose(A, Al, rtol=1e-12, atol=0)


def test_exact_integer_sums_match_int64_matmul():
    M, N, K = 6, 21, 1024
    gen = inputs.generator(42)
    Wq, Ws = inputs.random_packed(gen, N, K, scale_bytes=[0x30, 0x38, 0x40])
    X = inputs.integer_activations(gen, M, K)
    Y, _ = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), 1.0)
    Wd4 = _decode_here(Wq.numpy(), Ws.numpy(), 1.0) * 4          # integers
    assert np.array_equal(Wd4, np.rint(Wd4))
    Yint = X.to(torch.int64).numpy() @ Wd4.astype(np.int64)
    assert np.array_equal(Y * 4, Yint.astype(np.float64))


def test_one_hot_and_invariants():
    M, N, K = 4, 24, 256
    gen = inputs.generator(9)
    Wq, Ws = inputs.random_packed(gen, N, K, scale_bytes=range(0x7F))
    g = np.float32(0.37)
    Wd = oracle.dequantize(Wq.numpy(), Ws.numpy(), g)
    assert np.array_equal(Wd, _decode_here(Wq.numpy(), Ws.numpy(), g))
    ks = [0, 17, 100, 255]
    X = torch.zeros(M, K, dtype=torch.bfloat16)
    X[torch.arange(M), ks] = 1.0
    Y, _ = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g)
    assert np.array_equal(Y, Wd[ks, :])

    X = inputs.activations(gen, M, K)
    Y, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g)
    Yn, An = oracle.gemm(inputs.bf16_bits(-X), Wq.numpy(), Ws.numpy(), g)
    Y2, _ = oracle.gemm(inputs.bf16_bits(X * 2), Wq.numpy(), Ws.numpy(), g)
    Yg, _ = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g * 2)
    assert np.array_equal(Yn, -Y) and np.array_equal(An, A)
    assert np.array_equal(Y2, 2 * Y) and np.array_equal(Yg, 2 * Y)
    cols = np.array([23, 0, 5], dtype=np.int32)
    Yc, Ac = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g, cols=cols)
    assert np.array_equal(Yc, Y[:, cols]) and np.array_equal(Ac, A[:, cols])


def test_tolerance_admits_any_fp32_summation_order():
    for K in (1024, 5120, 17408):
        assert (K - 1) * 2.0 ** -24 < 2e-3
    assert oracle.tolerance(np.array([0.0]))[0] == 1e-6
