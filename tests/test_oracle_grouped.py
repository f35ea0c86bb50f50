"""Pins of oracle.grouped_gemm (mixture-of-experts grouped GEMM; "SparkInfer" README, section
"Layout & scoring": fused MoE FFN kernel, router with expert dispatch), against facts fixed
outside the function:

  * brute force: every row recomputed as a float64 dot product of its bf16 x with the exactly
    dequantised weights of the expert that owns the row (oracle.dequantize, pinned on its own);
  * a row's result depends only on its expert: moving a row to another expert's block changes it
    to that expert's result, and experts with no rows take no part;
  * identical experts reduce to the plain GEMM over all rows;
  * bad offsets are rejected.
"""
import numpy as np
import pytest
import torch

import oracle
from skinny_gemm_nvfp4_amd import inputs


def _case(seed, E, T, N, K):
    gen = inputs.generator(seed)
    Wq = np.stack([inputs.random_packed(gen, N, K, scale_bytes=list(range(0x20, 0x48)))[0].numpy()
                   for _ in range(E)])
    Ws = np.stack([inputs.random_packed(gen, N, K, scale_bytes=list(range(0x20, 0x48)))[1].numpy()
                   for _ in range(E)])
    g = np.array([0.01 * (e + 1) for e in range(E)], dtype=np.float32)
    X = inputs.activations(gen, T, K)
    return inputs.bf16_bits(X), X, Wq, Ws, g


def test_matches_brute_force_rows():
    E, T, N, K = 5, 9, 13, 64
    xb, X, Wq, Ws, g = _case(1, E, T, N, K)
    offsets = [0, 2, 2, 6, 7, 9]           # expert 1 has no rows
    Y, A = oracle.grouped_gemm(xb, offsets, Wq, Ws, g)
    x64 = X.to(torch.float64).numpy()
    for e in range(E):
        Wd = oracle.dequantize(Wq[e], Ws[e], g[e])          # exact [K][N]
        for t in range(offsets[e], offsets[e + 1]):
            want = np.array([sum(x64[t, k] * Wd[k, n] for k in range(K)) for n in range(N)])
            assert np.allclose(Y[t], want, rtol=0, atol=1e-12 * (1 + np.abs(want).max()))
            assert np.allclose(A[t], np.abs(x64[t][:, None] * Wd).sum(axis=0), rtol=1e-12)


def test_rows_follow_their_expert():
    E, T, N, K = 3, 4, 8, 32
    xb, _, Wq, Ws, g = _case(2, E, T, N, K)
    Y1, _ = oracle.grouped_gemm(xb, [0, 2, 4, 4], Wq, Ws, g)
    Y2, _ = oracle.grouped_gemm(xb, [0, 1, 4, 4], Wq, Ws, g)
    assert np.array_equal(Y1[0], Y2[0]) and np.array_equal(Y1[2:], Y2[2:])
    assert not np.array_equal(Y1[1], Y2[1])            # row 1 moved from expert 0 to 1
    Y3, _ = oracle.grouped_gemm(xb, [0, 0, 0, 4], Wq, Ws, g)
    Yp, _ = oracle.gemm(xb, Wq[2], Ws[2], g[2])
    assert np.array_equal(Y3, Yp)


def test_identical_experts_reduce_to_plain_gemm():
    E, T, N, K = 4, 7, 10, 48
    xb, _, Wq, Ws, g = _case(3, E, T, N, K)
    Wq[:] = Wq[0]
    Ws[:] = Ws[0]
    Y, _ = oracle.grouped_gemm(xb, [0, 3, 3, 5, 7], Wq, Ws, np.float32(0.5))
    Yp, _ = oracle.gemm(xb, Wq[0], Ws[0], 0.5)
    assert np.array_equal(Y, Yp)


@pytest.mark.parametrize("offsets", [[0, 2, 1, 4], [1, 2, 3, 4], [0, 1, 2, 5], [0, 4]])
def test_rejects_bad_offsets(offsets):
    xb, _, Wq, Ws, g = _case(4, 3, 4, 8, 32)
    with pytest.raises(ValueError):
        oracle.grouped_gemm(xb, offsets, Wq, Ws, g)
