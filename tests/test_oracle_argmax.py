"""Pins of oracle.argmax_rows (greedy token per row of the lm_head GEMM; "SparkInfer" README,
greedy decode and verification), against things fixed independently of the oracle:

  * brute force: a pure-Python scan keeping the first strictly larger value, on small matrices
    drawn from a handful of integers so that ties are frequent;
  * construction: packed weights whose winning column is known without computing anything (one
    column holds the largest code at the largest scale where the one-hot row is 1);
  * sign: all-negative rows pick the value closest to zero (a mistake taking |Y| fails);
  * -0 and +0 are equal, so the earlier column wins.
"""
import numpy as np
import pytest
import torch

import oracle
from skinny_gemm_nvfp4_amd import inputs


def _brute_argmax(row):
    best = 0
    for n in range(1, len(row)):
        if row[n] > row[best]:
            best = n
    return best


@pytest.mark.parametrize("seed", range(5))
def test_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    Y = rng.integers(-3, 4, size=(17, 23)).astype(np.float64)
    got = oracle.argmax_rows(Y)
    assert [int(v) for v in got] == [_brute_argmax(list(r)) for r in Y]


def test_negative_rows_and_signed_zero():
    Y = np.array([[-5.0, -0.25, -3.0, -0.25],
                  [-0.0, 0.0, -1.0, 0.0],
                  [0.0, -0.0, -1.0, 2.0 ** -149]])
    assert oracle.argmax_rows(Y).tolist() == [1, 0, 3]


def test_rejects_nan_and_empty():
    with pytest.raises(ValueError):
        oracle.argmax_rows(np.array([[0.0, np.nan]]))
    with pytest.raises(ValueError):
        oracle.argmax_rows(np.zeros((2, 0)))


@pytest.mark.parametrize("K,N", [(64, 37), (512, 1000)])
def test_constructed_winner_through_the_gemm(K, N):
    """Plain-layout bytes: codes 0x1 (0.5) everywhere at scale byte 0x38 (1.0); column n_m gets
    code 0x7 (6.0) at k_m with scale byte 0x7E (448) on that block. With X one-hot at k_m, row m's
    largest output is column n_m by construction (6 * 448 against at most 0.5 * 448)."""
    Wq = np.full((N, K // 2), 0x11, dtype=np.uint8)
    Ws = np.full((N, K // 16), 0x38, dtype=np.uint8)
    M = 6
    rng = np.random.default_rng(K + N)
    ks = rng.choice(K, size=M, replace=False)
    ns = rng.choice(N, size=M, replace=False)
    X = np.zeros((M, K), dtype=np.float32)
    for m in range(M):
        X[m, ks[m]] = 1.0
        k, n = ks[m], ns[m]
        shift = 4 * (k % 2)
        Wq[n, k // 2] = (Wq[n, k // 2] & ~(0xF << shift)) | (0x7 << shift)
        Ws[:, k // 16] = np.where(np.arange(N) == n, 0x7E, Ws[:, k // 16])
    Xb = inputs.bf16_bits(torch.from_numpy(X).to(torch.bfloat16))
    Y, _ = oracle.gemm(Xb, Wq, Ws, 1.0)
    assert oracle.argmax_rows(Y).tolist() == [int(n) for n in ns]
    # every other scale byte of the constructed blocks is 448 only in its own column
    assert np.all(Y[np.arange(M), ns] == 6.0 * 448.0)
