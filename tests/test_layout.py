"""The test-side conversion between the oracle's plain byte layout and the library's packed
layout, checked element by element against the layout's definition in include/nvfp4.h."""
import numpy as np

from skinny_gemm_nvfp4_amd import binding
import torch
import pytest

from parity import from_library_layout, to_library_layout


@pytest.mark.parametrize("N,K", [(1, 16), (4, 32), (5, 48), (9, 96), (13, 272)])
def test_layout_matches_header_definition(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    Wq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    Ws = rng.integers(0, 256, size=(N, K // 16), dtype=np.uint8)
    q, s = to_library_layout(Wq, Ws, K)
    NG, CH = -(-N // 4), -(-K // 32)
    assert q.shape == (NG, CH, 4, 16) and s.shape == (NG, CH, 4, 2)
    # Byte (g, c, j, i): codes of column 4g + j at k = 32c + 2i (low nibble) and 32c + 2i + 1.
    for g in range(NG):
        for c in range(CH):
            for j in range(4):
                n = 4 * g + j
                for i in range(16):
                    k = 32 * c + 2 * i
                    want = Wq[n, k // 2] if (n < N and k < K) else 0
                    assert q[g, c, j, i] == want
                for b in range(2):
                    blk = 2 * c + b
                    want = Ws[n, blk] if (n < N and 16 * blk < K) else 0
                    assert s[g, c, j, b] == want
    back_q, back_s, pad_zero = from_library_layout(q, s, N, K)
    assert pad_zero
    assert np.array_equal(back_q, Wq) and np.array_equal(back_s, Ws)


def test_nonzero_padding_is_reported():
    Wq = np.zeros((5, 8), dtype=np.uint8)
    Ws = np.zeros((5, 1), dtype=np.uint8)
    q, s = to_library_layout(Wq, Ws, 16)
    q[1, 0, 3, 0] = 1          # column 7 >= N = 5
    assert not from_library_layout(q, s, 5, 16)[2]
    q[1, 0, 3, 0] = 0
    s[0, 0, 0, 1] = 0x38       # block 1 of a K = 16 matrix
    assert not from_library_layout(q, s, 5, 16)[2]


def test_interleave_is_a_column_permutation():
    """interleave_gate_up only moves columns: gate column j lands at 8 (j // 4) + j % 4, up
    column j at that + 4."""
    K, I = 3, 12
    W = torch.arange(K * 2 * I, dtype=torch.float32).reshape(K, 2 * I)
    Wi = binding.interleave_gate_up(W)
    for j in range(I):
        assert torch.equal(Wi[:, 8 * (j // 4) + j % 4], W[:, j])
        assert torch.equal(Wi[:, 8 * (j // 4) + 4 + j % 4], W[:, I + j])
