"""The workloads at full size: GPU pack bit-exact against the oracle, then GPU GEMM against the
oracle GEMM (every column where the oracle finishes in seconds, else a seeded column sample that
includes both ends of N). The GEMM runs through nvfp4_gemm, the entry point the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
from skinny_gemm_nvfp4_amd import inputs
from parity import assert_pack_equal, check_close, gpu_gemm, say

pytestmark = pytest.mark.gpu


def _columns(N: int, sample: int, seed: int):
    if sample is None or sample >= N:
        return None
    gen = inputs.generator(seed)
    mid = torch.randperm(N, generator=gen)[:sample].numpy()
    ends = np.r_[np.arange(16), np.arange(N - 16, N)]
    return np.unique(np.r_[mid, ends]).astype(np.int32)


def _run(workload, device, sample=None):
    for gm in workload.gemms:
        M, N, K = gm.shape
        (packed_d, packed_o) = assert_pack_equal(gm.W, device, f"{workload.name}.{gm.name}")
        say(f"gemm {workload.name}.{gm.name} M={M} N={N} K={K}")
        Y = gpu_gemm(gm.X, packed_d, device)
        cols = _columns(N, sample, seed=N + K + M)
        Wq_o, Ws_o, g_o = packed_o
        Yref, A = oracle.gemm(inputs.bf16_bits(gm.X), Wq_o, Ws_o, g_o, cols=cols)
        Ysel = Y if cols is None else Y[:, cols]
        worst = check_close(Ysel, Yref, A, f"{workload.name}.{gm.name}")
        say(f"  worst error / bound = {worst:.3g}")


def test_single_gemv(device):
    _run(inputs.single_gemv(), device)


def test_dense_layer_m1(device):
    _run(inputs.dense_layer_m1(), device)


def test_verify_m16(device):
    _run(inputs.verify_m16(), device, sample=2048)


def test_batched_verify_m128(device):
    _run(inputs.batched_verify_m128(), device, sample=512)
