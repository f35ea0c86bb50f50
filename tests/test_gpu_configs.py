"""The workloads at full size: GPU pack bit-exact against the oracle, then GPU GEMM against the
oracle GEMM on every output (every row and every column: the double-precision oracle does the
M = 128 layer, about 42 G multiply-adds, in seconds on the host cores). The GEMM runs through
nvfp4_gemm, the entry point the benchmark times.
"""
import pytest

import oracle
from skinny_gemm_nvfp4_amd import inputs
from parity import assert_pack_equal, check_close, gpu_gemm, say

pytestmark = pytest.mark.gpu


def _run(workload, device):
    for gm in workload.gemms:
        M, N, K = gm.shape
        (packed_d, packed_o) = assert_pack_equal(gm.W, device, f"{workload.name}.{gm.name}")
        say(f"gemm {workload.name}.{gm.name} M={M} N={N} K={K}")
        Y = gpu_gemm(gm.X, packed_d, device)
        Wq_o, Ws_o, g_o = packed_o
        Yref, A = oracle.gemm(inputs.bf16_bits(gm.X), Wq_o, Ws_o, g_o)
        assert Y.shape == (M, N)
        worst = check_close(Y, Yref, A, f"{workload.name}.{gm.name}")
        say(f"  worst error / bound = {worst:.3g} over {M * N} outputs")


def test_single_gemv(device):
    _run(inputs.single_gemv(), device)


def test_dense_layer_m1(device):
    _run(inputs.dense_layer_m1(), device)


def test_verify_m16(device):
    _run(inputs.verify_m16(), device)


def test_batched_verify_m128(device):
    _run(inputs.batched_verify_m128(), device)
