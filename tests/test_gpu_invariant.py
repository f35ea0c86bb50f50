"""Batch-invariant mode (NVFP4_PATH_INVARIANT) through the C ABI.

The property (the "SparkInfer" README's speculative decoding sections promise that a request which
speculates alone produces exactly the tokens it would produce with speculation disabled): row m of
Y is the same bits whatever M is and whatever the other rows of X hold. Checked bit for bit between calls of the HIP path on the same seeded
inputs (any number of rows, rows at any offset, 128-row slab boundaries, other rows replaced), and
every call against the oracle within |Y - Y_ref| <= 2e-3 * sum|x*w| + 1e-6.
"""
import numpy as np
import pytest
import torch

import oracle
import skinny_gemm_nvfp4_amd as nv
from skinny_gemm_nvfp4_amd import inputs
from parity import (FINITE_SCALES, assert_pack_equal, check_close, gpu_gemm, random_case, say,
                    to_device_packed)

pytestmark = pytest.mark.gpu

INV = nv.PATH_INVARIANT


@pytest.mark.parametrize("N,K", [(1000, 272), (520, 1040), (300, 5120), (34813, 256),
                                 (17, 16), (4096, 4096)])
def test_rows_identical_for_any_m(device, N, K):
    """Ragged N and K (K = 272 and 16 are not multiples of the 128-k window), a shape whose
    plan has remainder tiles (34813 columns: 8.5 tiles per compute unit), a narrow one whose
    plan cuts K across workgroups (4096 x 4096), and 200 rows = two slabs."""
    R = 200
    X, Wq, Ws, g = random_case(900 + N + K, R, N, K, FINITE_SCALES)
    packed = to_device_packed(Wq, Ws, g, device)
    say(f"invariant full R={R} N={N} K={K}")
    Y = gpu_gemm(X, packed, device, INV)
    Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g)
    check_close(Y, Yref, A, f"invariant R={R} N={N} K={K}")
    for M in (1, 2, 15, 16, 17, 33, 64, 100, 127, 128, 129):
        say(f"invariant prefix M={M} N={N} K={K}")
        Ym = gpu_gemm(X[:M], packed, device, INV)
        assert np.array_equal(Ym, Y[:M]), f"rows of the M={M} call differ from the R={R} call"
    for m0, m1 in ((37, 38), (150, 151), (120, 136), (199, 200), (60, 190)):
        say(f"invariant rows {m0}:{m1} N={N} K={K}")
        Ym = gpu_gemm(X[m0:m1], packed, device, INV)
        assert np.array_equal(Ym, Y[m0:m1]), f"rows {m0}:{m1} differ from the R={R} call"


def test_rows_do_not_depend_on_other_rows(device):
    """Row 5 alone, row 5 among 16 random rows and among 128 rows with huge and tiny values: the
    same bits."""
    M, N, K = 128, 2000, 3072
    X, Wq, Ws, g = random_case(961, M, N, K, FINITE_SCALES)
    packed = to_device_packed(Wq, Ws, g, device)
    say(f"invariant neighbours N={N} K={K}")
    y_alone = gpu_gemm(X[5:6], packed, device, INV)
    gen = inputs.generator(962)
    X2 = inputs.activations(gen, 16, K)
    X2[5] = X[5]
    y16 = gpu_gemm(X2, packed, device, INV)
    X3 = X.clone()
    X3[:5] = (X3[:5].float() * 3.0e4).to(torch.bfloat16)
    X3[6:] = (X3[6:].float() * 1.0e-20).to(torch.bfloat16)
    y128 = gpu_gemm(X3, packed, device, INV)
    assert np.array_equal(y16[5:6], y_alone)
    assert np.array_equal(y128[5:6], y_alone)
    Yref, A = oracle.gemm(inputs.bf16_bits(X3), Wq.numpy(), Ws.numpy(), g)
    check_close(y128, Yref, A, "invariant with extreme neighbours")


@pytest.mark.parametrize("gemm_name", ["gate_up", "down"])
def test_decode_and_verify_rows_match_at_layer_size(device, gemm_name):
    """The layer's gate_up and down weights (recipe-quantised, seeds as the M=16 workload): the
    16 rows of a verify call, each row decoded alone (M = 1), and the same 16 rows inside a
    128-row batch give the same bits; sampled columns against the oracle."""
    wl = inputs.verify_m16()
    gm = [g for g in wl.gemms if g.name == gemm_name][0]
    M, N, K = gm.shape
    packed_d, (Wq_o, Ws_o, g_o) = assert_pack_equal(gm.W, device, f"invariant {gemm_name}")
    say(f"invariant verify {gemm_name} M={M} N={N} K={K}")
    Y16 = gpu_gemm(gm.X, packed_d, device, INV)
    for m in (0, 7, 15):
        Y1 = gpu_gemm(gm.X[m:m + 1], packed_d, device, INV)
        assert np.array_equal(Y1, Y16[m:m + 1]), f"row {m} decoded alone differs"
    gen = inputs.generator(963)
    Xb = inputs.activations(gen, 128, K)
    Xb[32:48] = gm.X
    Y128 = gpu_gemm(Xb, packed_d, device, INV)
    assert np.array_equal(Y128[32:48], Y16), "verify rows inside a 128-row batch differ"
    gen = inputs.generator(964)
    cols = np.unique(np.r_[torch.randperm(N, generator=gen)[:512].numpy(),
                           np.arange(16), np.arange(N - 16, N)]).astype(np.int32)
    Yref, A = oracle.gemm(inputs.bf16_bits(gm.X), Wq_o, Ws_o, g_o, cols=cols)
    check_close(Y16[:, cols], Yref, A, f"invariant {gemm_name}")


@pytest.mark.parametrize("N,K", [(34816, 1024), (2048, 4096)])
def test_invariant_under_graph_capture(device, N, K):
    """After one eager call (which sizes the workspace of a split plan for 128 rows), calls at
    other M capture into a HIP graph; replays give the eager bits. 2048 x 4096 is a narrow
    shape whose plan cuts K across workgroups."""
    M = 48
    X, Wq, Ws, g = random_case(965, M, N, K, FINITE_SCALES)
    packed = to_device_packed(Wq, Ws, g, device)
    Xd = X.to(device)
    nv.gemm(Xd[:1], *packed, path=INV)   # eager, one row
    Y = torch.empty(M, N, dtype=torch.float32, device=device)
    nv.gemm(Xd, *packed, out=Y, path=INV)
    torch.cuda.synchronize()
    eager = Y.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nv.gemm(Xd, *packed, out=Y, path=INV)
    for r in range(3):
        Y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, eager), f"replay {r} differs from the eager call"
