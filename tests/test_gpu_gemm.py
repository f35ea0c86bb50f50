"""GPU GEMM (nvfp4_gemm / nvfp4_gemm_path through the C ABI) against the oracle.

Bars:
  * floating point: |Y - Y_ref| <= 2e-3 * sum_k |x*w| + 1e-6 for every output;
  * exact cases (integer sums, one-hot rows): bit equality.
"""
import numpy as np
import pytest
import torch

import oracle
import skinny_gemm_nvfp4_amd as nv
from skinny_gemm_nvfp4_amd import inputs
from parity import (FINITE_SCALES, check_close, gpu_gemm, random_case, say, to_device_packed)

pytestmark = pytest.mark.gpu

PATHS = [(nv.PATH_DOT, 4), (nv.PATH_DOT, 8), (nv.PATH_DOT, 12), (nv.PATH_DOT, 16),
         (nv.PATH_MFMA, 4), (nv.PATH_MFMA, 8),
         (nv.PATH_BATCH, 0), (nv.PATH_BATCH, 16), (nv.PATH_BATCH, 32), (nv.PATH_BATCH, 64),
         (nv.PATH_BATCH, 128), (nv.PATH_AUTO, 0)]
VALU_PATHS = (nv.PATH_DOT,)   # the dot-product kernel: M <= 8
SMALL_M = [1, 2, 3, 4, 5, 8, 15, 16, 17, 33, 130]
SMALL_N = [1, 15, 16, 17, 65]
SMALL_K = [16, 48, 256, 272, 528, 1024]


def _paths_for(M):
    return [(p, s) for p, s in PATHS if not (p in VALU_PATHS and M > 8)]


@pytest.mark.parametrize("path,split", PATHS)
def test_small_shapes(device, path, split):
    """Brute force over tiny shapes, every path and split forced, ragged N, K and M."""
    seed = 0
    for K in SMALL_K:
        for M in SMALL_M:
            if path in VALU_PATHS and M > 8:
                continue
            for N in SMALL_N:
                seed += 1
                X, Wq, Ws, g = random_case(seed, M, N, K, FINITE_SCALES)
                Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g)
                say(f"small path={path} split={split} M={M} N={N} K={K}")
                Y = gpu_gemm(X, to_device_packed(Wq, Ws, g, device), device, path, split)
                check_close(Y, Yref, A, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("path,split", PATHS)
def test_nan_scales_stay_in_their_columns(device, path, split):
    """Odd column groups carry NaN (E4M3 0x7F) block scales in their first 32 k; K is not a
    multiple of the kernels' windows, so a load that covers the end of one group's K (in the
    packed layout) also fetches the next group's first scale bytes. Those must not reach the
    sums: Y is NaN exactly where the oracle's is (every row of the odd groups' columns) and
    within the bound elsewhere."""
    seed = 5000
    for K in (272, 400, 528, 1040):
        for M in (1, 4, 16, 40, 128):
            if path in VALU_PATHS and M > 8:
                continue
            N = 40
            seed += 1
            X, Wq, Ws, g = random_case(seed, M, N, K, FINITE_SCALES)
            Ws = Ws.clone()
            for grp in range(1, N // 4, 2):
                Ws[4 * grp:4 * grp + 4, 0:2] = 0x7F
            Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g)
            assert np.isnan(Yref[:, 4:8]).all() and np.isfinite(Yref[:, 0:4]).all()
            say(f"nan scales path={path} split={split} M={M} N={N} K={K}")
            Y = gpu_gemm(X, to_device_packed(Wq, Ws, g, device), device, path, split)
            check_close(Y, Yref, A, f"NaN scales M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(1, 64, 256), (4, 33, 528), (16, 48, 1024),
                                   (128, 40, 512), (7, 16, 17408), (1, 17, 5120)])
def test_exact_integer_sums(device, M, N, K):
    """Scales in {0.5, 1, 2}, g = 1, X integers in [-8, 8]: every partial sum is a multiple of
    0.25 below 2^22, exact in fp32 in any order, so Y must equal the oracle bit for bit."""
    gen = inputs.generator(1000 + M + N + K)
    Wq, Ws = inputs.random_packed(gen, N, K, scale_bytes=[0x30, 0x38, 0x40])
    X = inputs.integer_activations(gen, M, K)
    Yref, _ = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), 1.0)
    for path, split in _paths_for(M):
        say(f"exact path={path} split={split} M={M} N={N} K={K}")
        Y = gpu_gemm(X, to_device_packed(Wq, Ws, 1.0, device), device, path, split)
        assert np.array_equal(Y, Yref), f"path {path} split {split}: not bit-exact"


@pytest.mark.parametrize("K", [32, 272, 5120])
def test_one_hot_rows_give_dequantised_weights(device, K):
    """x[m, k_m] = 1 and 0 elsewhere: Y[m, n] must be fp32(code * s * g) exactly, for every code
    and every finite scale byte."""
    N = 96
    gen = inputs.generator(77 + K)
    Wq, Ws = inputs.random_packed(gen, N, K, scale_bytes=FINITE_SCALES)
    g = np.float32(0.0137)
    Wd = oracle.dequantize(Wq.numpy(), Ws.numpy(), g)    # exact double [K][N]
    ks = torch.randperm(K, generator=gen)[:16]
    M = len(ks)
    X = torch.zeros(M, K, dtype=torch.bfloat16)
    X[torch.arange(M), ks] = 1.0
    expect = Wd[ks.numpy(), :].astype(np.float32).astype(np.float64)
    for path, split in _paths_for(M):
        if path in VALU_PATHS and M > 8:
            Xs, ex = X[:8], expect[:8]
        else:
            Xs, ex = X, expect
        say(f"one-hot path={path} split={split} K={K}")
        Y = gpu_gemm(Xs, to_device_packed(Wq, Ws, g, device), device, path, split)
        diff = np.argwhere(Y != ex)
        assert diff.size == 0, f"path {path}: {len(diff)} mismatches, first {diff[:3].tolist()}"


@pytest.mark.parametrize("K", [64, 256])
def test_nan_scale_propagates(device, K):
    N, M = 16, 2
    gen = inputs.generator(5)
    Wq, Ws = inputs.random_packed(gen, N, K, scale_bytes=[0x38])
    Ws[3, 1] = 0x7F
    Ws[9, 0] = 0xFF
    X = inputs.activations(gen, M, K)
    Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), 1.0)
    for path, split in _paths_for(M):
        Y = gpu_gemm(X, to_device_packed(Wq, Ws, 1.0, device), device, path, split)
        check_close(Y, Yref, A, "nan")
        assert np.isnan(Y[:, 3]).all() and np.isnan(Y[:, 9]).all()


def test_negative_scale_bytes(device):
    """The GEMM decodes every scale byte as E4M3, including ones with the sign bit set."""
    K, N, M = 256, 40, 3
    gen = inputs.generator(6)
    Wq, Ws = inputs.random_packed(gen, N, K, scale_bytes=list(range(0x80, 0xFF)))
    X = inputs.activations(gen, M, K)
    Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), 0.5)
    for path, split in _paths_for(M):
        Y = gpu_gemm(X, to_device_packed(Wq, Ws, 0.5, device), device, path, split)
        check_close(Y, Yref, A, "negative scales")


def test_deterministic(device):
    X, Wq, Ws, g = random_case(9, 16, 2048, 5120, FINITE_SCALES)
    packed = to_device_packed(Wq, Ws, g, device)
    for path, split in _paths_for(16):
        a = gpu_gemm(X, packed, device, path, split)
        b = gpu_gemm(X, packed, device, path, split)
        assert np.array_equal(a, b), f"path {path} split {split} not reproducible"


@pytest.mark.parametrize("path,split", [(nv.PATH_MFMA, 4), (nv.PATH_MFMA, 8),
                                        (nv.PATH_BATCH, 128), (nv.PATH_BATCH, 32),
                                        (nv.PATH_DOT, 16)])
def test_many_columns_per_workgroup(device, path, split):
    """Enough columns that a persistent workgroup owns more column tiles than one pass takes
    (several chunks per workgroup), with a ragged last tile and a ragged row block."""
    M = {nv.PATH_DOT: 8, nv.PATH_BATCH: 131}.get(path, 19)
    N, K = 256 * 16 * 14 + 5, 256
    X, Wq, Ws, g = random_case(41, M, N, K, FINITE_SCALES)
    Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g)
    say(f"many-columns path={path} split={split} M={M} N={N} K={K}")
    Y = gpu_gemm(X, to_device_packed(Wq, Ws, g, device), device, path, split)
    check_close(Y, Yref, A, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("path,split,Ms", [(nv.PATH_MFMA, 4, (5, 16, 19)),
                                           (nv.PATH_MFMA, 8, (5, 16, 19)),
                                           (nv.PATH_BATCH, 128, (19, 100, 128)),
                                           (nv.PATH_BATCH, 0, (100,))])
def test_reduction_store_widths_agree(device, path, split, Ms):
    """The 16-row and slab kernels store four adjacent outputs per thread when Y is 16-byte
    aligned and N % 4 == 0, one per thread otherwise (Y only 4-byte aligned): the same bits
    either way, and within the bound of the oracle. Several chunks (passes) of tiles per
    workgroup, a part-filled last tile (57492 / 4 groups do not split evenly over the
    workgroups), ragged row blocks, and 128-row groups whose rows go through in two halves."""
    N, K = 256 * 16 * 14 + 4 * 37, 256
    for M in Ms:
        X, Wq, Ws, g = random_case(70 + M, M, N, K, FINITE_SCALES)
        p = to_device_packed(Wq, Ws, g, device)
        Xd = X.to(device)
        say(f"store widths path={path} split={split} M={M} N={N} K={K}")
        Ya = nv.gemm(Xd, *p, path=path, split=split)
        buf = torch.full((M * N + 1,), float("nan"), dtype=torch.float32, device=device)
        Yb = buf[1:].view(M, N)
        nv.gemm(Xd, *p, path=path, split=split, out=Yb)
        torch.cuda.synchronize()
        a, b = Ya.cpu().numpy(), Yb.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"M={M}: store widths differ"
        Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g)
        check_close(a.astype(np.float64), Yref, A, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,split", [(16, 34813, 0), (100, 34813, 0), (128, 34813, 128),
                                       (33, 18431, 0), (128, 22521, 128), (16, 22521, 16),
                                       (128, 1795, 32), (70, 4099, 64)])
def test_batch_remainder_tiles(device, M, N, split):
    """Column shares that leave an odd tile per workgroup (9, 7, 5, ... tiles of 16), whose four
    MFMA k-steps are split across the four consumer wavefronts and meet in LDS; ragged N, ragged
    last window (K = 272), ragged row blocks and row groups."""
    K = 272
    X, Wq, Ws, g = random_case(500 + M + N, M, N, K, FINITE_SCALES)
    Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g)
    say(f"remainder path=batch split={split} M={M} N={N} K={K}")
    Y = gpu_gemm(X, to_device_packed(Wq, Ws, g, device), device, nv.PATH_BATCH, split)
    check_close(Y, Yref, A, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K,rg", [(128, 1000, 2048, 16), (128, 1000, 2048, 32),
                                      (33, 520, 1040, 64), (131, 300, 512, 32),
                                      (128, 5120, 17408, 32), (16, 257, 272, 16)])
def test_batch_row_groups(device, M, N, K, rg):
    """Rows cut into row groups of rg rows, each with its own workgroups (tile sets on one XCD);
    ragged K, ragged rows, two 128-row slabs; reproducible bit for bit."""
    X, Wq, Ws, g = random_case(700 + M + N + rg, M, N, K, FINITE_SCALES)
    Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g)
    say(f"row groups rg={rg} M={M} N={N} K={K}")
    packed = to_device_packed(Wq, Ws, g, device)
    Y = gpu_gemm(X, packed, device, nv.PATH_BATCH, rg)
    check_close(Y, Yref, A, f"rg={rg} M={M} N={N} K={K}")
    Y2 = gpu_gemm(X, packed, device, nv.PATH_BATCH, rg)
    assert np.array_equal(Y, Y2), "row-group plan not reproducible"


def test_auto_narrow_m128(device):
    """nvfp4_gemm on a narrow shape at M = 128 (few column tiles per compute unit), where the
    planner cuts the rows into row groups."""
    M, N, K = 128, 2048, 4096
    X, Wq, Ws, g = random_case(811, M, N, K, FINITE_SCALES)
    Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g)
    say(f"auto narrow M={M} N={N} K={K}")
    Y = gpu_gemm(X, to_device_packed(Wq, Ws, g, device), device, nv.PATH_AUTO, 0)
    check_close(Y, Yref, A, f"M={M} N={N} K={K}")
