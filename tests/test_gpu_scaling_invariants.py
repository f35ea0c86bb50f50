"""Exact scaling invariants of the HIP GEMM, per kernel family, through the C ABI.

The GEMM is linear in X and in the tensor scale g. Multiplying every input of a floating-point sum
by 2 multiplies every rounded partial sum by 2 (no overflow or underflow at these magnitudes), in
IEEE arithmetic and in the matrix cores' accumulation alike, so for the fixed summation order
every kernel has:
  * Y(2X) = 2Y,
  * Y(2g) = 2Y (g multiplies the finished sum once),
bit for bit. Negation commutes with round-to-nearest, so the VALU kernels (dot product, grouped)
also give Y(-X) = -Y bit for bit. The bf16 matrix-core instruction does not: adding its products
to a non-zero accumulator it truncates the aligned addends instead of rounding them to nearest
(measured on gfx950 for v_mfma_f32_16x16x32_bf16: about 3% of outputs differ in the last bits
between D(A, C) and -D(-A, -C), while D(A, 0) is sign-symmetric), so on the matrix-core kernels
Y(-X) is held to the oracle's tolerance around -Y_ref instead. A kernel that mixed rows, dropped a
term, or let a row's arithmetic depend on another row breaks one of these checks; the oracle is
checked once per case as well, so a degenerate output cannot satisfy them.
+0 and -0 compare equal.
"""
import numpy as np
import pytest
import torch

import oracle
import skinny_gemm_nvfp4_amd as nv
from skinny_gemm_nvfp4_amd import inputs
from parity import FINITE_SCALES, check_close, random_case, say, to_device_packed

pytestmark = pytest.mark.gpu

# One shape per kernel family (and the automatic choice at the three workload M).
FAMILIES = [(nv.PATH_DOT, 12, 1, 1000, 5120), (nv.PATH_DOT, 16, 4, 520, 1024),
            (nv.PATH_MFMA, 4, 16, 2000, 5120), (nv.PATH_MFMA, 8, 33, 700, 1040),
            (nv.PATH_BATCH, 0, 128, 1500, 2048), (nv.PATH_BATCH, 0, 77, 300, 17408),
            (nv.PATH_INVARIANT, 0, 20, 900, 1024),
            (nv.PATH_AUTO, 0, 1, 7168, 512), (nv.PATH_AUTO, 0, 16, 3000, 1024),
            (nv.PATH_AUTO, 0, 128, 5120, 1024)]


def _gemm(X, p, N, path, split, device):
    Y = nv.gemm(X.to(device), p.Wq, p.Ws, p.g, N, path=path, split=split)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


@pytest.mark.parametrize("path,split,M,N,K", FAMILIES)
def test_sign_and_scale_invariants(device, path, split, M, N, K):
    X, Wq, Ws, g = random_case(8800 + M + N + K + path, M, N, K, FINITE_SCALES)
    label = f"invariants path={path} split={split} M={M} N={N} K={K}"
    say(label)
    p = to_device_packed(Wq, Ws, g, device)
    p2 = to_device_packed(Wq, Ws, np.float32(2.0) * g, device)
    Y = _gemm(X, p, N, path, split, device)
    Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq.numpy(), Ws.numpy(), g)
    check_close(Y.astype(np.float64), Yref, A, label)
    assert np.count_nonzero(Y) > Y.size // 2, f"{label}: degenerate output"
    Yneg = _gemm(-X, p, N, path, split, device)
    if path == nv.PATH_DOT or (path == nv.PATH_AUTO and M <= 4):
        assert np.array_equal(Yneg, -Y), f"{label}: Y(-X) != -Y"
    else:
        check_close(Yneg.astype(np.float64), -Yref, A, f"{label}: Y(-X)")
    Y2x = _gemm(2 * X, p, N, path, split, device)
    assert np.array_equal(Y2x, np.float32(2) * Y), f"{label}: Y(2X) != 2Y"
    Y2g = _gemm(X, p2, N, path, split, device)
    assert np.array_equal(Y2g, np.float32(2) * Y), f"{label}: Y(2g) != 2Y"


@pytest.mark.parametrize("M", [1, 16, 128])
def test_argmax_follows_the_scaling(device, M):
    """The greedy-token call under X -> 2X and g -> 2g: same index, exactly doubled value."""
    N, K = 3001, 1024
    X, Wq, Ws, g = random_case(8900 + M, M, N, K, FINITE_SCALES)
    say(f"argmax invariants M={M}")
    p = to_device_packed(Wq, Ws, g, device)
    p2 = to_device_packed(Wq, Ws, np.float32(2.0) * g, device)
    idx, val = nv.gemm_argmax(X.to(device), p.Wq, p.Ws, p.g, N)
    idx2, val2 = nv.gemm_argmax((2 * X).to(device), p.Wq, p.Ws, p.g, N)
    idx3, val3 = nv.gemm_argmax(X.to(device), p2.Wq, p2.Ws, p2.g, N)
    torch.cuda.synchronize()
    for i, v in ((idx2, val2), (idx3, val3)):
        assert torch.equal(i.cpu(), idx.cpu())
        assert np.array_equal(v.cpu().numpy(), np.float32(2) * val.cpu().numpy())


def test_grouped_invariants(device):
    """The grouped (mixture-of-experts) kernel under X -> -X, X -> 2X and g -> 2g."""
    E, N, K, T = 6, 520, 1024, 40
    gen = inputs.generator(8950)
    packs = [inputs.random_packed(gen, N, K, FINITE_SCALES) for _ in range(E)]
    Wq = torch.stack([q for q, _ in packs])
    Ws = torch.stack([s for _, s in packs])
    counts = [7, 0, 13, 1, 19, 0]
    offsets = torch.tensor(np.r_[0, np.cumsum(counts)], dtype=torch.int32)
    X = inputs.activations(gen, T, K)
    g = torch.tensor([0.01, 0.02, 0.005, 0.3, 0.07, 1.0], dtype=torch.float32)
    from parity import to_library_layout
    lib = [to_library_layout(Wq[e].numpy(), Ws[e].numpy(), K) for e in range(E)]
    Wq_d = torch.from_numpy(np.stack([a for a, _ in lib])).to(device)
    Ws_d = torch.from_numpy(np.stack([b for _, b in lib])).to(device)
    off_d = offsets.to(device)

    def run(Xh, gh):
        Y = nv.gemm_grouped(Xh.to(device), off_d, Wq_d, Ws_d, gh.to(device), N)
        torch.cuda.synchronize()
        return Y.cpu().numpy()

    say("grouped invariants")
    Y = run(X, g)
    Yref, A = oracle.grouped_gemm(inputs.bf16_bits(X), offsets.numpy(), Wq.numpy(), Ws.numpy(),
                                  g.numpy())
    check_close(Y.astype(np.float64), Yref, A, "grouped")
    assert np.array_equal(run(-X, g), -Y)
    assert np.array_equal(run(2 * X, g), np.float32(2) * Y)
    assert np.array_equal(run(X, 2 * g), np.float32(2) * Y)
