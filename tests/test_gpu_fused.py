"""The GEMM with its decode-layer neighbours (nvfp4_gemm_fused through the C ABI) against the
oracle ("SparkInfer" README, section "Layout & scoring": RMSNorm and fused FFN kernels).

Bars (derived in the design doc):
  * RMSNorm: the oracle rounds the exact normalised activation to bf16 once; the kernel computes
    it in fp32 within a relative (K/64 + 40) 2^-24, so where the exact value lies within twice
    that of a bf16 rounding boundary either neighbour is correct (flagged by the oracle). The
    GEMM bar becomes |Y - Y_ref| <= 2e-3 sum|xhat w| + 1e-6 + sum_flagged ulp |w|.
  * SiLU(gate) * up: gate and up carry their GEMM tolerances t_g, t_u; SiLU has slope at most
    1.1, so |H - h_ref| <= pre + 2^-8 (|h_ref| + pre) + 2e-5 |h_ref| + 1e-30 with
    pre = 1.1 t_g (|up| + t_u) + (|silu(gate)| + 1.1 t_g) t_u (the 2^-8 covers the bf16 rounding
    of H, 2e-5 the fp32 exponential).
"""
import numpy as np
import pytest
import torch

import oracle
import skinny_gemm_nvfp4_amd as nv
from skinny_gemm_nvfp4_amd import inputs
from parity import FINITE_SCALES, say, to_device_packed

pytestmark = pytest.mark.gpu

EPS = inputs.RMSNORM_EPS


def _window(K):
    return 2.0 * (K / 64 + 40) * 2.0 ** -24


def _bits_of(t):
    return inputs.bf16_bits(t)


def _ref_gemm(X_bits, Wq, Ws, g, gamma_bits=None):
    """Oracle Y and its bound for the (optionally RMSNorm-ed) activations."""
    if gamma_bits is None:
        Y, A = oracle.gemm(X_bits, Wq, Ws, g)
        return Y, oracle.tolerance(A)
    K = X_bits.shape[1]
    xhat, flag, ulp = oracle.rmsnorm_bf16(X_bits, gamma_bits, EPS, _window(K))
    Y, A = oracle.gemm(xhat, Wq, Ws, g)
    allow_bits, _, _, _ = oracle.bf16_round(np.where(flag, ulp, 0.0))
    _, A_allow = oracle.gemm(allow_bits, Wq, Ws, g)
    return Y, oracle.tolerance(A) + A_allow


def _check_y(Y, Yref, tol, label):
    err = np.abs(Y.astype(np.float64) - Yref)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, f"{label}: {len(bad)} outputs outside the bound, first {bad[:3]}"


def _check_h(H_bits, Yref, tol, label):
    h = (H_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    M, N = Yref.shape
    cols = np.arange(N).reshape(N // 8, 2, 4)
    gi, ui = cols[:, 0, :].reshape(-1), cols[:, 1, :].reshape(-1)
    gate, up, tg, tu = Yref[:, gi], Yref[:, ui], tol[:, gi], tol[:, ui]
    href = oracle.silu_mul(gate, up)
    sg = np.abs(oracle.silu_mul(gate, np.ones_like(gate)))
    pre = 1.1 * tg * (np.abs(up) + tu) + (sg + 1.1 * tg) * tu
    bound = pre + 2.0 ** -8 * (np.abs(href) + pre) + 2e-5 * np.abs(href) + 1e-30
    bad = np.argwhere(~(np.abs(h - href) <= bound))
    assert bad.size == 0, f"{label}: {len(bad)} outputs of H outside the bound, first {bad[:3]}"


CASES = [(1, 1000, 1024), (3, 264, 5120), (4, 72, 272), (5, 200, 1024), (16, 1000, 512),
         (20, 136, 5120), (40, 64, 1024), (130, 520, 1040)]


@pytest.mark.parametrize("M,N,K", CASES)
@pytest.mark.parametrize("fuse", [1, 2, 3])
def test_fused_against_oracle(device, M, N, K, fuse):
    gen = inputs.generator(3000 + 7 * M + N + K + fuse)
    Wq, Ws = inputs.random_packed(gen, N, K, FINITE_SCALES)
    g = np.float32(0.011)
    X = inputs.activations(gen, M, K, outliers=4)
    gamma = inputs.norm_weight(gen, K)
    norm = bool(fuse & nv.FUSE_RMSNORM)
    label = f"fused={fuse} M={M} N={N} K={K}"
    say(label)
    Yref, tol = _ref_gemm(_bits_of(X), Wq.numpy(), Ws.numpy(), g,
                          _bits_of(gamma) if norm else None)
    p = to_device_packed(Wq, Ws, g, device)
    out = nv.gemm_fused(X.to(device), p.Wq, p.Ws, p.g, N,
                        gamma=gamma.to(device) if norm else None, eps=EPS,
                        silu_mul=bool(fuse & nv.FUSE_SILU_MUL))
    torch.cuda.synchronize()
    if fuse & nv.FUSE_SILU_MUL:
        _check_h(out.cpu().view(torch.int16).numpy().view(np.uint16), Yref, tol, label)
    else:
        _check_y(out.cpu().numpy(), Yref, tol, label)


@pytest.mark.parametrize("M", [5, 16, 19, 100])
def test_silu_store_widths_agree(device, M):
    """SiLU(gate) * up stored four outputs per thread (H 8-byte aligned, N % 8 == 0) or one (H
    only 2-byte aligned) gives the same bits, within the bound of the oracle; wide enough that a
    workgroup takes several chunks of tiles, with whole gate/up pairs split unevenly (M = 100:
    the slab kernel's 128-row group, its rows in two halves, the second ragged)."""
    N, K = 256 * 16 * 14 + 8 * 13, 256
    gen = inputs.generator(4100 + M)
    Wq, Ws = inputs.random_packed(gen, N, K, FINITE_SCALES)
    g = np.float32(0.011)
    X = inputs.activations(gen, M, K, outliers=4)
    label = f"silu store widths M={M} N={N} K={K}"
    say(label)
    p = to_device_packed(Wq, Ws, g, device)
    Xd = X.to(device)
    Ha = nv.gemm_fused(Xd, p.Wq, p.Ws, p.g, N, silu_mul=True)
    buf = torch.zeros(M * (N // 2) + 1, dtype=torch.bfloat16, device=device)
    Hb = buf[1:].view(M, N // 2)
    nv.gemm_fused(Xd, p.Wq, p.Ws, p.g, N, silu_mul=True, out=Hb)
    torch.cuda.synchronize()
    a = Ha.cpu().view(torch.int16).numpy().view(np.uint16)
    b = Hb.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(a, b), f"{label}: store widths differ"
    Yref, tol = _ref_gemm(_bits_of(X), Wq.numpy(), Ws.numpy(), g)
    _check_h(a, Yref, tol, label)


def test_rmsnorm_constant_rows(device):
    """Rows of one constant c with eps = 0 normalise to gamma * sign(c) exactly, so the fused
    GEMM equals the plain GEMM of gamma (bit for bit in exact-sum cases)."""
    M, N, K = 4, 96, 1024
    gen = inputs.generator(4040)
    Wq, Ws = inputs.random_packed(gen, N, K, scale_bytes=[0x30, 0x38, 0x40])
    gamma = inputs.integer_activations(gen, 1, K, -4, 4)[0]
    X = torch.tensor([[3.0], [-0.5], [1.0], [-96.0]]).repeat(1, K).to(torch.bfloat16)
    sign = torch.tensor([1.0, -1.0, 1.0, -1.0])[:, None]
    Xg = (sign * gamma.float()[None, :]).to(torch.bfloat16)
    Yref, _ = oracle.gemm(_bits_of(Xg), Wq.numpy(), Ws.numpy(), 1.0)
    p = to_device_packed(Wq, Ws, 1.0, device)
    for M_ in (4, 16):   # the dot-product kernel, then the 16-row kernel (rows padded by zeros)
        Xp = torch.cat([X, torch.zeros(M_ - 4, K, dtype=torch.bfloat16)]) if M_ > 4 else X
        say(f"rmsnorm constant rows M={M_}")
        Y = nv.gemm_fused(Xp.to(device), p.Wq, p.Ws, p.g, N, gamma=gamma.to(device), eps=0.0)
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy()[:4].astype(np.float64), Yref)


@pytest.mark.parametrize("M", [1, 16, 128])
def test_layer_shapes(device, M):
    """The layer's q/k/v projection after the input RMSNorm, and its gate/up projection (weight
    interleaved for the fused SiLU * up) after the post-attention RMSNorm, from the workload
    recipe (weights packed by the GPU, and by the oracle from the same fp32 tensor); the oracle
    checks every row and column."""
    gen = inputs.generator(5050 + M)
    K = inputs.HIDDEN
    X = inputs.activations(gen, M, K, outliers=4)
    gamma = inputs.norm_weight(gen, K)
    for name, fuse in (("qkv", 1), ("gate_up", 3)):
        N = inputs.LAYER_SHAPES[name][1]
        W = inputs.weights(gen, K, N)
        if fuse & nv.FUSE_SILU_MUL:
            W = nv.interleave_gate_up(W)
        label = f"layer {name} M={M} fuse={fuse}"
        say(label)
        p = nv.pack(W.to(device))
        Wq_o, Ws_o, g_o = oracle.quantize(W.numpy())
        out = nv.gemm_fused(X.to(device), p.Wq, p.Ws, p.g, N, gamma=gamma.to(device), eps=EPS,
                            silu_mul=bool(fuse & nv.FUSE_SILU_MUL))
        torch.cuda.synchronize()
        Yref, tol = _ref_gemm(_bits_of(X), Wq_o, Ws_o, g_o, _bits_of(gamma))
        if fuse & nv.FUSE_SILU_MUL:
            _check_h(out.cpu().view(torch.int16).numpy().view(np.uint16), Yref, tol, label)
        else:
            _check_y(out.cpu().numpy(), Yref, tol, label)



def test_fused_graph_replays_match_eager(device):
    """Fused calls (M = 1 in one kernel; M = 64 as an RMSNorm kernel writing the caller's
    workspace, then the slab kernel with the SiLU * up epilogue) captured in a HIP graph reproduce
    the eager bits on every replay, with the workspace clobbered between replays."""
    K, N = 1024, 2048
    gen = inputs.generator(6060)
    W = nv.interleave_gate_up(inputs.weights(gen, K, N))
    p = nv.pack(W.to(device))
    gamma = inputs.norm_weight(gen, K).to(device)
    Xs = [inputs.activations(gen, M, K).to(device) for M in (1, 64)]
    Hs = [torch.empty((X.shape[0], N // 2), dtype=torch.bfloat16, device=device) for X in Xs]
    fuse = nv.FUSE_RMSNORM | nv.FUSE_SILU_MUL
    Ws = [nv.fused_workspace(fuse, X.shape[0], N, K, device) for X in Xs]
    assert Ws[0] is None and Ws[1] is not None

    def step():
        for X, H, ws in zip(Xs, Hs, Ws):
            nv.gemm_fused(X, p.Wq, p.Ws, p.g, N, gamma=gamma, eps=EPS, silu_mul=True, out=H,
                          workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = [H.clone() for H in Hs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for H in Hs:
            H.fill_(0)
        Ws[1].fill_(0x5A)
        torch.cuda.synchronize()
        say(f"fused graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for H, E in zip(Hs, eager):
            assert torch.equal(H, E), f"replay {rep} differs"


@pytest.mark.parametrize("M", [1, 5, 17])
def test_smallest_shapes(device, M):
    """N = 8 (one gate/up pair) and K = 16 (one scale block), every fuse mode."""
    N, K = 8, 16
    gen = inputs.generator(7070 + M)
    Wq, Ws = inputs.random_packed(gen, N, K, FINITE_SCALES)
    g = np.float32(0.02)
    X = inputs.activations(gen, M, K)
    gamma = inputs.norm_weight(gen, K)
    p = to_device_packed(Wq, Ws, g, device)
    for fuse in (1, 2, 3):
        norm = bool(fuse & nv.FUSE_RMSNORM)
        label = f"smallest fused={fuse} M={M}"
        say(label)
        Yref, tol = _ref_gemm(_bits_of(X), Wq.numpy(), Ws.numpy(), g,
                              _bits_of(gamma) if norm else None)
        out = nv.gemm_fused(X.to(device), p.Wq, p.Ws, p.g, N,
                            gamma=gamma.to(device) if norm else None, eps=EPS,
                            silu_mul=bool(fuse & nv.FUSE_SILU_MUL))
        torch.cuda.synchronize()
        if fuse & nv.FUSE_SILU_MUL:
            _check_h(out.cpu().view(torch.int16).numpy().view(np.uint16), Yref, tol, label)
        else:
            _check_y(out.cpu().numpy(), Yref, tol, label)
