"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle, compare.

The HIP path is reached only through the C ABI (skinny_gemm_nvfp4_amd.binding). The oracle never
sees a value the HIP path produced: the GEMM oracle consumes the oracle's own packed bytes, and
the packed bytes of the two sides are compared for bit equality first.

The oracle keeps the plain layout Wq[N][K/2], Ws[N][K/16]; the library's layout (include/nvfp4.h)
groups 4 columns and 32-k chunks. to_library_layout / from_library_layout move bytes between the
two, written here from the header's definition (byte (g, c, j, i) of Wq holds plain byte
(4g + j, 16c + i); byte (g, c, j, b) of Ws holds plain byte (4g + j, 2c + b); padding is zero).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import skinny_gemm_nvfp4_amd as nv
from skinny_gemm_nvfp4_amd import inputs


def say(msg: str) -> None:
    """Progress line naming the case, flushed before the GPU step runs."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_library_layout(Wq_plain: np.ndarray, Ws_plain: np.ndarray, K: int):
    """Plain [N][K/2], [N][K/16] bytes -> library layout [NG][CH][4][16], [NG][CH][4][2]."""
    N = Wq_plain.shape[0]
    NG, CH = -(-N // 4), -(-K // 32)
    P = np.zeros((4 * NG, 16 * CH), dtype=np.uint8)
    P[:N, :K // 2] = Wq_plain
    S = np.zeros((4 * NG, 2 * CH), dtype=np.uint8)
    S[:N, :K // 16] = Ws_plain
    Wq = np.ascontiguousarray(P.reshape(NG, 4, CH, 16).transpose(0, 2, 1, 3))
    Ws = np.ascontiguousarray(S.reshape(NG, 4, CH, 2).transpose(0, 2, 1, 3))
    return Wq, Ws


def from_library_layout(Wq: np.ndarray, Ws: np.ndarray, N: int, K: int):
    """Library layout -> plain bytes, and whether every padding byte is zero."""
    NG, CH = Wq.shape[0], Wq.shape[1]
    P = Wq.transpose(0, 2, 1, 3).reshape(4 * NG, 16 * CH).copy()
    S = Ws.transpose(0, 2, 1, 3).reshape(4 * NG, 2 * CH).copy()
    Wq_plain = P[:N, :K // 2].copy()
    Ws_plain = S[:N, :K // 16].copy()
    P[:N, :K // 2] = 0
    S[:N, :K // 16] = 0
    return Wq_plain, Ws_plain, not P.any() and not S.any()


def gpu_pack(W: torch.Tensor, device) -> nv.Packed:
    p = nv.pack(W.to(device))
    torch.cuda.synchronize()
    return p


def assert_pack_equal(W: torch.Tensor, device, label: str = ""):
    """GPU pack of fp32 W must equal the oracle quantiser byte for byte. Returns both sides."""
    K, N = W.shape
    say(f"pack {label} K={K} N={N}")
    packed = gpu_pack(W, device)
    Wq_o, Ws_o, g_o = oracle.quantize(W.numpy())
    g_gpu = np.float32(packed.g.cpu().numpy()[0])
    assert g_gpu.tobytes() == np.float32(g_o).tobytes(), f"g differs: {g_gpu} vs {g_o}"
    wq_gpu, ws_gpu, pad_zero = from_library_layout(packed.Wq.cpu().numpy(),
                                                   packed.Ws.cpu().numpy(), N, K)
    assert pad_zero, "padding bytes of the packed layout are not zero"
    bad_s = np.argwhere(ws_gpu != Ws_o)
    assert bad_s.size == 0, f"{len(bad_s)} scale bytes differ, first at {bad_s[:4].tolist()}"
    bad_q = np.argwhere(wq_gpu != Wq_o)
    assert bad_q.size == 0, f"{len(bad_q)} code bytes differ, first at {bad_q[:4].tolist()}"
    return packed, (Wq_o, Ws_o, g_o)


def gpu_gemm(X: torch.Tensor, packed_dev, device, path=nv.PATH_AUTO, split=0) -> np.ndarray:
    Wq, Ws, g, N = packed_dev
    Y = nv.gemm(X.to(device), Wq, Ws, g, N, path=path, split=split)
    torch.cuda.synchronize()
    return Y.cpu().numpy().astype(np.float64)


def check_close(Y: np.ndarray, Yref: np.ndarray, A: np.ndarray, label: str = "") -> float:
    """|Y - Yref| <= 2e-3 * sum|x*w| + 1e-6 per output. Returns the worst ratio error/bound."""
    assert Y.shape == Yref.shape, (Y.shape, Yref.shape)
    nan_ref = np.isnan(Yref)
    assert np.array_equal(np.isnan(Y), nan_ref), f"{label}: NaN pattern differs"
    ok = ~nan_ref
    err = np.abs(Y[ok] - Yref[ok])
    bound = oracle.tolerance(A[ok])
    worst = float(np.max(err / bound)) if err.size else 0.0
    bad = np.argwhere(~(err <= bound))
    assert bad.size == 0, f"{label}: {bad.size} outputs out of tolerance, worst ratio {worst:.3g}"
    return worst


def random_case(seed: int, M: int, N: int, K: int, scale_bytes=None, g: float = 0.01):
    """Random packed weights (bytes straight from the generator) and bf16 activations."""
    gen = inputs.generator(seed)
    Wq, Ws = inputs.random_packed(gen, N, K, scale_bytes)
    X = inputs.activations(gen, M, K)
    return X, Wq, Ws, np.float32(g)


def to_device_packed(Wq: torch.Tensor, Ws: torch.Tensor, g, device) -> nv.Packed:
    """Plain-layout bytes (as the oracle takes them) -> library layout on the device."""
    N, K = Wq.shape[0], 2 * Wq.shape[1]
    wq, ws = to_library_layout(np.asarray(Wq), np.asarray(Ws), K)
    return nv.Packed(torch.from_numpy(wq).to(device), torch.from_numpy(ws).to(device),
                     torch.tensor([float(g)], dtype=torch.float32, device=device), N)


# Finite, non-negative E4M3 scale bytes: every value a quantiser can emit.
FINITE_SCALES = list(range(0x00, 0x7F))
