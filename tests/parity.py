"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle, compare.

The HIP path is reached only through the C ABI (skinny_gemm_nvfp4_amd.binding). The oracle never
sees a value the HIP path produced: the GEMM oracle consumes the oracle's own packed bytes, and
the packed bytes of the two sides are compared for bit equality first.
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


def gpu_pack(W: torch.Tensor, device) -> tuple:
    Wq, Ws, g = nv.pack(W.to(device))
    torch.cuda.synchronize()
    return Wq, Ws, g


def assert_pack_equal(W: torch.Tensor, device, label: str = ""):
    """GPU pack of fp32 W must equal the oracle quantiser byte for byte. Returns both sides."""
    say(f"pack {label} K={W.shape[0]} N={W.shape[1]}")
    Wq_d, Ws_d, g_d = gpu_pack(W, device)
    Wq_o, Ws_o, g_o = oracle.quantize(W.numpy())
    g_gpu = np.float32(g_d.cpu().numpy()[0])
    assert g_gpu.tobytes() == np.float32(g_o).tobytes(), f"g differs: {g_gpu} vs {g_o}"
    ws_gpu = Ws_d.cpu().numpy()
    bad_s = np.argwhere(ws_gpu != Ws_o)
    assert bad_s.size == 0, f"{len(bad_s)} scale bytes differ, first at {bad_s[:4].tolist()}"
    wq_gpu = Wq_d.cpu().numpy()
    bad_q = np.argwhere(wq_gpu != Wq_o)
    assert bad_q.size == 0, f"{len(bad_q)} code bytes differ, first at {bad_q[:4].tolist()}"
    return (Wq_d, Ws_d, g_d), (Wq_o, Ws_o, g_o)


def gpu_gemm(X: torch.Tensor, packed_dev, device, path=nv.PATH_AUTO, split=0) -> np.ndarray:
    Wq, Ws, g = packed_dev
    Y = nv.gemm(X.to(device), Wq, Ws, g, path=path, split=split)
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


def to_device_packed(Wq: torch.Tensor, Ws: torch.Tensor, g, device):
    return (Wq.to(device), Ws.to(device),
            torch.tensor([float(g)], dtype=torch.float32, device=device))


# Finite, non-negative E4M3 scale bytes: every value a quantiser can emit.
FINITE_SCALES = list(range(0x00, 0x7F))
