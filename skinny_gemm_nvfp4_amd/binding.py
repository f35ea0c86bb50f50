"""Thin ctypes binding of libnvfp4.so (include/nvfp4.h).

Argument marshalling only: every step of quantisation and of the GEMM runs in the HIP kernels.
PyTorch supplies device memory and the current stream. There is no fallback: if the library is
not built, or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import torch

from . import build as _build

SUCCESS = 0
ERROR_INVALID_VALUE = 1
ERROR_MISALIGNED = 2
ERROR_LAUNCH = 3
ERROR_SCRATCH_LIMIT = 4

PATH_AUTO = 0
PATH_DOT = 1
PATH_MFMA = 2
PATH_BATCH = 3       # split: rows per row group, 16, 32, 64 or 128 (0: chosen)
PATH_INVARIANT = 5   # row m of Y is the same bits for every M

FUSE_RMSNORM = 1     # nvfp4_gemm_fused: RMSNorm of X before the GEMM
FUSE_SILU_MUL = 2    # nvfp4_gemm_fused: SiLU(gate) * up of the interleaved gate/up output

_lib = None


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def library_path() -> str:
    return _build.LIB


def load_library() -> ctypes.CDLL:
    """Load the in-tree libnvfp4.so. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m skinny_gemm_nvfp4_amd.build` "
            "(the NVFP4 GEMM has no CPU fallback)")
    L = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    ci = ctypes.c_int
    L.nvfp4_pack.argtypes = [ci, ci, vp, vp, vp, vp, vp]
    L.nvfp4_pack.restype = ci
    L.nvfp4_gemm.argtypes = [ci, ci, ci, vp, vp, vp, vp, vp, vp]
    L.nvfp4_gemm.restype = ci
    L.nvfp4_gemm_path.argtypes = [ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, vp]
    L.nvfp4_gemm_path.restype = ci
    L.nvfp4_gemm_argmax.argtypes = [ci, ci, ci, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint64, vp]
    L.nvfp4_gemm_argmax.restype = ci
    L.nvfp4_gemm_argmax_path.argtypes = [ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, vp, vp,
                                         ctypes.c_uint64, vp]
    L.nvfp4_gemm_argmax_path.restype = ci
    L.nvfp4_gemm_argmax_noalloc.argtypes = [ci, ci, ci, vp, vp, vp, vp, vp, vp, vp]
    L.nvfp4_gemm_argmax_noalloc.restype = ci
    L.nvfp4_argmax_workspace_bytes.argtypes = [ci]
    L.nvfp4_argmax_workspace_bytes.restype = ctypes.c_uint64
    L.nvfp4_gemm_grouped.argtypes = [ci, ci, ci, ci, vp, vp, vp, vp, vp, vp, ci, vp]
    L.nvfp4_gemm_grouped.restype = ci
    L.nvfp4_gemm_fused.argtypes = [ci, ci, ci, ci, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp,
                                   ctypes.c_uint64, vp]
    L.nvfp4_gemm_fused.restype = ci
    L.nvfp4_fused_workspace_bytes.argtypes = [ci, ci, ci, ci]
    L.nvfp4_fused_workspace_bytes.restype = ctypes.c_uint64
    L.nvfp4_status_string.argtypes = [ci]
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_abi_version.argtypes = []
    L.nvfp4_abi_version.restype = ci
    L.nvfp4_codes_bytes.argtypes = [ci, ci]
    L.nvfp4_codes_bytes.restype = ctypes.c_uint64
    L.nvfp4_scales_bytes.argtypes = [ci, ci]
    L.nvfp4_scales_bytes.restype = ctypes.c_uint64
    _lib = L
    return L


def status_string(status: int) -> str:
    return load_library().nvfp4_status_string(int(status)).decode()


def abi_version() -> int:
    return load_library().nvfp4_abi_version()


# ---- raw entry points: same names and arguments as the C ABI (ints are device addresses) ----

def nvfp4_pack(K: int, N: int, W: int, Wq: int, Wscale: int, gscale: int,
               stream: Optional[int]) -> int:
    return load_library().nvfp4_pack(K, N, W, Wq, Wscale, gscale, stream)


def nvfp4_gemm(M: int, N: int, K: int, X: int, Wq: int, Wscale: int, gscale: int, Y: int,
               stream: Optional[int]) -> int:
    return load_library().nvfp4_gemm(M, N, K, X, Wq, Wscale, gscale, Y, stream)


def nvfp4_gemm_path(path: int, split: int, M: int, N: int, K: int, X: int, Wq: int, Wscale: int,
                    gscale: int, Y: int, stream: Optional[int]) -> int:
    return load_library().nvfp4_gemm_path(path, split, M, N, K, X, Wq, Wscale, gscale, Y, stream)


def nvfp4_gemm_argmax(M: int, N: int, K: int, X: int, Wq: int, Wscale: int, gscale: int,
                      index: int, value: int, workspace: int, workspace_bytes: int,
                      stream: Optional[int]) -> int:
    return load_library().nvfp4_gemm_argmax(M, N, K, X, Wq, Wscale, gscale, index, value,
                                            workspace, workspace_bytes, stream)


def nvfp4_gemm_argmax_path(path: int, split: int, M: int, N: int, K: int, X: int, Wq: int,
                           Wscale: int, gscale: int, index: int, value: int, workspace: int,
                           workspace_bytes: int, stream: Optional[int]) -> int:
    return load_library().nvfp4_gemm_argmax_path(path, split, M, N, K, X, Wq, Wscale, gscale,
                                                 index, value, workspace, workspace_bytes, stream)


def nvfp4_gemm_argmax_noalloc(M: int, N: int, K: int, X: int, Wq: int, Wscale: int, gscale: int,
                              index: int, value: int, stream: Optional[int]) -> int:
    return load_library().nvfp4_gemm_argmax_noalloc(M, N, K, X, Wq, Wscale, gscale, index, value,
                                                    stream)


def nvfp4_argmax_workspace_bytes(M: int) -> int:
    return load_library().nvfp4_argmax_workspace_bytes(M)


def nvfp4_gemm_grouped(T: int, E: int, N: int, K: int, X: int, offsets: int, Wq: int,
                       Wscale: int, gscale: int, Y: int, rows_per_item: int,
                       stream: Optional[int]) -> int:
    return load_library().nvfp4_gemm_grouped(T, E, N, K, X, offsets, Wq, Wscale, gscale, Y,
                                             rows_per_item, stream)


def nvfp4_gemm_fused(fuse: int, M: int, N: int, K: int, X: int, gamma: int, eps: float,
                     Wq: int, Wscale: int, gscale: int, out: int, workspace: int,
                     workspace_bytes: int, stream: Optional[int]) -> int:
    return load_library().nvfp4_gemm_fused(fuse, M, N, K, X, gamma, eps, Wq, Wscale, gscale,
                                           out, workspace, workspace_bytes, stream)


def nvfp4_fused_workspace_bytes(fuse: int, M: int, N: int, K: int) -> int:
    return load_library().nvfp4_fused_workspace_bytes(fuse, M, N, K)


def nvfp4_codes_bytes(N: int, K: int) -> int:
    return load_library().nvfp4_codes_bytes(N, K)


def nvfp4_scales_bytes(N: int, K: int) -> int:
    return load_library().nvfp4_scales_bytes(N, K)


# ---- packed layout (include/nvfp4.h): 4-column groups x 32-k chunks ----

def codes_shape(N: int, K: int):
    """Shape of Wq: [ceil(N/4)][ceil(K/32)][4][16] bytes."""
    return (-(-N // 4), -(-K // 32), 4, 16)


def scales_shape(N: int, K: int):
    """Shape of Wscale: [ceil(N/4)][ceil(K/32)][4][2] bytes."""
    return (-(-N // 4), -(-K // 32), 4, 2)


class Packed(NamedTuple):
    """NVFP4 weights as nvfp4_pack writes them: codes, block scales, tensor scale, and the true
    column count N (the arrays are padded to a multiple of 4 columns)."""
    Wq: torch.Tensor
    Ws: torch.Tensor
    g: torch.Tensor
    N: int


# ---- tensor-level helpers ----

def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check_device(t: torch.Tensor, name: str, dtype: torch.dtype, shape) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def pack(W: torch.Tensor, stream=None, out=None) -> Packed:
    """Quantise fp32 W[K, N] (device) to Packed(Wq, Ws, g, N) in the layout of include/nvfp4.h."""
    K, N = W.shape
    _check_device(W, "W", torch.float32, (K, N))
    if out is None:
        Wq = torch.empty(codes_shape(N, K), dtype=torch.uint8, device=W.device)
        Ws = torch.empty(scales_shape(N, K), dtype=torch.uint8, device=W.device)
        g = torch.empty(1, dtype=torch.float32, device=W.device)
    else:
        Wq, Ws, g = out[:3]
        _check_device(Wq, "Wq", torch.uint8, codes_shape(N, K))
        _check_device(Ws, "Ws", torch.uint8, scales_shape(N, K))
        _check_device(g, "g", torch.float32, (1,))
    st = nvfp4_pack(K, N, W.data_ptr(), Wq.data_ptr(), Ws.data_ptr(), g.data_ptr(),
                    _stream(stream))
    if st != SUCCESS:
        raise NVFP4Error(st, "nvfp4_pack")
    return Packed(Wq, Ws, g, N)


def gemm(X: torch.Tensor, Wq: torch.Tensor, Ws: torch.Tensor, g: torch.Tensor, N: int,
         stream=None, out: Optional[torch.Tensor] = None, path: int = PATH_AUTO, split: int = 0
         ) -> torch.Tensor:
    """Y[M, N] = X[M, K] . dequant(Wq, Ws, g) in fp32. X is bf16 on the device; Wq/Ws are in the
    packed layout (Packed from pack(), or codes_shape/scales_shape arrays)."""
    M, K = X.shape
    _check_device(X, "X", torch.bfloat16, (M, K))
    _check_device(Wq, "Wq", torch.uint8, codes_shape(N, K))
    _check_device(Ws, "Ws", torch.uint8, scales_shape(N, K))
    _check_device(g, "g", torch.float32, (1,))
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    else:
        _check_device(out, "out", torch.float32, (M, N))
    if path == PATH_AUTO and split == 0:
        st = nvfp4_gemm(M, N, K, X.data_ptr(), Wq.data_ptr(), Ws.data_ptr(), g.data_ptr(),
                        out.data_ptr(), _stream(stream))
    else:
        st = nvfp4_gemm_path(path, split, M, N, K, X.data_ptr(), Wq.data_ptr(), Ws.data_ptr(),
                             g.data_ptr(), out.data_ptr(), _stream(stream))
    if st != SUCCESS:
        raise NVFP4Error(st, "nvfp4_gemm")
    return out


def argmax_workspace(M: int, device) -> torch.Tensor:
    """A workspace for gemm_argmax with M rows on `device` (uint8, nvfp4_argmax_workspace_bytes)."""
    with torch.cuda.device(device):
        nbytes = nvfp4_argmax_workspace_bytes(M)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def gemm_argmax(X: torch.Tensor, Wq: torch.Tensor, Ws: torch.Tensor, g: torch.Tensor, N: int,
                stream=None, out=None, workspace: Optional[torch.Tensor] = None,
                path: int = PATH_AUTO, split: int = 0):
    """Greedy token per row of X . dequant(Wq, Ws, g) without writing the logits: returns
    (index int32 [M], value fp32 [M]), the first column of each row's maximum and that maximum,
    for the Y that gemm() with the same path and split computes."""
    M, K = X.shape
    _check_device(X, "X", torch.bfloat16, (M, K))
    _check_device(Wq, "Wq", torch.uint8, codes_shape(N, K))
    _check_device(Ws, "Ws", torch.uint8, scales_shape(N, K))
    _check_device(g, "g", torch.float32, (1,))
    if out is None:
        index = torch.empty(M, dtype=torch.int32, device=X.device)
        value = torch.empty(M, dtype=torch.float32, device=X.device)
    else:
        index, value = out
        _check_device(index, "index", torch.int32, (M,))
        _check_device(value, "value", torch.float32, (M,))
    if workspace is None:
        workspace = argmax_workspace(M, X.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    if path == PATH_AUTO and split == 0:
        st = nvfp4_gemm_argmax(M, N, K, X.data_ptr(), Wq.data_ptr(), Ws.data_ptr(), g.data_ptr(),
                               index.data_ptr(), value.data_ptr(), workspace.data_ptr(),
                               ws_bytes, _stream(stream))
    else:
        st = nvfp4_gemm_argmax_path(path, split, M, N, K, X.data_ptr(), Wq.data_ptr(),
                                    Ws.data_ptr(), g.data_ptr(), index.data_ptr(),
                                    value.data_ptr(), workspace.data_ptr(), ws_bytes,
                                    _stream(stream))
    if st != SUCCESS:
        raise NVFP4Error(st, "nvfp4_gemm_argmax")
    return index, value


def pack_experts(Ws_fp32, stream=None):
    """Quantise a list of E fp32 W[K, N] (device) into back-to-back expert arrays:
    (Wq [E][codes_shape], Ws [E][scales_shape], g [E]), one nvfp4_pack per expert."""
    K, N = Ws_fp32[0].shape
    E = len(Ws_fp32)
    dev = Ws_fp32[0].device
    Wq = torch.empty((E,) + codes_shape(N, K), dtype=torch.uint8, device=dev)
    Wsc = torch.empty((E,) + scales_shape(N, K), dtype=torch.uint8, device=dev)
    g = torch.empty(E, dtype=torch.float32, device=dev)
    for e, W in enumerate(Ws_fp32):
        pack(W, stream=stream, out=(Wq[e], Wsc[e], g[e:e + 1]))
    return Wq, Wsc, g


def gemm_grouped(X: torch.Tensor, offsets: torch.Tensor, Wq: torch.Tensor, Ws: torch.Tensor,
                 g: torch.Tensor, N: int, rows_per_item: int = 0, stream=None,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Grouped GEMM: rows offsets[e] .. offsets[e+1]-1 of X (bf16 [T, K], sorted by expert)
    through expert e's packed weights Wq[e], Ws[e], g[e]; returns fp32 Y [T, N]."""
    T, K = X.shape
    E = Wq.shape[0]
    _check_device(X, "X", torch.bfloat16, (T, K))
    _check_device(offsets, "offsets", torch.int32, (E + 1,))
    _check_device(Wq, "Wq", torch.uint8, (E,) + codes_shape(N, K))
    _check_device(Ws, "Ws", torch.uint8, (E,) + scales_shape(N, K))
    _check_device(g, "g", torch.float32, (E,))
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=X.device)
    else:
        _check_device(out, "out", torch.float32, (T, N))
    st = nvfp4_gemm_grouped(T, E, N, K, X.data_ptr(), offsets.data_ptr(), Wq.data_ptr(),
                            Ws.data_ptr(), g.data_ptr(), out.data_ptr(), rows_per_item,
                            _stream(stream))
    if st != SUCCESS:
        raise NVFP4Error(st, "nvfp4_gemm_grouped")
    return out


def interleave_gate_up(W: torch.Tensor) -> torch.Tensor:
    """Column order nvfp4_gemm_fused's SiLU(gate) * up expects, from a fused gate/up weight
    W[K, 2I] whose first I columns are gate and last I are up: columns 8q .. 8q+3 become gate
    4q .. 4q+3 and 8q+4 .. 8q+7 up 4q .. 4q+3 (I % 4 == 0). A permutation, no arithmetic."""
    K, N2 = W.shape
    I = N2 // 2
    if N2 % 8:
        raise ValueError("the gate/up weight needs 2I columns with I % 4 == 0")
    g = W[:, :I].reshape(K, I // 4, 4)
    u = W[:, I:].reshape(K, I // 4, 4)
    return torch.stack([g, u], dim=2).reshape(K, N2).contiguous()


def fused_workspace(fuse: int, M: int, N: int, K: int, device) -> Optional[torch.Tensor]:
    """A device buffer of nvfp4_fused_workspace_bytes (None when the call needs none)."""
    n = nvfp4_fused_workspace_bytes(fuse, M, N, K)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def gemm_fused(X: torch.Tensor, Wq: torch.Tensor, Ws: torch.Tensor, g: torch.Tensor, N: int,
               gamma: Optional[torch.Tensor] = None, eps: float = 1e-6, silu_mul: bool = False,
               stream=None, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The GEMM with its layer neighbours: RMSNorm(X; gamma, eps) first when gamma is given, and
    SiLU(gate) * up of an interleaved gate/up weight (interleave_gate_up) when silu_mul. Returns
    fp32 Y [M, N], or bf16 H [M, N/2] with silu_mul. `workspace` (device bytes) is allocated here
    when the call needs one and none is given."""
    M, K = X.shape
    _check_device(X, "X", torch.bfloat16, (M, K))
    _check_device(Wq, "Wq", torch.uint8, codes_shape(N, K))
    _check_device(Ws, "Ws", torch.uint8, scales_shape(N, K))
    _check_device(g, "g", torch.float32, (1,))
    fuse = 0
    if gamma is not None:
        _check_device(gamma, "gamma", torch.bfloat16, (K,))
        fuse |= FUSE_RMSNORM
    if silu_mul:
        fuse |= FUSE_SILU_MUL
    if fuse == 0:
        raise ValueError("gemm_fused needs gamma, silu_mul or both (else use gemm)")
    shape, dtype = ((M, N // 2), torch.bfloat16) if silu_mul else ((M, N), torch.float32)
    if out is None:
        out = torch.empty(shape, dtype=dtype, device=X.device)
    else:
        _check_device(out, "out", dtype, shape)
    if workspace is None:
        workspace = fused_workspace(fuse, M, N, K, X.device)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = nvfp4_gemm_fused(fuse, M, N, K, X.data_ptr(), 0 if gamma is None else gamma.data_ptr(),
                          float(eps), Wq.data_ptr(), Ws.data_ptr(), g.data_ptr(), out.data_ptr(),
                          ws_ptr, ws_bytes, _stream(stream))
    if st != SUCCESS:
        raise NVFP4Error(st, "nvfp4_gemm_fused")
    return out
