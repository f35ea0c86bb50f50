"""CPU oracle for the NVFP4 skinny GEMM -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package. It
shares no code with the HIP library and imports nothing from it. Every function takes and returns
numpy arrays; the arithmetic is in nvfp4_oracle.c (decoders by closed form, rounding by
enumeration, the quantisation recipe in fp32 one step at a time, the GEMM in double).

What it computes, from the pages and the workload recipe:
  "Qwen3.8-27B-NVFP4-RTX5090" model card, table "Recipe (NVIDIA ModelOpt)": NVFP4 weights with group
  size 16; section "Why lm_head is NVFP4": decode streams every weight once per token.
  Per tensor g = amax / (6*448); per 16-block along K an E4M3 scale s = round(block_amax / (6g));
  codes = round-to-nearest E2M1 of w / (s*g); Y = X . (e2m1(code) * s * g).
  Greedy token per row = first column of the row maximum ("SparkInfer" README, greedy decode).
  Grouped GEMM: expert-sorted rows through their expert's weights ("SparkInfer" README, fused
  MoE FFN and expert dispatch).
  Layer neighbours: RMSNorm to bf16 before the GEMM, SiLU(gate) * up after it ("SparkInfer"
  README, RMSNorm and fused FFN kernels).
Pins for every function live in tests/test_oracle_*.py; none is "parity unpinned".
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    """Load the compiled oracle, compiling it first if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB) or (
            os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
        _build.build()
    L = ctypes.CDLL(_build.LIB)
    c_u8p = ctypes.POINTER(ctypes.c_uint8)
    c_fp = ctypes.POINTER(ctypes.c_float)
    c_dp = ctypes.POINTER(ctypes.c_double)
    L.oracle_e2m1_value.argtypes = [ctypes.c_int]
    L.oracle_e2m1_value.restype = ctypes.c_double
    L.oracle_e4m3_value.argtypes = [ctypes.c_int]
    L.oracle_e4m3_value.restype = ctypes.c_double
    L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    L.oracle_bf16_value.restype = ctypes.c_double
    L.oracle_e2m1_round.argtypes = [ctypes.c_float]
    L.oracle_e2m1_round.restype = ctypes.c_uint8
    L.oracle_e4m3_round.argtypes = [ctypes.c_float]
    L.oracle_e4m3_round.restype = ctypes.c_uint8
    L.oracle_e2m1_round_array.argtypes = [c_fp, ctypes.c_size_t, c_u8p]
    L.oracle_e2m1_round_array.restype = None
    L.oracle_e4m3_round_array.argtypes = [c_fp, ctypes.c_size_t, c_u8p]
    L.oracle_e4m3_round_array.restype = None
    L.oracle_quantize.argtypes = [ctypes.c_int, ctypes.c_int, c_fp, c_u8p, c_u8p, c_fp]
    L.oracle_quantize.restype = None
    L.oracle_dequantize.argtypes = [ctypes.c_int, ctypes.c_int, c_u8p, c_u8p, ctypes.c_float, c_dp]
    L.oracle_dequantize.restype = None
    L.oracle_gemm.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                              ctypes.POINTER(ctypes.c_uint16), c_u8p, c_u8p, ctypes.c_float,
                              ctypes.POINTER(ctypes.c_int), ctypes.c_int, c_dp, c_dp]
    L.oracle_gemm.restype = ctypes.c_int
    L.oracle_num_threads.argtypes = []
    L.oracle_num_threads.restype = ctypes.c_int
    L.oracle_set_num_threads.argtypes = [ctypes.c_int]
    L.oracle_set_num_threads.restype = None
    _lib = L
    return L


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return lib().oracle_e4m3_value(int(byte))


def bf16_value(bits: int) -> float:
    return lib().oracle_bf16_value(int(bits))


def e2m1_round(q) -> np.ndarray:
    """Nearest E2M1 code (ties to even, saturating) for every float32 in q."""
    q = np.ascontiguousarray(q, dtype=np.float32).reshape(-1)
    out = np.empty(q.size, dtype=np.uint8)
    lib().oracle_e2m1_round_array(_ptr(q, ctypes.c_float), q.size, _ptr(out, ctypes.c_uint8))
    return out


def e4m3_round(t) -> np.ndarray:
    """Nearest finite E4M3 byte (ties to even, saturating at 448) for every float32 in t."""
    t = np.ascontiguousarray(t, dtype=np.float32).reshape(-1)
    out = np.empty(t.size, dtype=np.uint8)
    lib().oracle_e4m3_round_array(_ptr(t, ctypes.c_float), t.size, _ptr(out, ctypes.c_uint8))
    return out


def quantize(W: np.ndarray):
    """fp32 W[K][N] -> (Wq uint8 [N][K/2], Ws uint8 [N][K/16], g float32)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    K, N = W.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    Wq = np.empty((N, K // 2), dtype=np.uint8)
    Ws = np.empty((N, K // 16), dtype=np.uint8)
    g = np.zeros(1, dtype=np.float32)
    lib().oracle_quantize(K, N, _ptr(W, ctypes.c_float), _ptr(Wq, ctypes.c_uint8),
                          _ptr(Ws, ctypes.c_uint8), _ptr(g, ctypes.c_float))
    return Wq, Ws, np.float32(g[0])


def dequantize(Wq: np.ndarray, Ws: np.ndarray, g) -> np.ndarray:
    """Exact dequantised weights, float64 [K][N]."""
    Wq = np.ascontiguousarray(Wq, dtype=np.uint8)
    Ws = np.ascontiguousarray(Ws, dtype=np.uint8)
    N, Kh = Wq.shape
    K = 2 * Kh
    if Ws.shape != (N, K // 16):
        raise ValueError("scale shape does not match the codes")
    Wd = np.empty((K, N), dtype=np.float64)
    lib().oracle_dequantize(K, N, _ptr(Wq, ctypes.c_uint8), _ptr(Ws, ctypes.c_uint8),
                            ctypes.c_float(float(g)), _ptr(Wd, ctypes.c_double))
    return Wd


def gemm(X_bits: np.ndarray, Wq: np.ndarray, Ws: np.ndarray, g, cols=None):
    """Y and A = sum |x*w| in float64, shape [M][len(cols)] (all N columns if cols is None).

    X_bits is the bf16 bit pattern as uint16 [M][K].
    """
    X_bits = np.ascontiguousarray(X_bits, dtype=np.uint16)
    Wq = np.ascontiguousarray(Wq, dtype=np.uint8)
    Ws = np.ascontiguousarray(Ws, dtype=np.uint8)
    M, K = X_bits.shape
    N = Wq.shape[0]
    if Wq.shape != (N, K // 2) or Ws.shape != (N, K // 16):
        raise ValueError("weight shapes do not match X")
    if cols is None:
        cols_arr = None
        ncols = N
    else:
        cols_arr = np.ascontiguousarray(cols, dtype=np.int32)
        if cols_arr.size and (cols_arr.min() < 0 or cols_arr.max() >= N):
            raise ValueError("column index out of range")
        ncols = cols_arr.size
    Y = np.empty((M, ncols), dtype=np.float64)
    A = np.empty((M, ncols), dtype=np.float64)
    rc = lib().oracle_gemm(M, N, K, _ptr(X_bits, ctypes.c_uint16), _ptr(Wq, ctypes.c_uint8),
                           _ptr(Ws, ctypes.c_uint8), ctypes.c_float(float(g)),
                           None if cols_arr is None else _ptr(cols_arr, ctypes.c_int), ncols,
                           _ptr(Y, ctypes.c_double), _ptr(A, ctypes.c_double))
    if rc:
        raise MemoryError("oracle_gemm could not allocate its buffers")
    return Y, A


def grouped_gemm(X_bits: np.ndarray, offsets, Wq: np.ndarray, Ws: np.ndarray, g):
    """Grouped (mixture-of-experts) GEMM: rows offsets[e] .. offsets[e+1]-1 of X go through
    expert e's weights, Y[t] = X[t] . dequant(Wq[e], Ws[e], g[e]). Returns Y and A = sum |x*w|,
    float64 [T][N].

    The pages' engine has a fused MoE FFN kernel and a sync-free router with expert dispatch
    ("SparkInfer" README, section "Layout & scoring"); its MoE targets read only the routed
    experts' weights per token. Rows arrive sorted by expert (the router's dispatch order);
    offsets has E + 1 non-decreasing entries from 0 to T. Each expert's block is the plain GEMM
    of this module, so the arithmetic is exactly gemm()'s.
    """
    X_bits = np.ascontiguousarray(X_bits, dtype=np.uint16)
    offsets = np.asarray(offsets, dtype=np.int64)
    E = Wq.shape[0]
    T, K = X_bits.shape
    N = Wq.shape[1]
    if offsets.shape != (E + 1,) or offsets[0] != 0 or offsets[-1] != T or \
            np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must be E + 1 non-decreasing entries from 0 to T")
    g = np.broadcast_to(np.asarray(g, dtype=np.float32), (E,))
    Y = np.zeros((T, N), dtype=np.float64)
    A = np.zeros((T, N), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            Y[r0:r1], A[r0:r1] = gemm(X_bits[r0:r1], Wq[e], Ws[e], g[e])
    return Y, A


def bf16_round(v: np.ndarray):
    """Round float64 values to bf16, to nearest with ties to even, in one step (no float32 in
    between). Returns (bf16 bit patterns uint16, the exact rounded values float64, the spacing
    of bf16 values at each input's binade float64, the distance of each input to the nearest
    rounding boundary float64). Finite inputs below the bf16 overflow threshold only."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                       # v = f * 2^e, 0.5 <= |f| < 1
    e = np.maximum(e, -125)                  # subnormal bf16 spacing stays 2^-133
    ulp = np.ldexp(1.0, e - 8)               # 8 significant bits
    q = v / ulp                              # exact: division by a power of two
    r = np.rint(q)                           # nearest integer, ties to even
    vals = r * ulp
    dist = np.abs(np.abs(q - np.floor(q)) - 0.5) * ulp
    bits = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return bits, vals, ulp, dist


def rmsnorm_bf16(X_bits: np.ndarray, gamma_bits: np.ndarray, eps: float, window: float):
    """RMSNorm of bf16 rows, rounded to the bf16 activations a GEMM takes:
    xhat[m, k] = bf16( x[m, k] * gamma[k] / sqrt(mean_k x[m, k]^2 + eps) ), computed in float64
    and rounded once.

    The pages' engine has an RMSNorm kernel next to its decode GEMV ("SparkInfer" README, section
    "Layout & scoring"); in a dense decoder layer it produces the input of the q/k/v and gate/up
    projections. The pages fix neither the precision nor the rounding of its output; the reading
    here is the exact value rounded to nearest-even bf16.

    A kernel computes the same value in fp32, within a relative error it states; where the exact
    value lies within `window` (relative) of a bf16 rounding boundary, either neighbour is a
    correct result. Returns (xhat bits uint16 [M][K], flag bool [M][K] marking those elements,
    ulp float64 [M][K] = the bf16 spacing there).
    """
    X_bits = np.ascontiguousarray(X_bits, dtype=np.uint16)
    gamma_bits = np.ascontiguousarray(gamma_bits, dtype=np.uint16)
    x = (X_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    gam = (gamma_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if x.ndim != 2 or gam.shape != (x.shape[1],):
        raise ValueError("X must be [M][K] and gamma [K]")
    ms = np.mean(x * x, axis=1, keepdims=True)
    v = x * gam[None, :] / np.sqrt(ms + float(eps))
    bits, _, ulp, dist = bf16_round(v)
    flag = dist < window * np.abs(v)
    return bits, flag, ulp


def silu_mul(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """Gated FFN activation of the dense layer family: SiLU(gate) * up = gate * up / (1 + e^-gate),
    float64, elementwise. The pages name the fused FFN next to the GEMMs ("SparkInfer" README,
    "Layout & scoring"); the SiLU gate is the reading taken for that family's FFN."""
    gate = np.asarray(gate, dtype=np.float64)
    up = np.asarray(up, dtype=np.float64)
    with np.errstate(over="ignore"):
        return gate * up / (1.0 + np.exp(-gate))


def argmax_rows(Y: np.ndarray) -> np.ndarray:
    """Greedy token of every row: the first column n holding max over n of Y[m, n] (int64 [M]).

    Greedy decode and greedy speculative verification pick this column of the lm_head's logits
    for each row ("SparkInfer" README: decode and the DSpark/DFlash2 figures are measured greedy,
    and a request speculating alone gets the tokens it gets without the drafter). Y is the
    oracle's own float64 result. Equal values (including -0 and +0) go to the smaller column;
    numpy's argmax is that definition (first occurrence of the maximum).
    """
    Y = np.asarray(Y, dtype=np.float64)
    if Y.ndim != 2 or Y.shape[1] == 0:
        raise ValueError("Y must be [M][N] with N >= 1")
    if np.isnan(Y).any():
        raise ValueError("NaN logits are outside the oracle's contract")
    return np.argmax(Y, axis=1)


def num_threads() -> int:
    """Threads the oracle's OpenMP loops run on."""
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops from now on (for timing it on one core)."""
    lib().oracle_set_num_threads(int(n))


def tolerance(A: np.ndarray) -> np.ndarray:
    """Per-output acceptance bound |Y - Y_ref| <= 2e-3 * sum|x*w| + 1e-6."""
    return 2e-3 * A + 1e-6
