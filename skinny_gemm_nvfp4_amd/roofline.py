"""Byte and flop accounting of the NVFP4 skinny GEMM, and the bandwidth model of decode.

Decode at concurrency 1 reads the whole model once per token, so tokens/s = read rate / bytes
per token; the page's model predicted 89.7 tok/s for the NVFP4-lm_head build from the earlier
build's 18.80 GiB at 81.6 tok/s and the lm_head's 2.54 GB -> 0.72 GB ("Qwen3.8-27B-NVFP4-RTX5090"
model card, section "Why lm_head is NVFP4, and why MTP is gone").

NVFP4 costs 4 bits per weight plus one E4M3 byte per 16 weights: 0.5625 byte per weight.
"""
from __future__ import annotations

# MI355X published peaks used for the roofline fractions.
HBM_PEAK_GBS = 8000.0            # HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA, TFLOP/s

BYTES_PER_WEIGHT = 0.5 + 1.0 / 16.0


def weight_bytes(K: int, N: int) -> int:
    """Packed NVFP4 bytes of a K x N weight: codes, block scales and the fp32 tensor scale."""
    return N * K // 2 + N * K // 16 + 4


def compulsory_bytes(M: int, N: int, K: int) -> int:
    """Bytes one GEMM call must move at least: packed weights, bf16 X in, fp32 Y out."""
    return weight_bytes(K, N) + 2 * M * K + 4 * M * N


def flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def hbm_time_s(M: int, N: int, K: int) -> float:
    return compulsory_bytes(M, N, K) / (HBM_PEAK_GBS * 1e9)


def mfma_time_s(M: int, N: int, K: int) -> float:
    """Time of the bf16 MFMA work at peak; M is padded to the 16-row MFMA tile."""
    m_pad = -(-M // 16) * 16
    return flops(m_pad, N, K) / (MFMA_BF16_PEAK_TFLOPS * 1e12)


def binding_roof(M: int, N: int, K: int) -> str:
    return "mfma" if mfma_time_s(M, N, K) > hbm_time_s(M, N, K) else "hbm"


def tokens_per_second(read_rate_bytes_s: float, bytes_per_token: float) -> float:
    """The bandwidth model: one full read of the weights per decoded token."""
    return read_rate_bytes_s / bytes_per_token


def predicted_tok_s_after_removing(bytes_per_token: float, tok_s: float,
                                   bytes_removed: float) -> float:
    """The page's prediction: same read rate, fewer bytes per token."""
    rate = bytes_per_token * tok_s
    return tokens_per_second(rate, bytes_per_token - bytes_removed)
