"""Seeded synthetic inputs for the NVFP4 skinny-GEMM workloads.

This module holds random draws and nothing of the method's arithmetic: no quantisation, no
decoding, no GEMM. Both the HIP path and the CPU oracle take their inputs from here, so it is the
only code the two share.

Recipe (the readings behind it are listed in the design doc):
  * A generator is ``torch.Generator("cpu").manual_seed(seed)``. Within one seed the weights are
    drawn first, in the order the workload lists them, then the activations.
  * Weights W[K, N] are fp32 ``randn * 0.02`` (normal, standard deviation 0.02).
  * Activations X[M, K] are fp32 ``randn``, optionally with a few outlier channels (K indices drawn
    with ``randperm`` after X) multiplied by 20, then cast to bf16 with round-to-nearest-even.
  * The 5120-hidden dense decoder layer matches the shapes of the pages' 27B dense model family:
    q/k/v fused N = 5120 + 2*1024, o_proj 5120x5120, gate/up fused N = 2*17408, down K = 17408.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np
import torch

HIDDEN = 5120
INTERMEDIATE = 17408
KV_DIM = 1024
VOCAB = 151936

# name -> (K, N) of the four projections of one dense decoder layer.
LAYER_SHAPES: Dict[str, Tuple[int, int]] = {
    "qkv": (HIDDEN, HIDDEN + 2 * KV_DIM),
    "o_proj": (HIDDEN, HIDDEN),
    "gate_up": (HIDDEN, 2 * INTERMEDIATE),
    "down": (INTERMEDIATE, HIDDEN),
}
LM_HEAD_SHAPE = (HIDDEN, VOCAB)


def generator(seed: int) -> torch.Generator:
    return torch.Generator("cpu").manual_seed(int(seed))


def weights(gen: torch.Generator, K: int, N: int) -> torch.Tensor:
    """fp32 W[K, N] drawn from N(0, 0.02^2) on the CPU."""
    return torch.randn(K, N, generator=gen, dtype=torch.float32) * 0.02


def weights_on_device(gen: torch.Generator, K: int, N: int, device) -> torch.Tensor:
    """fp32 W[K, N] from N(0, 0.02^2) drawn with a device generator (for the full weight pass)."""
    return torch.randn(K, N, generator=gen, dtype=torch.float32, device=device) * 0.02


def activations(gen: torch.Generator, M: int, K: int, outliers: int = 0) -> torch.Tensor:
    """bf16 X[M, K] from N(0, 1); ``outliers`` channels (same for every row) scaled by 20."""
    x = torch.randn(M, K, generator=gen, dtype=torch.float32)
    if outliers:
        idx = torch.randperm(K, generator=gen)[:outliers]
        x[:, idx] *= 20.0
    return x.to(torch.bfloat16)


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """The uint16 bit patterns of a bf16 tensor (what the oracle takes)."""
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclass
class Gemm:
    """One GEMM of a workload: fp32 weights to quantise and bf16 activations."""
    name: str
    W: torch.Tensor            # fp32 [K, N], CPU
    X: torch.Tensor            # bf16 [M, K], CPU

    @property
    def shape(self) -> Tuple[int, int, int]:
        M, K = self.X.shape
        return M, self.W.shape[1], K


@dataclass
class Workload:
    name: str
    description: str
    gemms: List[Gemm] = field(default_factory=list)


def single_gemv() -> Workload:
    """M=1, K=1024, N=2048, seed 0 (W drawn first, then X)."""
    gen = generator(0)
    W = weights(gen, 1024, 2048)
    X = activations(gen, 1, 1024)
    return Workload("single_gemv", "M=1 K=1024 N=2048 seed 0", [Gemm("gemv", W, X)])


def dense_layer_m1(names=("qkv", "o_proj", "gate_up", "down")) -> Workload:
    """One dense decoder layer at M=1. Seeds 1-4: the four weights; seed 5: x for K=5120;
    seed 6: x for K=17408. Four outlier channels x20 in each x."""
    seeds = {"qkv": 1, "o_proj": 2, "gate_up": 3, "down": 4}
    x5120 = activations(generator(5), 1, HIDDEN, outliers=4)
    x17408 = activations(generator(6), 1, INTERMEDIATE, outliers=4)
    gemms = []
    for name in names:
        K, N = LAYER_SHAPES[name]
        W = weights(generator(seeds[name]), K, N)
        gemms.append(Gemm(name, W, x17408 if K == INTERMEDIATE else x5120))
    return Workload("dense_layer_m1", "dense 5120-hidden layer, M=1, seeds 1-6", gemms)


def verify_m16() -> Workload:
    """Speculative verify of one request: M=16 on gate_up and down, seed 7."""
    gen = generator(7)
    Wg = weights(gen, *LAYER_SHAPES["gate_up"])
    Wd = weights(gen, *LAYER_SHAPES["down"])
    xg = activations(gen, 16, HIDDEN)
    xd = activations(gen, 16, INTERMEDIATE)
    return Workload("verify_m16", "M=16 gate_up and down, seed 7",
                    [Gemm("gate_up", Wg, xg), Gemm("down", Wd, xd)])


def batched_verify_m128() -> Workload:
    """8 requests x 16 tokens: M=128 on the four layer shapes, seed 8."""
    gen = generator(8)
    Ws = {name: weights(gen, *LAYER_SHAPES[name]) for name in LAYER_SHAPES}
    x5120 = activations(gen, 128, HIDDEN)
    x17408 = activations(gen, 128, INTERMEDIATE)
    return Workload("batched_verify_m128", "M=128 on the four layer shapes, seed 8",
                    [Gemm(name, Ws[name], x17408 if LAYER_SHAPES[name][0] == INTERMEDIATE
                          else x5120) for name in LAYER_SHAPES])


def full_pass_shapes(layers: int = 64) -> List[Tuple[str, int, int]]:
    """(name, K, N) of every GEMM of the full weight pass, in pass order."""
    out = []
    for layer in range(layers):
        for name, (K, N) in LAYER_SHAPES.items():
            out.append((f"layer{layer}.{name}", K, N))
    out.append(("lm_head", *LM_HEAD_SHAPE))
    return out


def full_pass_activations(M: int) -> Dict[int, torch.Tensor]:
    """Seed 10: x for K=5120 and K=17408 at M rows (the M=1 pass uses the first row of M=16)."""
    gen = generator(10)
    x5120 = activations(gen, 16, HIDDEN)
    x17408 = activations(gen, 16, INTERMEDIATE)
    return {HIDDEN: x5120[:M].contiguous(), INTERMEDIATE: x17408[:M].contiguous()}


# --------------------------------------------------------------------------------------------
# Constructed inputs for the exactness tests: random bytes, no arithmetic of the method.
# --------------------------------------------------------------------------------------------

def random_packed(gen: torch.Generator, N: int, K: int, scale_bytes=None):
    """Random code bytes Wq[N][K/2] and scale bytes Ws[N][K/16].

    ``scale_bytes`` restricts the scale bytes to the given list (drawn uniformly from it);
    otherwise every byte value 0..255 may appear.
    """
    Wq = torch.randint(0, 256, (N, K // 2), generator=gen, dtype=torch.int32).to(torch.uint8)
    if scale_bytes is None:
        Ws = torch.randint(0, 256, (N, K // 16), generator=gen, dtype=torch.int32)
    else:
        choice = torch.tensor(list(scale_bytes), dtype=torch.int32)
        Ws = choice[torch.randint(0, len(choice), (N, K // 16), generator=gen)]
    return Wq, Ws.to(torch.uint8)


def integer_activations(gen: torch.Generator, M: int, K: int, lo: int = -8, hi: int = 8):
    """bf16 X[M, K] holding integers in [lo, hi] (exact in bf16)."""
    x = torch.randint(lo, hi + 1, (M, K), generator=gen, dtype=torch.int32)
    return x.to(torch.float32).to(torch.bfloat16)


# ---- mixture-of-experts workload (grouped GEMM) ----
# Expert shapes of a small mixture-of-experts model of the pages' family (a 3B-active MoE of the
# size the SparkInfer README benchmarks): hidden 2048, 128 experts, 8 routed per token, expert
# intermediate 768, so gate/up is K = 2048, N = 2 * 768 and down is K = 768, N = 2048.
MOE_HIDDEN = 2048
MOE_EXPERTS = 128
MOE_TOPK = 8
MOE_INTERMEDIATE = 768
MOE_SHAPES: Dict[str, Tuple[int, int]] = {
    "gate_up": (MOE_HIDDEN, 2 * MOE_INTERMEDIATE),
    "down": (MOE_INTERMEDIATE, MOE_HIDDEN),
}


def moe_routing(gen: torch.Generator, tokens: int, experts: int, topk: int):
    """Synthetic router output, sorted for dispatch: each token picks `topk` distinct experts
    uniformly (randperm per token). Returns (token of each dispatched row, offsets [E + 1]): rows
    are grouped by expert, tokens ascending within an expert; expert e owns rows offsets[e] ..
    offsets[e+1] - 1."""
    picks = [torch.randperm(experts, generator=gen)[:topk] for _ in range(tokens)]
    pairs = sorted((int(e), t) for t, p in enumerate(picks) for e in p)
    token_of_row = torch.tensor([t for _, t in pairs], dtype=torch.int64)
    counts = torch.zeros(experts, dtype=torch.int64)
    for e, _ in pairs:
        counts[e] += 1
    offsets = torch.zeros(experts + 1, dtype=torch.int32)
    offsets[1:] = torch.cumsum(counts, 0).to(torch.int32)
    return token_of_row, offsets


# ---- layer neighbours (RMSNorm before the GEMM) ----
RMSNORM_EPS = 1e-6


def norm_weight(gen: torch.Generator, K: int) -> torch.Tensor:
    """bf16 RMSNorm gain gamma[K] = 1 + 0.1 N(0, 1) (a trained norm's gains sit around 1)."""
    return (1.0 + 0.1 * torch.randn(K, generator=gen, dtype=torch.float32)).to(torch.bfloat16)


# ---- one GPU's share of an 8-way tensor-parallel layer ----
TP = 8
# name -> (K, N): column-parallel projections split N, row-parallel ones split K.
TP8_SHARD_SHAPES: Dict[str, Tuple[int, int]] = {
    "qkv": (HIDDEN, (HIDDEN + 2 * KV_DIM) // TP),
    "o_proj": (HIDDEN // TP, HIDDEN),
    "gate_up": (HIDDEN, 2 * INTERMEDIATE // TP),
    "down": (INTERMEDIATE // TP, HIDDEN),
}
