"""One GPU's share of the dense layer under 8-way tensor parallelism (the sharding plan: q/k/v
and gate/up split their columns, o_proj and down their K), at M = 1, 16 and 128, through
nvfp4_gemm, against the oracle. down's shard has K = 2176 and o_proj's K = 640, neither a
multiple of 512, so the dot-product kernel takes its per-lane K test."""
import numpy as np
import pytest

import oracle
from skinny_gemm_nvfp4_amd import inputs
from parity import assert_pack_equal, check_close, gpu_gemm, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [1, 16, 128])
def test_tp8_shard_shapes(device, M):
    gen = inputs.generator(4000 + M)
    for name, (K, N) in inputs.TP8_SHARD_SHAPES.items():
        W = inputs.weights(gen, K, N)
        X = inputs.activations(gen, M, K, outliers=4)
        packed_d, (Wq_o, Ws_o, g_o) = assert_pack_equal(W, device, f"tp8 {name}")
        say(f"tp8 shard {name} M={M} N={N} K={K}")
        Y = gpu_gemm(X, packed_d, device)
        Yref, A = oracle.gemm(inputs.bf16_bits(X), Wq_o, Ws_o, g_o)
        worst = check_close(Y, Yref, A, f"tp8 {name} M={M}")
        say(f"  worst error / bound = {worst:.3g}")
