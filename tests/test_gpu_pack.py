"""GPU pack (nvfp4_pack through the C ABI) must equal the oracle quantiser byte for byte.

The quantised bytes are unique under the recipe's readings (nearest, ties to even, saturation,
fp32 one step at a time), so the comparison is bit-exact for codes, scale bytes and g.
"""
import numpy as np
import pytest
import torch

from skinny_gemm_nvfp4_amd import inputs
from parity import assert_pack_equal

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K,N", [(16, 1), (32, 17), (48, 5), (272, 33), (1024, 2048)])
def test_pack_random_shapes(device, K, N):
    W = inputs.weights(inputs.generator(100 + K + N), K, N)
    assert_pack_equal(W, device, f"random K={K} N={N}")


def test_pack_zero_tensor(device):
    W = torch.zeros(64, 8)
    (Wq, Ws, g, _n), _ = assert_pack_equal(W, device, "zeros")
    assert float(g.cpu()[0]) == 0.0
    assert int(Wq.sum().cpu()) == 0 and int(Ws.sum().cpu()) == 0


def test_pack_signed_zeros_and_ties(device):
    # Blocks built so that w / (s g) lands exactly on E2M1 midpoints; the sign of tiny values
    # must survive as code 8 (-0).
    K, N = 32, 4
    W = torch.zeros(K, N)
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    W[:8, 0] = mids
    W[8:16, 0] = -mids
    W[:16, 1] = torch.linspace(-6, 6, 16)
    W[16:32, 2] = -1e-3
    W[16, 2] = 6.0
    W[:, 3] = -0.0
    assert_pack_equal(W, device, "ties")


def test_pack_wide_dynamic_range(device):
    # One huge block next to tiny ones: tiny blocks get subnormal or zero E4M3 scales.
    K, N = 256, 64
    gen = inputs.generator(7)
    W = inputs.weights(gen, K, N)
    W[:16, 0] *= 1e6
    W[:, 1:8] *= torch.logspace(-12, -2, 7)
    W[32:48, 9] = 0.0
    assert_pack_equal(W, device, "dynamic range")


def test_pack_denormal_inputs(device):
    # amax so small that g and s*g are fp32 subnormals; the two sides must still agree.
    K, N = 64, 16
    W = inputs.weights(inputs.generator(3), K, N) * 1e-33
    assert_pack_equal(W, device, "subnormal")


def test_pack_underflowing_tensor_scale(device):
    # amax / 2688 rounds to 0: every byte must be 0.
    W = torch.full((16, 3), 1e-45)
    (Wq, Ws, g, _n), _ = assert_pack_equal(W, device, "g underflow")
    assert float(g.cpu()[0]) == 0.0


def test_pack_layer_shapes(device):
    # Full-size quantisation of the dense-layer weights (seeds 1-4).
    for name, seed in (("qkv", 1), ("o_proj", 2), ("gate_up", 3), ("down", 4)):
        K, N = inputs.LAYER_SHAPES[name]
        W = inputs.weights(inputs.generator(seed), K, N)
        assert_pack_equal(W, device, name)


def test_pack_is_deterministic(device):
    W = inputs.weights(inputs.generator(11), 512, 300).to(device)
    import skinny_gemm_nvfp4_amd as nv
    a = nv.pack(W)
    b = nv.pack(W)
    torch.cuda.synchronize()
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    assert np.isfinite(float(a[2].cpu()[0]))
