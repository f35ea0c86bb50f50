"""Pins of the oracle's layer neighbours: bf16_round, rmsnorm_bf16 and silu_mul ("SparkInfer"
README, section "Layout & scoring": RMSNorm and fused FFN kernels beside the decode GEMV).

  * bf16_round against torch's float32 -> bfloat16 cast (round to nearest, ties to even) on
    values that are exact in float32 (so one rounding either way), ties and subnormals included;
  * rmsnorm closed forms: a constant row c with eps = 0 normalises to gamma * sign(c) exactly;
    a row (3, 4, 0, ..., 0) has mean square 25 / K; scaling a row does not change its result
    (eps = 0); eps enters under the square root;
  * the flag marks exactly the values near a rounding boundary;
  * silu_mul: silu(0) = 0, silu(x) - silu(-x) = x, silu(x) -> x for large x and -> 0 for very
    negative x, and the product with up.
"""
import numpy as np
import torch

import oracle


def _bits(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def test_bf16_round_matches_torch_cast_on_float32_values():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-39).astype(np.float32),   # subnormal
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -133,
                                  3 * 2 ** -134, 0.0], dtype=np.float32)])        # ties
    bits, vals, ulp, dist = oracle.bf16_round(v.astype(np.float64))
    assert np.array_equal(bits, _bits(v))
    assert np.all(np.abs(vals - v) <= ulp / 2)
    assert dist[-6] == 0.0 and dist[-5] == 0.0          # exact ties sit on a boundary


def test_rmsnorm_constant_rows_give_gamma():
    K = 64
    gamma = np.linspace(0.5, 1.5, K).astype(np.float32)
    gb = _bits(gamma)
    g = (gb.astype(np.uint32) << 16).view(np.float32)
    X = np.stack([np.full(K, 3.0), np.full(K, -0.25)]).astype(np.float32)
    xhat, flag, _ = oracle.rmsnorm_bf16(_bits(X), gb, 0.0, 1e-6)
    got = (xhat.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(got[0], g) and np.array_equal(got[1], -g)
    assert not flag.any()


def test_rmsnorm_mean_square_scale_invariance_and_eps():
    K = 32
    x = np.zeros((1, K), dtype=np.float32)
    x[0, 0], x[0, 1] = 3.0, 4.0
    ones = _bits(np.ones(K, dtype=np.float32))
    xhat, _, _ = oracle.rmsnorm_bf16(_bits(x), ones, 0.0, 0.0)
    got = (xhat.astype(np.uint32) << 16).view(np.float32)
    rms = np.sqrt(25.0 / K)
    assert got[0, 0] == np.float32(torch.tensor(3.0 / rms).to(torch.bfloat16).item())
    assert got[0, 1] == np.float32(torch.tensor(4.0 / rms).to(torch.bfloat16).item())
    rng = np.random.default_rng(1)
    y = rng.standard_normal((3, 256)).astype(np.float32)
    yb = _bits(y)
    y2 = (yb.astype(np.uint32) << 16).view(np.float32) * 4.0     # exact scaling of bf16 values
    g = _bits(rng.uniform(0.5, 1.5, 256).astype(np.float32))
    a, _, _ = oracle.rmsnorm_bf16(yb, g, 0.0, 0.0)
    b, _, _ = oracle.rmsnorm_bf16(_bits(y2), g, 0.0, 0.0)
    assert np.array_equal(a, b)
    c, _, _ = oracle.rmsnorm_bf16(_bits(np.full((1, 16), 1.0, np.float32)), ones[:16], 3.0, 0.0)
    assert (c.astype(np.uint32) << 16).view(np.float32)[0, 0] == np.float32(0.5)   # 1/sqrt(1+3)


def test_rmsnorm_flags_values_near_boundaries():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((4, 512)).astype(np.float32)
    gb = _bits(rng.uniform(0.8, 1.2, 512).astype(np.float32))
    xb = _bits(X)
    _, f_small, _ = oracle.rmsnorm_bf16(xb, gb, 1e-6, 1e-7)
    _, f_big, ulp = oracle.rmsnorm_bf16(xb, gb, 1e-6, 1e-3)
    assert f_small.sum() < f_big.sum() and np.all(f_big[f_small])
    # about 2 * window / (relative spacing) of the elements are flagged
    assert 0.05 < f_big.mean() < 0.8
    assert np.all(ulp > 0)


def test_silu_mul_identities():
    x = np.linspace(-30, 30, 601)
    s = oracle.silu_mul(x, np.ones_like(x))
    assert s[300] == 0.0
    assert np.allclose(s - s[::-1], x, rtol=0, atol=1e-12)
    assert abs(oracle.silu_mul(np.array([40.0]), np.array([1.0]))[0] - 40.0) < 1e-12
    assert abs(oracle.silu_mul(np.array([-800.0]), np.array([1.0]))[0]) == 0.0
    assert np.allclose(oracle.silu_mul(x, np.full_like(x, 2.5)), 2.5 * s, rtol=1e-15, atol=0)
