"""Pins of the oracle's rounding (nearest representable value, ties to the even code, saturating).

The oracle rounds by enumerating candidates. The pins use different routes:
  * E2M1: every fp32 in [2^-3, 8) (where all decision boundaries lie), exhaustively, against a
    grid snap written with numpy's rint (half to even); sampled smaller and larger values,
    infinities and the sign rule.
  * E4M3: torch's fp32 -> float8_e4m3fn cast (OCP E4M3FN, round half to even) at every value,
    midpoint and neighbouring ulp of the format below 464, and on 4 million random inputs; the
    saturation above 448 (where torch gives NaN from 480 on) against the closed form.
"""
import numpy as np
import pytest
import torch

import oracle
from golden_data import e2m1_table

TABLE = e2m1_table()


def _e2m1_by_rint(q: np.ndarray) -> np.ndarray:
    """Independent route: snap |q| to the E2M1 grid of its binade with rint, then look up the
    code of the snapped value in the OCP table."""
    a = np.abs(q.astype(np.float64))
    v = np.where(a < 2.0, np.rint(2.0 * a) / 2.0,
                 np.where(a < 4.0, np.rint(a), 2.0 * np.rint(a / 2.0)))
    v = np.minimum(v, 6.0)
    mag_codes = {TABLE[c]: c for c in range(8)}
    codes = np.zeros(q.shape, dtype=np.uint8)
    for value, c in mag_codes.items():
        codes[v == value] = c
    return codes | (np.signbit(q).astype(np.uint8) << 3)


def test_e2m1_exhaustive_where_decisions_are():
    # Every fp32 in [2^-3, 8): all E2M1 decision boundaries (0.25 .. 5) and the saturation
    # onset lie here; below 2^-3 everything is code 0 (checked by sampling below).
    lo = int(np.float32(0.125).view(np.uint32))
    top = int(np.float32(8.0).view(np.uint32))
    step = 1 << 24
    for start in range(lo, top, step):
        bits = np.arange(start, min(start + step, top), dtype=np.uint32)
        q = bits.view(np.float32)
        got = oracle.e2m1_round(q)
        want = _e2m1_by_rint(q)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"{bad.size} mismatches, first q={q[bad[0]]!r}"


def test_e2m1_small_values_round_to_zero():
    gen = np.random.default_rng(4)
    bits = gen.integers(0, int(np.float32(0.125).view(np.uint32)), 4_000_000, dtype=np.uint32)
    q = np.r_[bits.view(np.float32), np.float32([0.0, 1e-45, 0.1249999])]
    assert np.array_equal(oracle.e2m1_round(q), _e2m1_by_rint(q))
    assert (oracle.e2m1_round(q) == 0).all()


def test_e2m1_large_and_special():
    gen = np.random.default_rng(0)
    big = (gen.random(200_000) * 1e6).astype(np.float32) + np.float32(8.0)
    vals = np.r_[big, np.float32([8.0, 6.5, 7.0, 1e30, 3.4e38, np.inf])].astype(np.float32)
    assert (oracle.e2m1_round(vals) == 7).all()
    assert (oracle.e2m1_round(-vals) == 15).all()


def test_e2m1_sign_symmetry_and_negative_zero():
    gen = np.random.default_rng(1)
    q = (gen.standard_normal(1_000_000) * 3).astype(np.float32)
    assert np.array_equal(oracle.e2m1_round(-q), oracle.e2m1_round(q) ^ 8)
    assert oracle.e2m1_round(np.float32([-0.0, -0.1, -0.25]))[0] == 8
    assert (oracle.e2m1_round(np.float32([-0.1, -0.25])) == 8).all()
    assert oracle.e2m1_round(np.float32([0.0]))[0] == 0


def test_e2m1_midpoints_go_to_even_code():
    mids = np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert oracle.e2m1_round(mids).tolist() == [0, 2, 2, 4, 4, 6, 6]


def _torch_e4m3(t: np.ndarray) -> np.ndarray:
    return torch.from_numpy(t.astype(np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def _format_neighbourhood() -> np.ndarray:
    vals = np.array([oracle.e4m3_value(b) for b in range(0x7F)], dtype=np.float64)
    mids = (vals[:-1] + vals[1:]) / 2.0
    pts = np.r_[vals, mids, 448.0 + 8.0].astype(np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    down = np.nextafter(pts, np.float32(0.0))
    out = np.r_[pts, up, down].astype(np.float32)
    return out[(out >= 0) & (out < 464.0)]


def test_e4m3_against_torch_at_format_landmarks():
    t = _format_neighbourhood()
    got = oracle.e4m3_round(t)
    want = _torch_e4m3(t)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"first mismatch t={t[bad[0]]!r}: {got[bad[0]]:#x} vs {want[bad[0]]:#x}"


@pytest.mark.parametrize("dist", ["uniform", "log"])
def test_e4m3_against_torch_random(dist):
    gen = np.random.default_rng(2 if dist == "uniform" else 3)
    if dist == "uniform":
        t = (gen.random(4_000_000) * 464.0).astype(np.float32)
    else:
        t = np.exp(gen.uniform(np.log(1e-45), np.log(463.0), 4_000_000)).astype(np.float32)
    t = t[t < 464.0]
    got = oracle.e4m3_round(t)
    want = _torch_e4m3(t)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"first mismatch t={t[bad[0]]!r}: {got[bad[0]]:#x} vs {want[bad[0]]:#x}"


def test_e4m3_saturates_at_448():
    t = np.float32([448.0, 463.9, 464.0, 479.0, 480.0, 1e6, 3.4e38, np.inf])
    assert (oracle.e4m3_round(t) == 0x7E).all()
    assert (oracle.e4m3_round(-t) == 0xFE).all()


def test_e4m3_exhaustive_one_binade_and_subnormals():
    # Every fp32 in [1, 2) and every fp32 below 2^-6 that lies on a multiple of 2^-16.
    lo = int(np.float32(1.0).view(np.uint32))
    hi = int(np.float32(2.0).view(np.uint32))
    t = np.arange(lo, hi, dtype=np.uint32).view(np.float32)
    assert np.array_equal(oracle.e4m3_round(t), _torch_e4m3(t))
    sub = (np.arange(0, 1 << 10, dtype=np.float64) * 2.0 ** -16).astype(np.float32)
    assert np.array_equal(oracle.e4m3_round(sub), _torch_e4m3(sub))
