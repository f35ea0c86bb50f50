"""Pins of the oracle's element decoders against sources other than the oracle itself.

  * E2M1: the OCP MX v1.0 value table (tests/golden/e2m1_values.txt).
  * E4M3: torch's float8_e4m3fn (the OCP E4M3FN format) over all 256 bytes, and the OFP8
    landmarks (tests/golden/e4m3_landmarks.txt).
  * bf16 widening: torch's bfloat16 -> float64 over all 65536 bit patterns.
  * products: every (code, finite scale) product is exact in double, fp32 and bf16 (the property
    the HIP decode relies on).
"""
import numpy as np
import torch

import oracle
from golden_data import e2m1_table, e4m3_landmarks


def test_e2m1_matches_ocp_table():
    table = e2m1_table()
    for code in range(16):
        got = oracle.e2m1_value(code)
        assert got == table[code], (code, got, table[code])
        assert np.signbit(got) == np.signbit(table[code]), f"sign of zero, code {code}"


def test_e4m3_matches_torch_all_bytes():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    for b in range(256):
        got = oracle.e4m3_value(b)
        if np.isnan(ref[b]):
            assert np.isnan(got), b
        else:
            assert got == ref[b], (hex(b), got, ref[b])
            assert np.signbit(got) == np.signbit(ref[b]), hex(b)
    assert [b for b in range(256) if np.isnan(oracle.e4m3_value(b))] == [0x7F, 0xFF]


def test_e4m3_landmarks():
    for b, v in e4m3_landmarks().items():
        got = oracle.e4m3_value(b)
        if np.isnan(v):
            assert np.isnan(got)
        else:
            assert got == v and np.signbit(got) == np.signbit(v), (hex(b), got, v)


def test_bf16_widening_all_patterns():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_value(b) for b in range(0, 65536, 1)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_code_times_scale_exact_in_bf16():
    table = e2m1_table()
    for b in range(0x7F):
        s = oracle.e4m3_value(b)
        for code in range(16):
            p = table[code] * s
            assert float(np.float32(p)) == p
            as_bf16 = torch.tensor([p], dtype=torch.float64).to(torch.bfloat16).to(torch.float64)
            assert float(as_bf16[0]) == p, (code, hex(b))
