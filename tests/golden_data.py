"""Readers for the cited fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def e2m1_table() -> np.ndarray:
    """float64[16]: value of each E2M1 code, from the OCP MX v1.0 table."""
    vals = np.full(16, np.nan)
    for code, value in _rows("e2m1_values.txt"):
        vals[int(code)] = float(value)
    assert not np.isnan(vals).any()
    return vals


def e4m3_landmarks() -> dict:
    return {int(b, 16): float(v) for b, v in _rows("e4m3_landmarks.txt")}


def bandwidth_model() -> dict:
    return {k: float(v) for k, v in _rows("bandwidth_model.txt")}
