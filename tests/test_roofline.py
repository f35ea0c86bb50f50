"""The byte accounting and the bandwidth-model converter against the figures the page prints
("Qwen3.8-27B-NVFP4-RTX5090" model card, section "Why lm_head is NVFP4, and why MTP is gone"),
stored with their citation in tests/golden/bandwidth_model.txt."""
import pytest

from golden_data import bandwidth_model
from skinny_gemm_nvfp4_amd import inputs, roofline

P = bandwidth_model()
GIB = 2.0 ** 30


def test_lm_head_bytes_match_the_page():
    rows, cols = int(P["lm_head_rows"]), int(P["lm_head_cols"])
    nvfp4_gb = roofline.weight_bytes(cols, rows) / 1e9
    bf16_gb = rows * cols * 2 / 1e9
    assert round(nvfp4_gb, 2) == P["lm_head_nvfp4_gb"]      # 0.72 GB: 4.5 bits per weight
    assert round(bf16_gb, 2) == P["lm_head_bf16_gb"]        # 2.54 GB


def test_read_rate_is_about_92_percent_of_spec():
    rate = P["earlier_build_weight_stream_gib_per_token"] * GIB * P["earlier_build_decode_tok_s"]
    frac = rate / (P["rtx5090_spec_bandwidth_tb_s"] * 1e12)
    assert frac == pytest.approx(P["read_rate_fraction_of_spec_approx"], abs=0.005)


def test_bandwidth_model_reproduces_the_prediction():
    removed = (P["lm_head_bf16_gb"] - P["lm_head_nvfp4_gb"]) * 1e9
    pred = roofline.predicted_tok_s_after_removing(
        P["earlier_build_weight_stream_gib_per_token"] * GIB, P["earlier_build_decode_tok_s"],
        removed)
    assert round(pred, 1) == P["predicted_tok_s_with_nvfp4_lm_head"]
    # the page's measurement lands within 1.4% of the model
    assert abs(P["measured_tok_s_with_nvfp4_lm_head"] / pred - 1) < 0.014


def test_layer_and_full_pass_bytes():
    layer = sum(roofline.compulsory_bytes(1, N, K) for K, N in inputs.LAYER_SHAPES.values())
    assert layer == pytest.approx(186.07e6, rel=1e-3)
    weights = sum(roofline.weight_bytes(K, N) for _, K, N in inputs.full_pass_shapes())
    assert weights == pytest.approx(12.33e9, rel=1e-3)


def test_binding_roof():
    assert roofline.binding_roof(1, 34816, 5120) == "hbm"
    assert roofline.binding_roof(16, 34816, 5120) == "hbm"
    assert roofline.binding_roof(128, 34816, 5120) == "mfma"
