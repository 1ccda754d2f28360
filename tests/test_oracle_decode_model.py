"""The rebuilt two-term decode model reproduces every number the first page prints."""
import pytest

from oracle import decode_model as dm
from weight_only_quantized_w4a16_amd import synth

W = 7.50e9       # the page's W (rounded to the 7.50 B it prints)


def _model_values():
    return {
        "floor_bf16_ms": dm.step_bf16(W, 1) * 1e3,
        "floor_int4_g128_ms": dm.step_w4a16(W, 1) * 1e3,
        "floor_8bit_ms": dm.step_w8a8_fp8(W, 1) * 1e3,
        "slope_bf16_us": 2 * W / dm.H100_SXM.p_bf16 * 1e6,
        "slope_fp8_us": 2 * W / dm.H100_SXM.p_fp8 * 1e6,
        "dequant_tax_ms": dm.dequant_tax(W) * 1e3,
        "w4a16_own_ridge_B": dm.w4a16_own_ridge(),
        "m_star_B": dm.m_star(),
        "bf16_ridge_B": dm.bf16_ridge(),
        "w4a16_stops_paying_B": dm.w4a16_stops_paying(),
        "w4a16_vs_fp8_B": dm.w4a16_vs_fp8(),
        "step_bf16_B480_ms": dm.step_bf16(W, 480) * 1e3,
        "step_fp8_B480_ms": dm.step_w8a8_fp8(W, 480) * 1e3,
        "step_w4a16_B480_ms": dm.step_w4a16(W, 480) * 1e3,
    }


def test_reproduces_page_numbers(golden):
    g = golden("decode_model_h100.txt")
    vals = _model_values()
    assert set(g) == set(vals)
    for key, (want, tol) in g.items():
        assert abs(vals[key] - want) <= tol, (key, vals[key], want)


def test_regime_boundaries_are_where_the_curves_meet():
    b = dm.w4a16_stops_paying()
    assert dm.step_w4a16(W, b) == pytest.approx(dm.step_bf16(W, b), rel=1e-12)
    b = dm.w4a16_own_ridge()
    assert dm.step_w4a16(W, b) == pytest.approx(W * dm.B_INT4_G128 / dm.H100_SXM.beta, rel=1e-12)
    # W8A8 halves both terms: its speed-up over bf16 is batch invariant
    for B in (1, 64, 480, 1024):
        assert dm.step_bf16(W, B) / dm.step_w8a8_fp8(W, B) == pytest.approx(2.0)
    # the tax is constant in B above the ridge
    assert dm.step_w4a16(W, 1024) - dm.step_bf16(W, 1024) == pytest.approx(dm.dequant_tax(W))


def test_streamed_parameter_count(golden):
    g = golden("stack_params.txt")
    p = synth.stack_params("8b")
    assert abs(p / 1e9 - g["llama3_8b_streamed_params_B"][0]) <= g["llama3_8b_streamed_params_B"][1]
    assert abs(2 * p / 1e9 - g["llama3_8b_bf16_GB"][0]) <= g["llama3_8b_bf16_GB"][1]
