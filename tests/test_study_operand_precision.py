"""The operand-precision study (tests/study_operand_precision.py): its format
emulations pinned to closed forms, and the conclusions the kernel design rests
on, asserted on the study's numbers."""
import numpy as np
import pytest

import study_operand_precision as sp

TOL = 2e-3  # the attention tolerance the kernels are held to


def test_bf16_rounding_closed_forms():
    x = np.array([1.0, 1 + 2.0**-8, 1 + 3 * 2.0**-8, 1 + 2.0**-7, -(1 + 2.0**-8 + 2.0**-20)],
                 np.float32)
    assert list(sp.bf16_rne(x)) == [1.0, 1.0, 1 + 2.0**-6, 1 + 2.0**-7, -(1 + 2.0**-7)]
    assert list(sp.bf16_trunc(x)) == [1.0, 1.0, 1 + 2.0**-7, 1 + 2.0**-7, -1.0]


def test_binary16_toward_zero_closed_forms():
    x = np.array([1.0, 1 + 2.0**-11, 1 + 1.9 * 2.0**-10, 65504.0, 2.0**-24 * 1.5, 0.0])
    assert list(sp.f16_rtz(x)) == [1.0, 1.0, 1 + 2.0**-10, 65504.0, 2.0**-24, 0.0]
    assert list(sp.f16_rne(np.array([1 + 2.0**-11, 1 + 3 * 2.0**-11]))) == [1.0, 1 + 2.0**-9]


def test_e4m3_closed_forms():
    x = np.array([1.0, 1.0625, 1.1875, 448.0, 500.0, 2.0**-9, 1.5 * 2.0**-9, 2.0**-11, -3.3,
                  0.0])
    # ties to even on the 1/8 mantissa step; subnormal step 2^-9; saturation at 448
    expect = [1.0, 1.0, 1.25, 448.0, 448.0, 2.0**-9, 2 * 2.0**-9, 0.0, -3.25, 0.0]
    assert list(sp.e4m3(x)) == expect
    # every finite e4m3 value is a fixed point of the rounding
    vals = [m / 8 * 2.0**-6 for m in range(8)]
    vals += [(1 + m / 8) * 2.0**e for e in range(-6, 9) for m in range(8)]
    vals = np.array([v for v in vals if v <= 448.0])
    assert np.array_equal(sp.e4m3(vals), vals) and np.array_equal(sp.e4m3(-vals), -vals)


def test_fixed_point_step():
    v = np.array([[-3.0, 1.5, 0.75, 3.0]])
    # 3 bits: step 3 / (2^2 - 1) = 1; 1.5 ties to even (2), 0.75 rounds to 1
    assert np.array_equal(sp.fixed(v, 3), np.array([[-3.0, 2.0, 1.0, 3.0]]))
    # 16 bits: within half a step of 3/32767; the row maximum is exact
    f16b = sp.fixed(v, 16)
    assert np.abs(f16b - v).max() <= 3.0 / 32767 / 2 and f16b[0, 3] == 3.0 and f16b[0, 0] == -3.0


@pytest.fixture(scope="module")
def results():
    return sp.run_study()


def test_kernel_formats_sit_well_inside_the_tolerance(results):
    for name, r in results.items():
        assert r["qk"]["kernel"] <= TOL / 6, name
        assert r["pv"]["kernel"] == r["qk"]["kernel"], name


def test_single_bf16_keys_are_not_enough(results):
    """One bf16 part for k_hat costs 5-26x the error of the hi/lo split and exceeds
    the tolerance on RoPE'd VAR data: hence two bf16 MFMAs per k-step."""
    for name, r in results.items():
        assert r["qk"]["bf16"] >= 5 * r["qk"]["kernel"], name
    assert results["var_d20_int3_rope"]["qk"]["bf16"] > TOL


def test_single_mfma_alternatives_lose_their_margin(results):
    """binary16 k_hat, or binary16 code*s with the zero as a bias, come within 2x of
    the tolerance on RoPE'd VAR data, against 8x for the hi/lo split."""
    r = results["var_d20_int3_rope"]["qk"]
    assert r["f16"] > 4 * r["kernel"] and r["f16"] > TOL / 2
    assert r["f16_cs_bias"] > TOL / 2


def test_folding_the_scale_into_the_query(results):
    """q (.) s in 24-bit fixed point against integer codes matches the kernel;
    16 bits adds up to 2.1x the kernel's error (RoPE data)."""
    for name, r in results.items():
        assert abs(r["qk"]["fix24"] - r["qk"]["kernel"]) <= 0.02 * r["qk"]["kernel"], name
        assert r["qk"]["fix16"] >= r["qk"]["kernel"] * 0.999, name
    assert results["video_int4_rope"]["qk"]["fix16"] > 1.5 * results["video_int4_rope"]["qk"]["kernel"]


def test_bf16_weights_and_values_use_the_whole_tolerance(results):
    for name, r in results.items():
        assert r["pv"]["bf16_pv"] >= 4 * r["pv"]["kernel"], name
        assert r["pv"]["bf16_pv"] > TOL / 2, name


def test_fp8_operands_are_an_order_too_coarse(results):
    for name, r in results.items():
        assert r["qk"]["e4m3_kq"] > 10 * TOL, name
        assert r["pv"]["e4m3_pv"] > 5 * TOL, name
        assert r["pv"]["e4m3_all"] > 10 * TOL, name
