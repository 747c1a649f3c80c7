"""Pins of the float pass rule (tests/tolerance.py) at hand-evaluated values.

The rule is |D - ref| <= 2^-10 |alpha| absdot + 2^-8 |beta c| + ulp_out, with
ulp_out the spacing of the output format at max(|ref|, |D|): 2^(e - p + 1)
for e = max(floor(log2 m), e_min), p = 8 / 11 / 24 significant bits and
e_min = -126 / -14 / -126 for bf16 / fp16 / fp32. A slip in any of these
constants would loosen (or tighten) every float parity test, so each is
fixed here by a value worked out from the format definitions."""
import numpy as np
import pytest

from tests import tolerance


@pytest.mark.parametrize("m, dtype, want", [
    (1.0, "bf16", 2.0 ** -7),       # bf16: 8 significant bits, 1.0 has exponent 0
    (1.99, "bf16", 2.0 ** -7),      # still in [1, 2)
    (2.0, "bf16", 2.0 ** -6),       # next binade
    (3.0, "bf16", 2.0 ** -6),
    (0.75, "bf16", 2.0 ** -8),
    (1.0, "f16", 2.0 ** -10),       # fp16: 11 significant bits
    (65504.0, "f16", 32.0),         # fp16 max: exponent 15
    (2.0 ** -14, "f16", 2.0 ** -24),  # smallest fp16 normal
    (2.0 ** -20, "f16", 2.0 ** -24),  # fp16 subnormal: spacing stays 2^-24
    (1.0, "f32", 2.0 ** -23),       # fp32: 24 significant bits
    (1024.0, "f32", 2.0 ** -13),
    (2.0 ** -130, "bf16", 2.0 ** -133),  # bf16 subnormal: e clamps at -126
    (2.0 ** -140, "f32", 2.0 ** -149),   # fp32 subnormal spacing
    (0.0, "bf16", 2.0 ** -133),     # zero takes the subnormal spacing
    (0.0, "f16", 2.0 ** -24),
])
def test_ulp_out_hand_values(m, dtype, want):
    assert tolerance.ulp_out(m, dtype) == want


def test_ulp_out_matches_numpy_spacing_for_fp16_and_fp32():
    # numpy's spacing() is an independent definition of the same quantity for
    # the IEEE formats it has (for positive x it is the gap to the next float)
    g = np.random.default_rng(0)
    for dt, npdt in (("f16", np.float16), ("f32", np.float32)):
        x = np.abs(g.standard_normal(2000)) * np.float64(2.0) ** g.integers(-30, 12, 2000)
        x = x.astype(npdt)
        x = x[np.isfinite(x) & (x > 0)]
        want = np.spacing(x).astype(np.float64)
        got = tolerance.ulp_out(x.astype(np.float64), dt)
        assert np.array_equal(got, want), dt


def test_bound_terms_add_up():
    # ref 1.0, absdot 3.0, alpha -2, beta 0.5, c = 4, bf16 out:
    # 2^-10 * 2 * 3 + 2^-8 * |0.5 * 4| + ulp_bf16(1.0) = 6/1024 + 2/256 + 1/128
    b = tolerance.bound(np.array([1.0]), np.array([3.0]), np.array([1.0]), -2.0, 0.5, np.array([4.0]), "bf16")
    assert b[0] == 6 / 1024 + 2 / 256 + 1 / 128
    # beta = 0 drops the C term even when c is NaN
    b0 = tolerance.bound(np.array([1.0]), np.array([3.0]), np.array([1.0]), -2.0, 0.0, np.array([np.nan]), "bf16")
    assert b0[0] == 6 / 1024 + 1 / 128


def test_check_accepts_at_bound_and_rejects_beyond():
    ref = np.array([[1.0]])
    absdot = np.array([[0.0]])
    # exactly one bf16 ulp away passes; a bit more fails
    tolerance.check(ref + 2.0 ** -7, ref, absdot, 1.0, 0.0, None, "bf16")
    with pytest.raises(AssertionError):
        tolerance.check(ref + 2.0 ** -7 + 2.0 ** -20, ref, absdot, 1.0, 0.0, None, "bf16")
    # a NaN output never passes
    with pytest.raises(AssertionError):
        tolerance.check(np.array([[np.nan]]), ref, absdot, 1.0, 0.0, None, "f32")
