"""The bf16 half-ulp used by the output bar, pinned to the bf16 format itself:
round-to-nearest-even into bf16 (8 significant bits, from the float32 bit
pattern) moves a value by at most the half-ulp, and that bound is reached."""
import numpy as np

import sas_inputs as si
from parity_bars import bf16_half_ulp, o_bound


def _spacing_above(x):
    """Distance from |x| (a bf16 value) to the next bf16 value above it."""
    bits = si.f32_to_bf16_bits(np.abs(x).astype(np.float32)).astype(np.uint32)
    nxt = si.bf16_bits_to_f32((bits + 1).astype(np.uint16))
    return nxt.astype(np.float64) - np.abs(x).astype(np.float64)


def test_half_ulp_is_half_the_bf16_spacing():
    g = np.random.default_rng(0)
    x = si.bf16_bits_to_f32(si.f32_to_bf16_bits(
        (g.standard_normal(20000) * np.exp2(g.integers(-20, 20, 20000))).astype(np.float32)))
    assert np.array_equal(bf16_half_ulp(x), _spacing_above(x) / 2)


def test_rounding_stays_within_half_ulp_and_reaches_it():
    g = np.random.default_rng(1)
    x = (g.standard_normal(200000) * 4).astype(np.float32)
    r = si.bf16_bits_to_f32(si.f32_to_bf16_bits(x)).astype(np.float64)
    err = np.abs(r - x.astype(np.float64))
    h = bf16_half_ulp(x)
    assert np.all(err <= h)
    assert np.max(err / h) > 0.999


def test_known_values_and_bar():
    assert bf16_half_ulp(1.0) == 2.0 ** -8
    assert bf16_half_ulp(1.999) == 2.0 ** -8
    assert bf16_half_ulp(2.0) == 2.0 ** -7
    assert bf16_half_ulp(-5.0) == 2.0 ** -6
    assert bf16_half_ulp(0.0) == 0.0
    # storage rounding alone passes 1e-2 only from |o| = 4 up
    assert bf16_half_ulp(3.99) < 1e-2 < bf16_half_ulp(4.0)
    assert o_bound(np.array([0.0, 1.5]), "bf16").tolist() == [1e-2, 1e-2 + 2.0 ** -8]
    assert o_bound(np.array([3.0]), "f32").tolist() == [1e-5]
