"""The CPU oracle against facts fixed outside itself (no GPU needed)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.cider_oracle)


def test_linear_entry_points_compose_the_primitives():
    from w8a8_online_quantized_amd import inputs
    x = inputs.activations(8, 256)
    w = inputs.weights(16, 256)
    for gs in (0, 64, 128):
        wq, sw = oracle.quantize_weight(w, 8, gs)
        y, qa, sa = oracle.w8a8_linear(x, wq, sw, gs)
        q2, s2 = oracle.quantize_rows(x, gs, 127)
        assert np.array_equal(qa, q2)
        sw2 = sw[:, None] if gs == 0 else sw
        assert np.array_equal(y.view(np.uint16), pins._linear(oracle.cider_oracle, x, wq, sw2, gs).view(np.uint16))
    p, s4 = oracle.quantize_weight(w, 4, 0)
    y4, _, _ = oracle.w4a8_linear(x, p, s4)
    y8, _, _ = oracle.w8a8_linear(x, oracle.unpack_int4(p), s4, 0)
    assert np.array_equal(y4.view(np.uint16), y8.view(np.uint16))


def test_brute_rounding_routine_against_numpy_casts():
    """The brute force's own IEEE rounding agrees with numpy's fp32/fp16 casts
    on doubles, including ties, subnormals and overflow."""
    from fractions import Fraction
    from oracle import brute
    rng = np.random.default_rng(11)
    vals = list(rng.standard_normal(400) * np.exp2(rng.integers(-30, 20, 400)))
    vals += [65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
             1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -149, 1 + 2.0 ** -24]
    for v in vals:
        assert float(brute.f16(Fraction(v))) == float(np.float16(v)), v
        assert float(brute.f32(Fraction(v))) == float(np.float32(v)), v


def test_exactness_guard():
    """The fp64 integer dot product is exact only while 127*127*K < 2**53."""
    lim = oracle.cider_oracle._EXACT_K_LIMIT
    assert lim * 127 * 127 <= 2 ** 53 < (lim + 1) * 127 * 127
