"""Pins of the oracle's interleaved RoPE (aclnnKvRmsNormRopeCache, Formulas (1)).

The oracle is checked against values worked by hand from the printed formula,
against the complex-rotation closed form, and against the exact (float64)
value of the expression rounded once to float32.
"""
import numpy as np
import pytest

import oracle
from gen import bf16_bits, bits_to_f32, rope_table_bf16, rng_for
from tests._util import golden


def test_rope_hand_worked():
    g = golden("rope_hand.json")
    for case in g["cases"]:
        y = oracle.rope(case["x"], case["cos"], case["sin"])
        np.testing.assert_array_equal(y, np.array(case["y"], dtype=np.float32), err_msg=case.get("note"))


def test_zero_angle_is_deinterleave_not_identity():
    rng = rng_for(11)
    x = bits_to_f32(bf16_bits(rng.standard_normal(64).astype(np.float32)))
    y = oracle.rope(x, np.ones(64), np.zeros(64))
    np.testing.assert_array_equal(y, np.concatenate([x[0::2], x[1::2]]))
    assert not np.array_equal(y, x)


def _random_rows(seed, n, d):
    rng = rng_for(seed)
    x = bits_to_f32(bf16_bits(rng.standard_normal((n, d)).astype(np.float32) * 3))
    pos = rng.integers(0, 32768, size=n)
    c, s = rope_table_bf16(pos, d)
    return x, bits_to_f32(c), bits_to_f32(s)


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_rope_equals_complex_rotation(d):
    """With duplicated-halves tables, (y[i] + j*y[h+i]) = (x[2i] + j*x[2i+1]) * (c_i + j*s_i)."""
    x, c, s = _random_rows(12 + d, 200, d)
    h = d // 2
    for r in range(x.shape[0]):
        y = oracle.rope(x[r], c[r], s[r]).astype(np.float64)
        z = (x[r, 0::2] + 1j * x[r, 1::2]).astype(np.complex128)
        w = (c[r, :h] + 1j * s[r, :h]).astype(np.complex128)
        ref = z * w
        a, b = np.abs(x[r, 0::2]), np.abs(x[r, 1::2])
        tol_re = 2.0 ** -23 * np.maximum(a * np.abs(c[r, :h]) + b * np.abs(s[r, :h]), 1e-30)
        tol_im = 2.0 ** -23 * np.maximum(b * np.abs(c[r, :h]) + a * np.abs(s[r, :h]), 1e-30)
        assert np.all(np.abs(y[:h] - ref.real) <= tol_re)
        assert np.all(np.abs(y[h:] - ref.imag) <= tol_im)


def test_rope_bf16_inputs_are_correctly_rounded():
    """bf16 x bf16 products are exact in float32, so each output is the exact
    value of x1*c - x2*s (resp. x2*c + x1*s) rounded once: compare bit for bit
    with that value computed exactly in float64 and rounded to float32."""
    d = 64
    x, c, s = _random_rows(13, 500, d)
    h = d // 2
    for r in range(x.shape[0]):
        y = oracle.rope(x[r], c[r], s[r])
        x1 = x[r, 0::2].astype(np.float64)
        x2 = x[r, 1::2].astype(np.float64)
        cc = c[r].astype(np.float64)
        ss = s[r].astype(np.float64)
        lo = x1 * cc[:h] - x2 * ss[:h]
        hi = x2 * cc[h:] + x1 * ss[h:]
        np.testing.assert_array_equal(y, np.concatenate([lo, hi]).astype(np.float32))


def test_rope_pair_norm_preserved():
    """y[i]^2 + y[h+i]^2 = (x[2i]^2 + x[2i+1]^2) (c_i^2 + s_i^2), within rounding."""
    d = 64
    x, c, s = _random_rows(14, 300, d)
    h = d // 2
    for r in range(x.shape[0]):
        y = oracle.rope(x[r], c[r], s[r]).astype(np.float64)
        lhs = y[:h] ** 2 + y[h:] ** 2
        rhs = (x[r, 0::2].astype(np.float64) ** 2 + x[r, 1::2].astype(np.float64) ** 2) * \
              (c[r, :h].astype(np.float64) ** 2 + s[r, :h].astype(np.float64) ** 2)
        np.testing.assert_allclose(lhs, rhs, rtol=2e-6, atol=1e-30)


def test_rope_quarter_turn_and_half_turn():
    rng = rng_for(15)
    x = bits_to_f32(bf16_bits(rng.standard_normal(16).astype(np.float32)))
    h = 8
    y = oracle.rope(x, np.zeros(16), np.ones(16))
    np.testing.assert_array_equal(y, np.concatenate([-x[1::2], x[0::2]]))
    y = oracle.rope(x, -np.ones(16), np.zeros(16))
    np.testing.assert_array_equal(y[:h], -x[0::2])
    np.testing.assert_array_equal(y[h:], -x[1::2])
