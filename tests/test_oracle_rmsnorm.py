"""Pins of the oracle's RMSNorm (aclnnKvRmsNormRopeCache, Formulas (2) rmsNorm;
aclnnMlaPrologV3WeightNz, RmsNorm formula).

Hand-worked float32 cases, the canonical summation order, a float64 library
routine (torch.nn.functional.rms_norm) and the invariant
sqrt(mean((y/gamma)^2)) = sqrt(ms / (ms + eps)).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gen import bf16_bits, bits_to_f32, rng_for
from tests._util import f32_bits, f32_from_hex, golden


def test_rmsnorm_hand_worked():
    g = golden("rmsnorm_hand.json")
    for case in g["cases"]:
        y = oracle.rmsnorm(case["x"], case["gamma"], case["eps"])
        if "y_bits" in case:
            np.testing.assert_array_equal(f32_bits(y), f32_bits(f32_from_hex(case["y_bits"])),
                                          err_msg=case["note"])
        else:
            np.testing.assert_array_equal(y, np.array(case["y"], dtype=np.float32),
                                          err_msg=case["note"])


def test_sumsq_canonical_order():
    s = golden("rmsnorm_hand.json")["sumsq_order"]
    x = np.zeros(s["n"], dtype=np.float32)
    for k, v in s["x_nonzero"].items():
        x[int(k)] = v
    got = oracle.sumsq(x)
    assert f32_bits(np.float32(got)) == int(s["sumsq_bits"], 16), s["note"]


def test_sumsq_within_pairwise_bound():
    """|S_pairwise - S_exact| <= (chunk terms + 6 levels) * u * S for nonnegative terms."""
    rng = rng_for(21)
    for n in [1, 7, 8, 9, 64, 511, 512, 513, 1000, 4096]:
        x = rng.standard_normal(n).astype(np.float32)
        got = float(oracle.sumsq(x))
        exact = float(np.sum(x.astype(np.float64) ** 2))
        per_lane_terms = 8 * math.ceil(math.ceil(n / 8) / 64)
        bound = (per_lane_terms + 6 + 1) * 2.0 ** -24 * exact
        assert abs(got - exact) <= bound, (n, got, exact)


@pytest.mark.parametrize("n", [8, 64, 128, 512, 576, 1024])
def test_rmsnorm_vs_torch_float64(n):
    rng = rng_for(22 + n)
    for eps in [1e-6, 0.0, 1e-2]:
        x = bits_to_f32(bf16_bits(rng.standard_normal((20, n)).astype(np.float32) * 2))
        gm = bits_to_f32(bf16_bits(rng.uniform(0.5, 1.5, n).astype(np.float32)))
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (n,),
                                           weight=torch.from_numpy(gm.astype(np.float64)),
                                           eps=eps).numpy()
        for r in range(x.shape[0]):
            y = oracle.rmsnorm(x[r], gm, eps).astype(np.float64)
            # error budget: sum of squares (<= ~16u relative), sqrt, divide, multiply
            tol = 24 * 2.0 ** -24 * np.abs(ref[r]) + 1e-30
            assert np.all(np.abs(y - ref[r]) <= tol), (n, eps, r)


def test_rmsnorm_invariant():
    rng = rng_for(23)
    n = 512
    for eps in [1e-6, 1e-3]:
        for _ in range(50):
            x = bits_to_f32(bf16_bits(rng.standard_normal(n).astype(np.float32)))
            gm = bits_to_f32(bf16_bits(rng.uniform(0.5, 1.5, n).astype(np.float32)))
            y = oracle.rmsnorm(x, gm, eps).astype(np.float64)
            ms = np.mean(x.astype(np.float64) ** 2)
            lhs = math.sqrt(np.mean((y / gm) ** 2))
            rhs = math.sqrt(ms / (ms + eps))
            assert abs(lhs - rhs) <= 32 * 2.0 ** -24, (lhs, rhs)


def test_rmsnorm_gamma_is_elementwise():
    """Scaling gamma[i] by 2 scales y[i] alone by exactly 2."""
    rng = rng_for(24)
    x = bits_to_f32(bf16_bits(rng.standard_normal(64).astype(np.float32)))
    gm = np.ones(64, dtype=np.float32)
    y1 = oracle.rmsnorm(x, gm, 1e-6)
    gm[5] = 2
    y2 = oracle.rmsnorm(x, gm, 1e-6)
    assert y2[5] == 2 * y1[5]
    np.testing.assert_array_equal(np.delete(y1, 5), np.delete(y2, 5))


def test_rmsnorm_without_weight_and_zero_row():
    x = np.array([3, 4, 0, 0], dtype=np.float32)
    np.testing.assert_array_equal(oracle.rmsnorm(x, None, 0.0), oracle.rmsnorm(x, np.ones(4), 0.0))
    z = oracle.rmsnorm(np.zeros(8), np.ones(8), 1e-6)
    np.testing.assert_array_equal(z, np.zeros(8, dtype=np.float32))


def test_bf16_rounding_pins():
    """float32 -> bf16: nearest, ties to even; NaN stays NaN."""
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5,
                     65504.0, 3.0e38, np.inf, -np.inf], dtype=np.float32)
    want = np.array([0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x4780, 0x7F62, 0x7F80, 0xFF80],
                    dtype=np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_bf16(vals), want)
    nanb = oracle.f32_to_bf16(np.array([np.nan], dtype=np.float32))[0]
    assert (nanb & 0x7F80) == 0x7F80 and (nanb & 0x7F) != 0
    rng = rng_for(25)
    a = rng.standard_normal(10000).astype(np.float32) * 100
    b = oracle.f32_to_bf16(a)
    back = oracle.bf16_to_f32(b).astype(np.float64)
    # nearest: no other bf16 value is closer (check the two neighbours)
    up = oracle.bf16_to_f32((b.astype(np.int32) + 1).astype(np.uint16)).astype(np.float64)
    dn = oracle.bf16_to_f32((b.astype(np.int32) - 1).astype(np.uint16)).astype(np.float64)
    err = np.abs(back - a)
    assert np.all(err <= np.abs(up - a)) and np.all(err <= np.abs(dn - a))
