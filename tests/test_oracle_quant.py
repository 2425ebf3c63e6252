"""Pins of the oracle's per-row int8 quantisation (aclnnMlaPrologV3WeightNz,
Dequant Scale Query Nope formula: scale = RowMax(abs(y))/127,
code = round(y/scale); applied to the ckv cache row as in quantisation
scenario 1 of aclnnKvRmsNormRopeCache)."""
import numpy as np

import oracle
from gen import bf16_bits, bits_to_f32, rng_for
from tests._util import golden


def test_quant_hand_worked():
    for case in golden("quant_hand.json")["cases"]:
        code, scale = oracle.quant_row(case["y"])
        assert scale == np.float32(case["scale"]), case["note"]
        np.testing.assert_array_equal(code, np.array(case["codes"], dtype=np.int8), err_msg=case["note"])


def test_quant_bounds_float64():
    """Checked in float64: |code*scale - y| <= scale*(1/2 + 2^-16); |code| <= 127;
    the element of largest magnitude gets |code| = 127; the scale is the
    correctly rounded RowMax/127."""
    rng = rng_for(31)
    for _ in range(300):
        n = int(rng.integers(1, 700))
        y = (rng.standard_normal(n) * rng.uniform(1e-3, 1e3)).astype(np.float32)
        code, scale = oracle.quant_row(y)
        amax = np.max(np.abs(y.astype(np.float64)))
        assert scale == np.float32(np.float64(np.float32(amax)) / 127.0)
        s = float(scale)
        err = np.abs(code.astype(np.float64) * s - y.astype(np.float64))
        assert np.all(err <= s * (0.5 + 2.0 ** -16))
        assert np.all(np.abs(code.astype(np.int32)) <= 127)
        assert abs(int(code[np.argmax(np.abs(y))])) == 127


def test_quant_ties_to_even_through_the_division():
    """y/scale landing exactly on k + 1/2 rounds to the even neighbour."""
    y = np.array([127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5], dtype=np.float32)
    code, scale = oracle.quant_row(y)
    assert scale == 1.0
    np.testing.assert_array_equal(code, np.array([127, 0, 2, 2, 0, -2, -2, 126], dtype=np.int8))


def test_quant_end_to_end_token_int8_row():
    """The int8 row of a token is quant_row applied to the float32 RMSNorm
    output (no intermediate bf16 rounding)."""
    rng = rng_for(32)
    Dv, Dk = 512, 64
    kv = bf16_bits(rng.standard_normal((1, 1, 1, Dv + Dk)).astype(np.float32) * 2)
    gamma = bf16_bits(rng.uniform(0.5, 1.5, Dv).astype(np.float32))
    cs = bf16_bits(np.cos(np.arange(Dk) * 0.1).astype(np.float32)).reshape(1, 1, 1, Dk)
    sn = bf16_bits(np.sin(np.arange(Dk) * 0.1).astype(np.float32)).reshape(1, 1, 1, Dk)
    slot = np.array([3], dtype=np.int64)
    kc = np.zeros((2, 4, 1, Dk), dtype=np.uint16)
    ck = np.zeros((2, 4, 1, Dv), dtype=np.int8)
    sc = np.zeros((2, 4, 1), dtype=np.float32)
    oracle.paged_norm_rope_cache(kv, gamma, cs, sn, slot, kc, ck, sc, eps=1e-6)
    yn, yr = oracle.token_outputs(kv.reshape(-1), gamma, cs.reshape(-1), sn.reshape(-1), Dv, Dk, 1e-6)
    code, scale = oracle.quant_row(yn)
    np.testing.assert_array_equal(ck[0, 3, 0], code)
    assert sc[0, 3, 0] == scale
    np.testing.assert_array_equal(kc[0, 3, 0], oracle.f32_to_bf16(yr))
    # rows not addressed keep their bytes
    assert np.all(ck.reshape(8, Dv)[[0, 1, 2, 4, 5, 6, 7]] == 0)


def test_quant_end_to_end_exact_ties():
    """Rows built so that rms = 64 exactly (eps = 4096 - mean(x^2)), gamma = 1
    and max|x| = 127: then y = x/64, scale = 1/64 and y/scale = x, so the
    stored codes are rint(x) with ties to even (thousands of exact ties)."""
    rng = rng_for(950)
    Dv, Dk, T = 512, 64, 16
    base = np.zeros(Dv, np.float32)
    base[0] = 127.0
    base[1:181] = rng.choice(np.arange(-126.5, 127.0, 1.0, dtype=np.float32), 180, replace=False)
    ms = np.float32(float(np.sum(base.astype(np.float64) ** 2)) / Dv)
    eps = float(np.float32(4096.0) - ms)
    rows = np.stack([rng.permutation(base) for _ in range(T)])
    kv = np.concatenate([rows, np.zeros((T, Dk), np.float32)], axis=1)
    kvb = bf16_bits(kv).reshape(1, 1, T, Dv + Dk)
    gamma = bf16_bits(np.ones(Dv, np.float32))
    cs = np.zeros((1, 1, T, Dk), np.uint16)
    slots = np.arange(T, dtype=np.int64)
    kc = np.zeros((1, T, 1, Dk), np.uint16)
    ck = np.zeros((1, T, 1, Dv), np.int8)
    sc = np.zeros((1, T, 1), np.float32)
    oracle.paged_norm_rope_cache(kvb, gamma, cs, cs, slots, kc, ck, sc, eps=eps)
    np.testing.assert_array_equal(ck.reshape(T, Dv), np.rint(rows).astype(np.int8))
    assert np.all(sc == np.float32(1 / 64))


def test_quant_subnormal_scale_saturates():
    """RowMax/127 = 1.40 * 2^-149 rounds to the subnormal 2^-149, so y/scale
    reaches 178 for the row maximum: codes saturate at +-127 (the row maximum
    maps to the largest code); elements below 127 * scale keep rint(y/scale)."""
    u = np.float32(2.0 ** -149)
    code, scale = oracle.quant_row(np.array([178, 100, -150, 0, 3], np.float32) * u)
    assert scale == u
    np.testing.assert_array_equal(code, np.array([127, 100, -127, 0, 3], dtype=np.int8))
