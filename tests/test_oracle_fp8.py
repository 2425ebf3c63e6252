"""Pins of the oracle's FLOAT8 E4M3FN ckv quantisation (a ckv cache type of
aclnnKvRmsNormRopeCache, quantisation scenario 1; scale rule read by analogy
with the RowMax/127 rule of aclnnMlaPrologV3WeightNz as RowMax/448).

The code table is pinned by hand-worked values; encoding against an
independent float64 nearest-value search (ties to the even code) on every
representable value, every midpoint and its neighbours, and random values;
the row quantiser by hand-worked rows and float64 bounds."""
import numpy as np
import pytest

import gen
import oracle
from tests._util import golden


def table64():
    """All 127 finite non-negative E4M3FN values, computed from the format
    definition in float64 (independently of the oracle)."""
    vals = []
    for c in range(127):
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def nearest64(a):
    """Code of the nearest E4M3FN value to float64 a, ties to even, saturating."""
    t = table64()
    s = 0x80 if np.signbit(a) else 0
    a = abs(a)
    if a >= t[-1]:
        return s | 126
    d = np.abs(t - a)
    best = np.flatnonzero(d == d.min())
    c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
    return s | int(c)


def test_decode_hand_worked():
    g = golden("e4m3_hand.json")
    for d in g["decode"]:
        v = oracle.e4m3_decode(int(d["code"], 16))
        assert v == np.float32(d["value"]) and np.signbit(v) == np.signbit(d["value"]), d["note"]
    assert np.isnan(oracle.e4m3_decode(0x7F)) and np.isnan(oracle.e4m3_decode(0xFF))


def test_decode_matches_format_definition():
    t = table64()
    for c in range(127):
        assert oracle.e4m3_decode(c) == np.float32(t[c])
        assert oracle.e4m3_decode(0x80 | c) == -np.float32(t[c])


def test_encode_hand_worked():
    for e in golden("e4m3_hand.json")["encode"]:
        assert oracle.e4m3_encode(e["value"]) == int(e["code"], 16), e["note"]


def test_encode_values_midpoints_and_neighbours():
    t = table64()
    pts = list(t)
    for i in range(126):
        mid = (t[i] + t[i + 1]) / 2
        mid32 = np.float32(mid)
        assert mid32 == mid                      # midpoints are exact in float32
        pts += [mid, float(np.nextafter(mid32, np.float32(0))), float(np.nextafter(mid32, np.float32(1e9)))]
    pts = np.array(pts, dtype=np.float32)
    for v in np.concatenate([pts, -pts]):
        assert oracle.e4m3_encode(v) == nearest64(float(v)), v
    got = oracle.e4m3_encode_array(np.concatenate([pts, -pts]))
    want = np.array([nearest64(float(v)) for v in np.concatenate([pts, -pts])], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


def test_encode_random_values():
    rng = gen.rng_for(71)
    v = (rng.standard_normal(20000) * np.exp2(rng.uniform(-12, 9, 20000))).astype(np.float32)
    got = oracle.e4m3_encode_array(v)
    want = np.array([nearest64(float(x)) for x in v], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


def test_quant_row_fp8_hand_worked():
    code, scale = oracle.quant_row_fp8([448, 1, -1.0625, 0.5, 0])
    assert scale == 1.0
    np.testing.assert_array_equal(code, np.array([0x7E, 0x38, 0xB8, 0x30, 0x00], dtype=np.uint8))
    code, scale = oracle.quant_row_fp8([0, 0, 0])
    assert scale == 0 and np.all(code == 0)
    code, scale = oracle.quant_row_fp8([-896, 2, 3])
    assert scale == 2.0
    np.testing.assert_array_equal(code, np.array([0xFE, 0x38, 0x3C], dtype=np.uint8))


def test_quant_row_fp8_bounds_float64():
    """|decode(code) * scale - y| <= half the E4M3FN spacing at |y/scale| (plus
    the quotient's rounding), the largest magnitude maps to 448, and the scale
    is the correctly rounded RowMax / 448."""
    rng = gen.rng_for(72)
    t = table64()
    for _ in range(200):
        n = int(rng.integers(1, 600))
        y = (rng.standard_normal(n) * rng.uniform(1e-3, 1e3)).astype(np.float32)
        code, scale = oracle.quant_row_fp8(y)
        amax = float(np.max(np.abs(y)))
        assert scale == np.float32(amax / 448.0)
        s = float(scale)
        dec = np.array([oracle.e4m3_decode(c) for c in code], dtype=np.float64)
        q = np.abs(y.astype(np.float64) / s)
        idx = np.clip(np.searchsorted(t, q), 1, 126)
        spacing = t[idx] - t[idx - 1]
        assert np.all(np.abs(dec * s - y) <= s * (spacing / 2 + q * 2.0 ** -23) + 1e-45)
        assert abs(dec[np.argmax(np.abs(y))]) == 448.0


@pytest.mark.parametrize("mode", ["paged", "norm"])
def test_fp8_rows_end_to_end(mode):
    """The fp8 ckv row of a token is quant_row_fp8 of its float32 RMSNorm
    output; k rows and placement as for the other cache types."""
    if mode == "paged":
        case = gen.kvrc_paged_case(73, B=2, S=30, Dv=64, Dk=16, num_blocks=8, block_size=16,
                                   slot_kind="random", skip_frac=0.1, ckv_dtype="fp8")
        idx = case["slot_mapping"]
        rows_of = {t: int(v) for t, v in enumerate(idx) if v >= 0}
    else:
        case = gen.kvrc_norm_case(74, B=2, S=12, Dv=64, Dk=16, Bc=2, Sc=20, n_skip=2,
                                  ckv_dtype="fp8")
        rows_of = {b * 12 + s: b * 20 + int(case["index"][b, s]) for b in range(2)
                   for s in range(12) if case["index"][b, s] >= 0}
    got = oracle.run_kvrc_case(case)
    ck = got["ckv_cache"].reshape(-1, 64)
    sc = got["ckv_scale"].reshape(-1)
    kv = case["kv"].reshape(-1, 80)
    for t, r in rows_of.items():
        yn, _ = oracle.token_outputs(kv[t], case["gamma"], case["cos"].reshape(-1, 16)[t],
                                     case["sin"].reshape(-1, 16)[t], 64, 16, case["eps"])
        code, scale = oracle.quant_row_fp8(yn)
        np.testing.assert_array_equal(ck[r], code)
        assert sc[r] == scale
    untouched = np.setdiff1d(np.arange(ck.shape[0]), list(rows_of.values()))
    assert np.all(ck[untouched] == gen.FP8_SENTINEL) and np.all(sc[untouched] == gen.SCALE_SENTINEL)


def test_quant_row_fp8_subnormal_scale():
    """RowMax/448 = 1.43 * 2^-149 rounds to the subnormal 2^-149: y/scale is
    640 for the row maximum, which saturates to 448 (0x7e); 300 takes the
    nearest value 288 (0x79); a row maximum below 224 * 2^-149 gives scale 0
    and all-zero codes."""
    u = np.float32(2.0 ** -149)
    code, scale = oracle.quant_row_fp8(np.array([640, 300, -500, 0, -1], np.float32) * u)
    assert scale == u
    np.testing.assert_array_equal(code, np.array([0x7E, 0x79, 0xFE, 0x00, 0xB8], dtype=np.uint8))
    code, scale = oracle.quant_row_fp8(np.array([200, -3], np.float32) * u)
    assert scale == 0 and np.all(code == 0)
