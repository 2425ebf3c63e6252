"""Pins of the MLA kv-path head oracle (aclnnMlaPrologV3WeightNz, the third
and fourth paths: c^KV = alpha_kv * RmsNorm(x W^DKV) into the ckv cache,
k^R = ROPE(x W^KR) into the k cache).

* float64 -> bf16 rounding: hand-worked ties, a double-rounding trap,
  subnormal ties, overflow (tests/golden/bf16_round_hand.json);
* the projection: exact rational sums on a small case;
* identity weights reduce the head to the fused norm-rope-cache of the
  aclnnKvRmsNormRopeCache page, whose float32 oracle is pinned separately;
* alpha: a power of two scales every output exactly;
* the RMS invariant of the normalised rows; RoPE special angles;
* scatter: -1 skips, untouched rows keep their bytes, bad slots rejected;
* the block-indexed placement: a hand-worked token -> row table, rejected
  entries, and the head equal to the per-token head on those rows;
* quantised ckv rows: the float64 E4M3FN rounding against the library's
  float32 conversion on every midpoint and its float32 neighbours, code
  decoding of all 256 codes, hand-worked int8 / fp8 rows, and the
  dequantisation error bound of the whole head.
"""
from fractions import Fraction

import numpy as np
import pytest

import gen
import oracle
from oracle import mla_kv_head as M
from tests._util import golden


def test_f64_to_bf16_hand_worked():
    for c in golden("bf16_round_hand.json")["cases"]:
        got = int(M.f64_to_bf16(np.array([float(c["value"])]))[0])
        assert got == int(c["bits"], 16), c["note"]
    assert int(M.f64_to_bf16(np.array([np.nan]))[0]) & 0x7FFF > 0x7F80
    assert int(M.f64_to_bf16(np.array([-0.0]))[0]) == 0x8000


def test_f64_to_bf16_matches_nearest_search():
    """Against a brute-force nearest search over all finite bf16 values of
    the same binade (ties: even fraction)."""
    rng = gen.rng_for(80)
    v = rng.standard_normal(3000) * np.exp2(rng.integers(-130, 120, 3000))
    allb = np.arange(0x8000, dtype=np.uint16)
    allv = M.bf16_to_f64(allb)
    fin = np.isfinite(allv)
    allb, allv = allb[fin], allv[fin]
    got = M.f64_to_bf16(v)
    for x, gb in zip(v, got):
        d = np.abs(allv - abs(x))
        best = allb[d == d.min()]
        b = best[0] if best.size == 1 else best[best % 2 == 0][0]
        assert int(gb) == (int(b) | (0x8000 if x < 0 else 0)), x


def test_projection_exact_small():
    """c[t, j] = sum_k x[t, k] w[j, k] as exact rationals; the float64
    product is within its summation bound 64 * 2^-53 * sum |x w|."""
    rng = gen.rng_for(81)
    x = gen.bf16_bits(rng.standard_normal((3, 64)).astype(np.float32))
    w = gen.bf16_bits(rng.standard_normal((576, 64)).astype(np.float32))
    c = M.kv_project(x, w)
    xf, wf = M.bf16_to_f64(x), M.bf16_to_f64(w)
    for t in range(3):
        for j in (0, 1, 17, 511, 512, 575):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xf[t], wf[j]))
            bound = 64 * 2.0 ** -53 * float(np.sum(np.abs(xf[t] * wf[j])))
            assert abs(float(exact) - c[t, j]) <= bound


def _identity_case(seed, T, alpha=1.0):
    """He = 576 with W = I: c equals the token's own 576 inputs."""
    case = gen.mla_kv_head_case(seed, B=1, S=T, He=576, num_blocks=4, block_size=64,
                                slot_kind="random", alpha=alpha)
    case["w"] = gen.bf16_bits(np.eye(576, dtype=np.float32))
    return case


def test_identity_weights_reduce_to_norm_rope_cache():
    """With W = I the head is the fused norm-rope-cache of the
    aclnnKvRmsNormRopeCache page on kv = x (alpha 1): the float64 head and
    the float32 fused oracle agree within one bf16 ulp everywhere and are
    equal almost everywhere (they differ only where float32 rounding error
    crosses a bf16 rounding boundary)."""
    T = 200
    case = _identity_case(82, T)
    got = M.run_mla_case(case)
    kc = np.full((4, 64, 1, 64), gen.BF16_SENTINEL, np.uint16)
    ck = np.full((4, 64, 1, 512), gen.BF16_SENTINEL, np.uint16)
    oracle.paged_norm_rope_cache(case["x"].reshape(1, 1, T, 576), case["gamma"],
                                 case["cos"].reshape(1, 1, T, 64), case["sin"].reshape(1, 1, T, 64),
                                 case["slot_mapping"], kc, ck, eps=case["eps"])
    from tests._util import bf16_ulp_diff
    for a, b in ((got["ckv_cache"], ck), (got["k_cache"], kc)):
        d = bf16_ulp_diff(a.reshape(-1), b.reshape(-1))
        assert d.max() <= 1 and np.mean(d == 0) > 0.99
    # RoPE of exact inputs with per-element exact products: bit-equal
    np.testing.assert_array_equal(got["k_cache"], kc)


def test_alpha_power_of_two_is_exact():
    T = 64
    a1 = M.run_mla_case(_identity_case(83, T, alpha=1.0))
    a2 = M.run_mla_case(_identity_case(83, T, alpha=2.0))
    y1 = M.bf16_to_f64(a1["ckv_cache"])
    y2 = M.bf16_to_f64(a2["ckv_cache"])
    written = y1 != 7.0
    np.testing.assert_array_equal(y2[written], 2 * y1[written])
    np.testing.assert_array_equal(a1["k_cache"], a2["k_cache"])


def test_rms_invariant_and_rope_angles():
    rng = gen.rng_for(84)
    case = gen.mla_kv_head_case(85, B=2, S=8, He=256, num_blocks=4, block_size=16,
                                alpha=0.75)
    y, kr = M.kv_head_rows(case["x"], case["w"], case["gamma"], case["alpha"], case["cos"],
                           case["sin"], case["eps"])
    c = M.kv_project(case["x"], case["w"])
    ms = np.mean(c[:, :512] ** 2, axis=1)
    g = M.bf16_to_f64(case["gamma"])
    lhs = np.sqrt(np.mean((y / (0.75 * g)) ** 2, axis=1))
    np.testing.assert_allclose(lhs, np.sqrt(ms / (ms + case["eps"])), rtol=1e-12)
    # zero angle: kr is the de-interleaved rope input; quarter turn: (-x2, x1)
    one = np.full((16, 64), 0x3F80, np.uint16)
    zero = np.zeros((16, 64), np.uint16)
    _, k0 = M.kv_head_rows(case["x"], case["w"], case["gamma"], 1.0, one, zero, case["eps"])
    _, k1 = M.kv_head_rows(case["x"], case["w"], case["gamma"], 1.0, zero, one, case["eps"])
    r = c[:, 512:]
    np.testing.assert_array_equal(k0, np.concatenate([r[:, 0::2], r[:, 1::2]], axis=1))
    np.testing.assert_array_equal(k1, np.concatenate([-r[:, 1::2], r[:, 0::2]], axis=1))
    # pair norms are preserved by any angle
    p_in = r[:, 0::2] ** 2 + r[:, 1::2] ** 2
    p_out = kr[:, :32] ** 2 + kr[:, 32:] ** 2
    np.testing.assert_allclose(p_out, p_in, rtol=1e-2)          # bf16 cos/sin: |c^2+s^2-1| < 1e-2


def test_scatter_skips_and_untouched_rows():
    case = gen.mla_kv_head_case(86, B=2, S=30, He=128, num_blocks=8, block_size=16,
                                slot_kind="random", skip_frac=0.2)
    got = M.run_mla_case(case)
    v = case["slot_mapping"]
    y, kr = M.kv_head_rows(case["x"], case["w"], case["gamma"], case["alpha"], case["cos"],
                           case["sin"], case["eps"])
    ck, kc = got["ckv_cache"].reshape(-1, 512), got["k_cache"].reshape(-1, 64)
    for t, s in enumerate(v):
        if s >= 0:
            np.testing.assert_array_equal(ck[s], M.f64_to_bf16(y[t]))
            np.testing.assert_array_equal(kc[s], M.f64_to_bf16(kr[t]))
    untouched = np.setdiff1d(np.arange(ck.shape[0]), v[v >= 0])
    assert np.all(ck[untouched] == gen.BF16_SENTINEL) and np.all(kc[untouched] == gen.BF16_SENTINEL)
    bad = dict(case, slot_mapping=v.copy())
    bad["slot_mapping"][3] = bad["slot_mapping"][5] = 7
    with pytest.raises(M.MlaOracleError, match="duplicate"):
        M.run_mla_case(bad)
    bad["slot_mapping"] = v.copy()
    bad["slot_mapping"][0] = 8 * 16
    with pytest.raises(M.MlaOracleError, match="range"):
        M.run_mla_case(bad)


def test_block_index_slots_hand_worked():
    """B = 2 sequences of S = 5 tokens, chunks of 2 (3 per sequence):
    entries 4 (block 2), 7 (block 3, offset ignored), -1; 0 (block 0),
    11 (block 5), 2 (block 1). Worked by hand: token (b, s) -> row
    (entry // 2) * 2 + s % 2."""
    entries = np.array([4, 7, -1, 0, 11, 2], dtype=np.int64)
    got = M.block_index_slots(entries, 2, 5, 2, rows=16)
    np.testing.assert_array_equal(got, [4, 5, 6, 7, -1, 0, 1, 10, 11, 2])
    with pytest.raises(M.MlaOracleError, match="twice"):
        M.block_index_slots(np.array([4, 5, -1, 0, 11, 2]), 2, 5, 2, rows=16)   # block 2 twice
    with pytest.raises(M.MlaOracleError, match="range"):
        M.block_index_slots(np.array([4, 7, -1, 0, 16, 2]), 2, 5, 2, rows=16)
    with pytest.raises(M.MlaOracleError, match="entries"):
        M.block_index_slots(np.array([4, 7, -1, 0, 11]), 2, 5, 2, rows=16)


def test_block_indexed_head_equals_per_token_head():
    case = gen.mla_kv_head_blk_case(87, B=3, S=37, He=64, num_blocks=16, block_size=8,
                                    n_skip=2, entry_offsets=True)
    got = M.run_mla_case(case)
    slots = M.block_index_slots(case["block_index"], 3, 37, 8, rows=16 * 8)
    per_token = dict(case, mode="mla_paged", slot_mapping=slots)
    want = M.run_mla_case(per_token)
    for name in ("ckv_cache", "k_cache"):
        np.testing.assert_array_equal(got[name], want[name])
    # the skipped tokens are exactly those of the two -1 chunks (8 tokens, or
    # 5 for the last chunk of a sequence: 37 = 4 * 8 + 5)
    sizes = [8, 8, 8, 8, 5] * 3
    skipped = sum(sz for e, sz in zip(case["block_index"], sizes) if e < 0)
    assert np.count_nonzero(slots == -1) == skipped


def _torch_e4m3(v):
    import torch
    t = torch.tensor(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy(), t.view(torch.uint8).numpy()


def test_e4m3_decode_all_codes_match_library():
    """Every E4M3FN code decodes to the library's value of that code (NaN
    codes to NaN), and re-encodes to itself."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.tensor(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = M.e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(lib))
    ok = ~np.isnan(lib)
    np.testing.assert_array_equal(got[ok], lib[ok])
    assert np.sum(~ok) == 2 and set(codes[~ok]) == {0x7F, 0xFF}
    np.testing.assert_array_equal(M.e4m3_encode(M.e4m3_round(got[ok])), codes[ok])


def test_e4m3_round_matches_library_on_midpoints_and_random():
    """The float64 rounding against the library's float32 -> E4M3FN
    conversion (nearest, ties to even, saturating) on every midpoint between
    neighbouring values, the midpoints +- one float32 ulp, and random
    values over the whole range. All these inputs are float32 values, so the
    library sees the same numbers."""
    vals = M.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))          # 0 .. 448 ascending
    mids = (vals[:-1] + vals[1:]) / 2
    mids32 = mids.astype(np.float32)
    assert np.all(mids32 == mids)
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(0))
    rng = np.random.default_rng(5)
    rnd = (rng.uniform(-1, 1, 20000) * 2.0 ** rng.uniform(-12, np.log2(460), 20000)).astype(np.float32)
    v = np.concatenate([mids32, up, dn, -mids32, -up, vals.astype(np.float32), rnd,
                        np.float32([448, 460, 463.9, -463.9, 0.0, -0.0])])
    want, want_codes = _torch_e4m3(v)
    got = M.e4m3_round(v.astype(np.float64))
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(M.e4m3_encode(got), want_codes)
    # ties go to the even code: 17 -> 16, 19 -> 20, 2^-9 * 1.5 -> 2^-9 * 2
    np.testing.assert_array_equal(M.e4m3_round(np.array([17.0, 19.0, 1.5 * 2.0 ** -9])),
                                  [16.0, 20.0, 2.0 ** -8])


def test_quantize_rows_hand_worked():
    """int8: row max 254 -> scale 2; 63.5 / 2 = 31.75 -> 32, -127 / 2 = -63.5
    -> -64 (tie to even), 0.25 / 2 -> 0. fp8: row max 896 -> scale 2;
    34 / 2 = 17 -> 16 (tie to even), -36 / 2 = -18 exact, 1/256 / 2 = 2^-9
    (the smallest subnormal); codes 0x7E = (15, 6), 0x58 = (11, 0),
    0xD9 = sign + (11, 1), 0x01 = subnormal 1 (exponent field, mantissa). A zero row: scale 0, codes 0."""
    y = np.zeros((2, 512))
    y[0, :4] = [254.0, -127.0, 63.5, 0.25]
    q, s = M.quantize_rows(y, "int8")
    np.testing.assert_array_equal(s, [2.0, 0.0])
    np.testing.assert_array_equal(q[0, :4], [127, -64, 32, 0])
    assert not np.any(q[0, 4:]) and not np.any(q[1])
    y = np.zeros((2, 512))
    y[0, :4] = [896.0, 34.0, -36.0, 1 / 256]
    q, s = M.quantize_rows(y, "fp8")
    np.testing.assert_array_equal(s, [2.0, 0.0])
    np.testing.assert_array_equal(q[0, :4], [448.0, 16.0, -18.0, 2.0 ** -9])
    np.testing.assert_array_equal(M.e4m3_encode(q[0, :4]), [0x7E, 0x58, 0xD9, 0x01])


@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_quantised_head_scatter_and_error_bound(kind):
    """The quantised head writes, at each kept token's row, codes whose
    dequantised values lie within half a code step of y (a step of the
    scale for int8; for E4M3FN, relative 2^-4 of the value, or 2^-10 times
    the scale below the normal range), a code of magnitude 127 (448) at the
    row maximum, and the float32 of RowMax/127 (/448) as the scale; the k
    cache is the bf16 path's; untouched rows keep their sentinels."""
    case = gen.mla_kv_head_case(88, B=2, S=40, He=96, num_blocks=8, block_size=16,
                                slot_kind="random", skip_frac=0.2, ckv_dtype=kind)
    got = M.run_mla_case(case)
    ref = M.run_mla_case(gen.mla_kv_head_case(88, B=2, S=40, He=96, num_blocks=8, block_size=16,
                                              slot_kind="random", skip_frac=0.2))
    np.testing.assert_array_equal(got["k_cache"], ref["k_cache"])
    y, _ = M.kv_head_rows(case["x"], case["w"], case["gamma"], case["alpha"], case["cos"],
                          case["sin"], case["eps"])
    v = case["slot_mapping"]
    ck = got["ckv_cache"].reshape(-1, 512)
    sc = got["ckv_scale"].reshape(-1)
    div = 127.0 if kind == "int8" else 448.0
    for t, s in enumerate(v):
        if s < 0:
            continue
        amax = np.max(np.abs(y[t]))
        assert sc[s] == np.float32(amax / div)
        deq = (ck[s].astype(np.float64) if kind == "int8" else M.e4m3_decode(ck[s])) * (amax / div)
        err = np.abs(deq - y[t])
        if kind == "int8":
            assert np.all(err <= 0.5 * amax / div * (1 + 1e-12))
        else:
            bound = np.maximum(np.abs(y[t]) * 2.0 ** -4, 2.0 ** -10 * amax / div)
            assert np.all(err <= bound * (1 + 1e-12))
        code = ck[s][int(np.argmax(np.abs(y[t])))]
        assert abs(float(code) if kind == "int8" else M.e4m3_decode(code)) == div
    untouched = np.setdiff1d(np.arange(ck.shape[0]), v[v >= 0])
    sent = gen.INT8_SENTINEL if kind == "int8" else gen.FP8_SENTINEL
    assert np.all(ck[untouched] == sent) and np.all(sc[untouched] == gen.SCALE_SENTINEL)


def test_quantised_zero_rows_store_zero_scale_and_code_0x00():
    """alpha = 0 makes every row zero (zeros of both signs, the signs of
    the projection): scale 0 and code byte 0 everywhere, the rule of the
    norm-rope-cache operator's zero rows."""
    for kind in ("int8", "fp8"):
        case = gen.mla_kv_head_case(89, B=1, S=20, He=64, num_blocks=4, block_size=8,
                                    alpha=0.0, ckv_dtype=kind)
        y, _ = M.kv_head_rows(case["x"], case["w"], case["gamma"], case["alpha"], case["cos"],
                              case["sin"], case["eps"])
        assert not np.any(y) and np.any(np.signbit(y))
        got = M.run_mla_case(case)
        rows = case["slot_mapping"]
        assert np.all(got["ckv_cache"].reshape(-1, 512)[rows].view(np.uint8) == 0)
        assert np.all(got["ckv_scale"].reshape(-1)[rows] == 0.0)
