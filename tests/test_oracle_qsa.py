"""Pins of the oracle's QSAPrepare (openvino.opset17.qsa_prepare: one key per
complete block = mean of key_block_size raw keys, RMS-normalised with
k_norm_weight and rotated with the RoPE of the block's first token; only
blocks completed by the new tokens are computed; state carried in
past_incomplete_raw_keys / past_incomplete_rope / key_length).
"""
import math

import numpy as np
import pytest

import gen
import oracle
from gen import bf16_bits, bits_to_f32, rng_for
from tests._util import golden


def _arr(x, dtype):
    return None if x is None else np.ascontiguousarray(np.array(x, dtype=np.float64)).astype(dtype)


def test_qsa_hand_worked():
    for case in golden("qsa_hand.json")["cases"]:
        N, L, Di, Dr, kbs = case["N"], case["L"], case["Di"], case["Dr"], case["kbs"]
        raw = bf16_bits(_arr(case["raw"], np.float32))
        w = case["k_norm_weight"]
        w = None if w is None else bf16_bits(_arr(w, np.float32))
        rc = _arr(case["rope_cos"], np.float32)
        rs = _arr(case["rope_sin"], np.float32)
        praw = bf16_bits(_arr(case["past_raw"], np.float32))
        prope = _arr(case["past_rope"], np.float32)
        bk = np.full((N, case["Bcap"], Di), gen.BF16_SENTINEL, dtype=np.uint16)
        nraw = np.full((N, kbs - 1, Di), gen.BF16_SENTINEL, dtype=np.uint16)
        nrope = None if rc is None else np.full((N, 2 * Dr), -5.0, dtype=np.float32)
        kl = np.array(case["key_length"], dtype=np.int64)
        oracle.qsa_prepare(raw, bk, kl, rc, rs, w, praw, prope, nraw, nrope,
                           key_block_size=kbs, eps=case["eps"])
        np.testing.assert_array_equal(bits_to_f32(bk), _arr(case["block_keys"], np.float32),
                                      err_msg=case["name"])
        k = case["next_raw_rows"]
        if k:
            np.testing.assert_array_equal(bits_to_f32(nraw[:, :k]), _arr(case["next_raw"], np.float32))
            np.testing.assert_array_equal(nrope, _arr(case["next_rope"], np.float32))
        assert np.all(nraw[:, k:] == gen.BF16_SENTINEL)


def test_block_mean_within_summation_bound():
    """float32 sum of kbs values in order: |m - m_exact| <= (kbs-1) u sum|x| / kbs."""
    rng = rng_for(51)
    for kbs in [2, 3, 16, 64, 128]:
        rows = bf16_bits(rng.standard_normal((kbs, 32)).astype(np.float32))
        m, _ = oracle.qsa_block_key(rows)
        x = bits_to_f32(rows).astype(np.float64)
        exact = x.mean(axis=0)
        bound = (kbs - 1) * 2.0 ** -24 * np.abs(x).sum(axis=0) / kbs + 2.0 ** -24 * np.abs(exact)
        assert np.all(np.abs(m - exact) <= bound)


def test_constant_block_reduces_to_single_token_formula():
    """kbs copies of one bf16 row: the float32 mean is that row exactly, so the
    block key is rmsnorm + rope of the row."""
    rng = rng_for(52)
    Di, Dr, kbs = 128, 64, 64
    v = bf16_bits(rng.standard_normal(Di).astype(np.float32))
    rows = np.tile(v, (kbs, 1))
    w = bits_to_f32(bf16_bits(rng.uniform(0.5, 1.5, Di).astype(np.float32)))
    c, s = gen.rope_table_f32(np.array(777), Dr)
    m, z = oracle.qsa_block_key(rows, w, c, s, 1e-6)
    np.testing.assert_array_equal(m, bits_to_f32(v))
    y = oracle.rmsnorm(bits_to_f32(v), w, 1e-6)
    y[Di - Dr:] = oracle.rope(y[Di - Dr:], c, s)
    np.testing.assert_array_equal(z, y)


def test_rotation_acts_on_trailing_dims_only():
    rng = rng_for(53)
    Di, Dr, kbs = 64, 16, 4
    rows = bf16_bits(rng.standard_normal((kbs, Di)).astype(np.float32))
    c, s = gen.rope_table_f32(np.array(12345), Dr)
    _, z0 = oracle.qsa_block_key(rows, None, None, None)
    _, z1 = oracle.qsa_block_key(rows, None, c, s)
    np.testing.assert_array_equal(z0[: Di - Dr], z1[: Di - Dr])
    assert not np.array_equal(z0[Di - Dr:], z1[Di - Dr:])
    h = Dr // 2
    a = z0[Di - Dr:].astype(np.float64)
    b = z1[Di - Dr:].astype(np.float64)
    np.testing.assert_allclose(b[:h] ** 2 + b[h:] ** 2, a[0::2] ** 2 + a[1::2] ** 2, rtol=1e-5)


def _stream(seed, N, T, Di, Dr):
    rng = rng_for(seed)
    raw = bf16_bits(rng.standard_normal((N, T, Di)).astype(np.float32))
    pos = np.broadcast_to(np.arange(T), (N, T))
    rc, rs = gen.rope_table_f32(pos, Dr)
    w = bf16_bits(rng.uniform(0.5, 1.5, Di).astype(np.float32))
    return raw, np.ascontiguousarray(rc), np.ascontiguousarray(rs), w


def _full_history(raw, rc, rs, w, kbs, Bcap, eps):
    """Definition over the whole stream: block b = key of tokens
    [b*kbs, (b+1)*kbs) rotated at position b*kbs."""
    N, T, Di = raw.shape
    Dr = rc.shape[-1]
    bk = np.full((N, Bcap, Di), gen.BF16_SENTINEL, dtype=np.uint16)
    wf = bits_to_f32(w)
    for n in range(N):
        for b in range(T // kbs):
            _, z = oracle.qsa_block_key(raw[n, b * kbs:(b + 1) * kbs], wf, rc[n, b * kbs],
                                        rs[n, b * kbs], eps)
            bk[n, b] = oracle.f32_to_bf16(z)
    return bk


@pytest.mark.parametrize("seed", [54, 55, 56])
def test_split_invariance(seed):
    """Chaining calls over random chunk sizes (1, < kbs, = kbs, several kbs)
    gives, bit for bit, the block keys of the whole-history definition."""
    N, T, Di, Dr, kbs = 3, 300, 32, 8, 16
    Bcap = T // kbs + 1
    raw, rc, rs, w = _stream(seed, N, T, Di, Dr)
    want = _full_history(raw, rc, rs, w, kbs, Bcap, 1e-6)
    rng = rng_for(seed + 100)
    bk = np.full((N, Bcap, Di), gen.BF16_SENTINEL, dtype=np.uint16)
    state_raw = np.full((N, kbs - 1, Di), gen.BF16_NAN, dtype=np.uint16)
    state_rope = np.full((N, 2 * Dr), np.nan, dtype=np.float32)
    done = 0
    choices = [1, 2, kbs - 1, kbs, kbs + 1, 3 * kbs + 5, 7]
    while done < T:
        L = min(int(rng.choice(choices)), T - done)
        nraw = np.full_like(state_raw, gen.BF16_NAN)
        nrope = np.full_like(state_rope, np.nan)
        kl = np.full(N, done + L, dtype=np.int64)
        oracle.qsa_prepare(np.ascontiguousarray(raw[:, done:done + L]), bk, kl,
                           np.ascontiguousarray(rc[:, done:done + L]),
                           np.ascontiguousarray(rs[:, done:done + L]), w, state_raw, state_rope,
                           nraw, nrope, key_block_size=kbs, eps=1e-6)
        state_raw, state_rope = nraw, nrope
        done += L
    np.testing.assert_array_equal(bk, want)


def test_never_reads_invalid_state():
    """Invalid carried rows and an unused carried rope row are NaN in the
    generator; every written key must be finite."""
    case = gen.qsa_case(57, N=16, L=200, Di=64, Dr=32, kbs=32, past_max=1000)
    bk, nraw, nrope = oracle.run_qsa_case(case)
    written = bk != gen.BF16_SENTINEL
    vals = bits_to_f32(bk)
    assert np.all(np.isfinite(vals[written]))
    # and exactly the completed blocks were written
    for n in range(case["N"]):
        K = int(case["key_length"][n])
        P = K - case["L"]
        rows = set(np.where(np.any(written[n], axis=1))[0].tolist())
        assert rows <= set(range(P // 32, K // 32))
        r2 = K % 32
        assert np.all(np.isfinite(bits_to_f32(nraw[n, :r2])))
        if r2:
            assert np.all(np.isfinite(nrope[n]))


def test_disabled_features():
    case = gen.qsa_case(58, N=4, L=64, Di=32, Dr=8, kbs=8, past_max=100)
    N, kbs, Di = 4, 8, 32
    base, _, _ = oracle.run_qsa_case(case)
    no_norm = dict(case, k_norm_weight=None)
    bk1, _, _ = oracle.run_qsa_case(no_norm)
    no_rope = dict(case, rope_cos=None, rope_sin=None, past_incomplete_rope=None)
    bk2, _, _ = oracle.run_qsa_case(no_rope)
    assert not np.array_equal(base, bk1) and not np.array_equal(base, bk2)
    # without rope, the leading Di-Dr dims equal those of the rotated result
    np.testing.assert_array_equal(bk2[..., : Di - 8], base[..., : Di - 8])
    # without norm and rope, a key is the plain block mean
    plain = dict(case, k_norm_weight=None, rope_cos=None, rope_sin=None, past_incomplete_rope=None)
    bk3, _, _ = oracle.run_qsa_case(plain)
    n = 0
    K = int(case["key_length"][n])
    P = K - 64
    b = P // kbs + 1                        # a block made of new tokens only
    t0 = b * kbs - P
    m = bits_to_f32(case["raw_index_keys"][n, t0:t0 + kbs]).astype(np.float64).mean(axis=0)
    got = bits_to_f32(bk3[n, b]).astype(np.float64)
    assert np.all(np.abs(got - m) <= 2.0 ** -8 * np.abs(m) + 1e-6)


def test_empty_and_invalid():
    case = gen.qsa_case(59, N=2, L=0, Di=16, Dr=8, kbs=4, past_max=50)
    bk, nraw, _ = oracle.run_qsa_case(case)
    assert np.all(bk == gen.BF16_SENTINEL)
    case = gen.qsa_case(60, N=2, L=8, Di=16, Dr=8, kbs=4, past_max=50)
    bad = dict(case, key_length=np.array([3, 100], dtype=np.int64))   # K < L
    with pytest.raises(oracle.OracleError):
        oracle.run_qsa_case(bad)
    small = dict(case)
    small["caches"] = {"block_keys": gen.CacheSpec((2, 1, 16), np.uint16, gen.BF16_SENTINEL)}
    with pytest.raises(oracle.OracleError):
        oracle.run_qsa_case(small)


def test_broadcast_key_length():
    case = gen.qsa_case(61, N=3, L=40, Di=16, Dr=8, kbs=8, past_max=60, key_length_count=1)
    assert case["key_length"].shape == (1,)
    a, _, _ = oracle.run_qsa_case(case)
    full = dict(case, key_length=np.repeat(case["key_length"], 3))
    b, _, _ = oracle.run_qsa_case(full)
    np.testing.assert_array_equal(a, b)
