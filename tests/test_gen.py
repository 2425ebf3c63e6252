"""The seeded input generator: determinism and the structure of the five
named workloads (shapes, value ranges, slot uniqueness, skip counts)."""
import numpy as np

import gen


def test_bf16_bits_round_trip_and_rounding():
    a = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, np.inf], dtype=np.float32)
    np.testing.assert_array_equal(gen.bf16_bits(a),
                                  np.array([0x3F80, 0x3F80, 0x3F82, 0x8000, 0x7F80], dtype=np.uint16))
    b = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    np.testing.assert_array_equal(gen.bf16_bits(gen.bits_to_f32(b)), b)


def test_deterministic():
    a = gen.make_config("norm_tiny")
    b = gen.make_config("norm_tiny")
    for k in ["kv", "gamma", "cos", "sin", "index"]:
        np.testing.assert_array_equal(a[k], b[k])
    c = gen.make_config("norm_tiny", seed=99)
    assert not np.array_equal(a["kv"], c["kv"])


def test_norm_tiny_structure():
    c = gen.make_config("norm_tiny")
    assert c["kv"].shape == (2, 1, 16, 576) and c["cos"].shape == (2, 1, 16, 64)
    assert c["index"].shape == (2, 16) and c["index"].dtype == np.int64
    assert (c["index"] == -1).sum() == 3
    for b in range(2):
        v = c["index"][b][c["index"][b] >= 0]
        assert len(set(v.tolist())) == len(v) and v.min() >= 0 and v.max() < 32
    g = gen.bits_to_f32(c["gamma"])
    assert g.min() >= 0.5 and g.max() <= 1.5
    # position 0 has angle 0: cos 1, sin 0
    assert np.all(c["cos"][:, 0, 0] == 0x3F80) and np.all(c["sin"][:, 0, 0] == 0)


def test_decode_structure():
    c = gen.make_config("decode_paged")
    s = c["slot_mapping"]
    assert s.shape == (256,) and (s == -1).sum() == 13
    v = s[s >= 0]
    assert len(np.unique(v)) == len(v) and v.max() < 4096 * 128
    assert c["caches"]["ckv_cache"].shape == (4096, 128, 1, 512)


def test_prefill_structure():
    c = gen.make_config("prefill_paged")
    s = c["slot_mapping"]
    # B=8, S=4096: 32,768 tokens (the workload's "65,536 tokens" note disagrees
    # with its own B and S and with 32 blocks of 128 per sequence; B and S win)
    assert s.shape == (32768,) and np.all(s >= 0)
    assert len(np.unique(s)) == 32768
    tbl = c["block_table"]
    assert tbl.shape == (8, 32) and len(np.unique(tbl)) == 256
    # slot = table[b, s // 128] * 128 + s % 128
    b, pos = 5, 1000
    assert s[b * 4096 + pos] == tbl[b, pos // 128] * 128 + pos % 128


def test_quant_and_qsa_structure():
    c = gen.make_config("quant_paged")
    assert c["ckv_dtype"] == "int8" and c["caches"]["ckv_scale"].shape == (4096, 128, 1)
    assert c["block_table"].shape == (64, 8)
    q = gen.make_config("qsa")
    assert q["raw_index_keys"].shape == (32, 2048, 128)
    assert np.all(q["key_length"] == q["past"] + 2048)
    r = q["past"] % 64
    for n in range(32):
        rows = gen.bits_to_f32(q["past_incomplete_raw_keys"][n])
        assert np.all(np.isfinite(rows[: r[n]])) and np.all(np.isnan(rows[r[n]:]))
        assert np.isnan(q["past_incomplete_rope"][n]).all() == (r[n] == 0)
    assert q["caches"]["block_keys"].shape == (32, 160, 128)


def test_bytes_per_token():
    assert gen.kvrc_bytes_per_written_token(512, 64, "bf16") == 2568
    assert gen.kvrc_bytes_per_written_token(512, 64, "int8") == 2060
