"""Pins of the oracle's scatter (aclnnKvRmsNormRopeCache, restrictions on
index: Norm mode index [B,S] in [-1,Scache), repeats allowed only across
batches; PA_BNSD slot_mapping [B*S] in [-1, BlockNum*BlockSize), no repeats;
-1 skips the token) and of the empty-input rule (aclnnMlaPrologV3WeightNz,
shape restrictions: B, S or T of 0 leaves the caches as they are).

The reconstruction below is a brute-force dictionary {cache row -> expected
row} built from the oracle's per-token outputs; the whole-op result must equal
it byte for byte, including every byte no token addresses.
"""
import numpy as np
import pytest

import gen
import oracle


def _expected_rows(case):
    """{flat cache row: (k_row_bits, ckv_row, scale)} from per-token outputs."""
    B, S, Dv, Dk = case["B"], case["S"], case["Dv"], case["Dk"]
    kv = case["kv"].reshape(B * S, Dv + Dk)
    cs = case["cos"].reshape(B * S, Dk)
    sn = case["sin"].reshape(B * S, Dk)
    rows = {}
    for t in range(B * S):
        if case["mode"] == "paged":
            v = int(case["slot_mapping"][t])
            if v == -1:
                continue
            bs = case["block_size"]
            flat = (v // bs) * bs + v % bs
        elif case["mode"] == "paged_blk":
            bs = case["block_size"]
            b, s = divmod(t, S)
            v = int(case["block_index"][b * (-(-S // bs)) + s // bs])
            if v == -1:
                continue
            flat = (v // bs) * bs + s % bs
        else:
            b, s = divmod(t, S)
            v = int(case["index"][b, s])
            if v == -1:
                continue
            flat = b * case["Sc"] + v
        assert flat not in rows
        yn, yr = oracle.token_outputs(kv[t], case["gamma"], cs[t], sn[t], Dv, Dk, case["eps"])
        if case["ckv_dtype"] == "int8":
            code, scale = oracle.quant_row(yn)
            rows[flat] = (oracle.f32_to_bf16(yr), code, scale)
        elif case["ckv_dtype"] == "fp8":
            code, scale = oracle.quant_row_fp8(yn)
            rows[flat] = (oracle.f32_to_bf16(yr), code, scale)
        else:
            rows[flat] = (oracle.f32_to_bf16(yr), oracle.f32_to_bf16(yn), None)
    return rows


def _brute(case):
    caches = {k: spec.numpy() for k, spec in case["caches"].items()}
    Dv, Dk = case["Dv"], case["Dk"]
    kc = caches["k_cache"].reshape(-1, Dk)
    ck = caches["ckv_cache"].reshape(-1, Dv)
    sc = caches["ckv_scale"].reshape(-1) if "ckv_scale" in caches else None
    for flat, (k, c, s) in _expected_rows(case).items():
        kc[flat] = k
        ck[flat] = c
        if sc is not None:
            sc[flat] = s
    return caches


def _assert_same(a, b):
    for k in a:
        np.testing.assert_array_equal(a[k].view(np.uint8), b[k].view(np.uint8), err_msg=k)


@pytest.mark.parametrize("ckv", ["bf16", "int8", "fp8"])
def test_paged_scatter_brute_force(ckv):
    case = gen.kvrc_paged_case(41, B=3, S=37, Dv=64, Dk=16, num_blocks=16, block_size=16,
                               slot_kind="random", skip_frac=0.2, ckv_dtype=ckv, max_pos=4096)
    got = oracle.run_kvrc_case(case)
    _assert_same(got, _brute(case))
    # every -1 and every unreferenced row still holds the sentinel
    written = {int(v) for v in case["slot_mapping"] if v >= 0}
    kc = got["k_cache"].reshape(-1, 16)
    for r in range(kc.shape[0]):
        if r not in written:
            assert np.all(kc[r] == gen.BF16_SENTINEL)


def test_paged_table_layout_brute_force():
    case = gen.kvrc_paged_case(42, B=2, S=40, Dv=32, Dk=8, num_blocks=12, block_size=16,
                               slot_kind="table")
    _assert_same(oracle.run_kvrc_case(case), _brute(case))


@pytest.mark.parametrize("ckv", ["bf16", "int8", "fp8"])
def test_norm_scatter_brute_force(ckv):
    case = gen.kvrc_norm_case(43, B=3, S=10, Dv=64, Dk=16, Bc=4, Sc=24, n_skip=4, ckv_dtype=ckv)
    # the same index value in two batches is legal (separate namespaces)
    case["index"][1, 0] = 5
    case["index"][2, 0] = 5
    case["index"][1][np.where(case["index"][1] == 5)[0][1:]] = -1
    case["index"][2][np.where(case["index"][2] == 5)[0][1:]] = -1
    got = oracle.run_kvrc_case(case)
    _assert_same(got, _brute(case))
    # batch 3 of the cache is never addressed (Bc > B)
    assert np.all(got["k_cache"][3] == gen.BF16_SENTINEL)


def test_norm_equals_paged_view():
    """A Norm-mode call equals a paged call on the cache viewed as
    [Bc, Sc, 1, d] with slot = b*Sc + index[b, s]."""
    case = gen.kvrc_norm_case(44, B=2, S=12, Dv=64, Dk=8, Bc=2, Sc=16, n_skip=3)
    norm = oracle.run_kvrc_case(case)
    idx = case["index"]
    slots = np.where(idx >= 0, np.arange(2)[:, None] * 16 + idx, -1).reshape(-1).astype(np.int64)
    kc = case["caches"]["k_cache"].numpy().reshape(2, 16, 1, 8)
    ck = case["caches"]["ckv_cache"].numpy().reshape(2, 16, 1, 64)
    oracle.paged_norm_rope_cache(case["kv"], case["gamma"], case["cos"], case["sin"], slots, kc, ck,
                                 eps=case["eps"])
    np.testing.assert_array_equal(norm["k_cache"].reshape(-1), kc.reshape(-1))
    np.testing.assert_array_equal(norm["ckv_cache"].reshape(-1), ck.reshape(-1))


def test_empty_input_leaves_caches():
    case = gen.kvrc_paged_case(45, B=0, S=5, Dv=32, Dk=8, num_blocks=4, block_size=8,
                               slot_kind="random")
    got = oracle.run_kvrc_case(case)
    assert np.all(got["k_cache"] == gen.BF16_SENTINEL) and np.all(got["ckv_cache"] == gen.BF16_SENTINEL)


def test_invalid_indices_rejected():
    case = gen.kvrc_paged_case(46, B=1, S=8, Dv=32, Dk=8, num_blocks=4, block_size=8,
                               slot_kind="random")
    bad = dict(case)
    bad["slot_mapping"] = case["slot_mapping"].copy()
    bad["slot_mapping"][1] = bad["slot_mapping"][0]
    with pytest.raises(oracle.OracleError, match="duplicate"):
        oracle.run_kvrc_case(bad)
    bad["slot_mapping"] = case["slot_mapping"].copy()
    bad["slot_mapping"][2] = 32
    with pytest.raises(oracle.OracleError, match="range"):
        oracle.run_kvrc_case(bad)
    bad["slot_mapping"][2] = -2
    with pytest.raises(oracle.OracleError, match="range"):
        oracle.run_kvrc_case(bad)
    ncase = gen.kvrc_norm_case(47, B=2, S=4, Dv=32, Dk=8, Bc=2, Sc=8, n_skip=0)
    ncase["index"][0, 1] = ncase["index"][0, 0]
    with pytest.raises(oracle.OracleError, match="duplicate"):
        oracle.run_kvrc_case(ncase)


def test_threads_do_not_change_result():
    case = gen.kvrc_paged_case(48, B=4, S=33, Dv=128, Dk=32, num_blocks=32, block_size=16,
                               slot_kind="random", skip_frac=0.1, ckv_dtype="int8")
    a = oracle.run_kvrc_case(case, nthreads=1)
    b = oracle.run_kvrc_case(case, nthreads=4)
    _assert_same(a, b)


@pytest.mark.parametrize("ckv", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("S,offsets", [(64, False), (40, False), (37, True)])
def test_paged_blk_scatter_brute_force(ckv, S, offsets):
    """Block-indexed mode (PA_BLK_BNSD): ragged last chunk, skipped chunks and
    entries that are not multiples of the block size (only value / BS names
    the block)."""
    case = gen.kvrc_paged_blk_case(49, B=3, S=S, Dv=64, Dk=16, num_blocks=24, block_size=16,
                                   ckv_dtype=ckv, n_skip=2, entry_offsets=offsets)
    _assert_same(oracle.run_kvrc_case(case), _brute(case))


def test_paged_blk_equals_per_token_slots():
    """A block-indexed call equals a per-token paged call whose slot for token
    (b, s) is block*BS + s mod BS (block = entry / BS; -1 chunks -> -1)."""
    case = gen.kvrc_paged_blk_case(50, B=2, S=50, Dv=32, Dk=8, num_blocks=12, block_size=16,
                                   n_skip=1, entry_offsets=True)
    blk = oracle.run_kvrc_case(case)
    BS, S = 16, 50
    slots = []
    for b in range(2):
        for s in range(S):
            v = int(case["block_index"][b * 4 + s // BS])
            slots.append(-1 if v < 0 else (v // BS) * BS + s % BS)
    per_token = dict(case, mode="paged", slot_mapping=np.array(slots, dtype=np.int64))
    _assert_same(blk, oracle.run_kvrc_case(per_token))


def test_paged_blk_invalid_rejected():
    case = gen.kvrc_paged_blk_case(51, B=2, S=32, Dv=32, Dk=8, num_blocks=8, block_size=16)
    bad = dict(case, block_index=case["block_index"].copy())
    bad["block_index"][1] = bad["block_index"][0] + 3           # same block, other offset
    with pytest.raises(oracle.OracleError, match="duplicate"):
        oracle.run_kvrc_case(bad)
    bad["block_index"] = case["block_index"].copy()
    bad["block_index"][2] = 8 * 16
    with pytest.raises(oracle.OracleError, match="range"):
        oracle.run_kvrc_case(bad)
