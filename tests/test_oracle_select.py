"""Pins of the block-selection oracle (aclnnNsaCompressAttentionInfer,
Formulas: compressed scores, selection pooling, head-group sum, top-k) over
QSAPrepare block keys.

* hand-worked cases with a closed form (tests/golden/select_hand.json);
* one head with unit ratios reduces to scipy's softmax;
* the pooling against an independent restatement as a convolution with two
  box filters, and the invariant sum_j P_slc'[j] = H * (l/d);
* block rows beyond key_length // key_block_size are never read (NaN there);
* top-k order (descending, ties by ascending index), padding with -1, and
  the empty sequence.
"""
import numpy as np
import pytest
import scipy.special

import gen
from oracle import qsa_select as S
from tests._util import golden


def _bits(a):
    return gen.bf16_bits(np.asarray(a, np.float32))


def test_hand_worked():
    g = golden("select_hand.json")
    r = np.exp(g["a"])
    den = 1 + r + r * r
    for c in g["cases"]:
        q, keys = _bits(c["q"]), _bits(c["keys"])
        scores, idx = S.select_sequence(q, keys, key_length=3 * 64, kbs=64, scale=c["scale"],
                                        sel_ratio=c["sel_ratio"], cmp_ratio=c["cmp_ratio"],
                                        k=c["k"])
        want = np.array([(p[0] + p[1] * r + p[2] * r * r) / den for p in c["poly"]])
        np.testing.assert_allclose(scores, want, rtol=1e-13, err_msg=c["note"])
        np.testing.assert_array_equal(idx, c["indices"], err_msg=c["note"])


def test_unit_ratios_one_head_is_softmax():
    rng = gen.rng_for(90)
    q = _bits(rng.standard_normal((1, 128)))
    keys = _bits(rng.standard_normal((40, 128)))
    scale = 1 / np.sqrt(128)
    scores, idx = S.select_sequence(q, keys, 40 * 16 + 7, 16, scale, 1, 1, 5)
    logits = scale * (S.bf16_to_f64(q) @ S.bf16_to_f64(keys).T)[0]
    np.testing.assert_allclose(scores, scipy.special.softmax(logits), rtol=1e-12)
    np.testing.assert_array_equal(idx, np.argsort(-logits, kind="stable")[:5])


@pytest.mark.parametrize("sel,cmp", [(1, 1), (2, 1), (4, 1), (2, 2), (3, 2), (4, 3)])
def test_pooling_is_a_double_box_filter(sel, cmp):
    """P_slc'[j] = (Q conv box(l'/d) conv box(l/d))[(l'/d) j]: each term
    Q[(l'/d) j - m - n] of the double sum is one tap of the two filters."""
    rng = gen.rng_for(91 + sel * 10 + cmp)
    H, nb = 3, 37
    q = _bits(rng.standard_normal((H, 64)))
    keys = _bits(rng.standard_normal((nb + 5, 64)))
    scores, _ = S.select_sequence(q, keys, nb * 32, 32, 0.125, sel, cmp, 4)
    p = S.compressed_scores(S.bf16_to_f64(q), S.bf16_to_f64(keys[:nb]), 0.125)
    full = np.convolve(np.convolve(p.sum(axis=0), np.ones(sel)), np.ones(cmp))
    J = S.num_selection_blocks(nb, sel, cmp)
    last = len(full) - 1                          # largest index with a tap in range
    assert len(scores) == J and sel * (J - 1) <= last < sel * J
    np.testing.assert_allclose(scores, full[sel * np.arange(J)], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(scores.sum(), H * cmp, rtol=1e-12)


def test_rows_beyond_the_block_count_are_not_read():
    rng = gen.rng_for(92)
    q = _bits(rng.standard_normal((4, 32)))
    keys = _bits(rng.standard_normal((20, 32)))
    keys[13:] = gen.BF16_NAN
    scores, idx = S.select_sequence(q, keys, 13 * 8 + 7, 8, 0.2, 2, 1, 3)
    assert np.all(np.isfinite(scores)) and len(scores) == S.num_selection_blocks(13, 2, 1)
    assert np.all((idx >= 0) & (idx < len(scores)))


def test_topk_ties_padding_and_empty():
    assert list(S.topk_indices(np.array([0.5, 1.0, 0.5, 1.0, 0.2]), 4)) == [1, 3, 0, 2]
    assert list(S.topk_indices(np.array([0.3, 0.1]), 4)) == [0, 1, -1, -1]
    q = _bits(np.ones((2, 8)))
    keys = _bits(np.ones((4, 8)))
    scores, idx = S.select_sequence(q, keys, 7, 8, 1.0, 1, 1, 3)      # 7 < 8: no block
    assert len(scores) == 0 and list(idx) == [-1, -1, -1]
    with pytest.raises(S.SelectOracleError):
        S.select_sequence(q, keys, 5 * 8, 8, 1.0, 1, 1, 3)             # 5 blocks > capacity 4


def test_case_runner():
    case = gen.qsa_select_case(93, N=5, H=4, Di=64, Bcap=12, kbs=16, sel_ratio=2, cmp_ratio=1,
                               topk=3)
    scores, idx = S.run_select_case(case)
    for n in range(5):
        nb = int(case["key_length"][n]) // 16
        J = S.num_selection_blocks(nb, 2, 1)
        assert np.all(scores[n, J:] == 0)
        sel = idx[n][idx[n] >= 0]
        assert len(sel) == min(3, J) and len(set(sel)) == len(sel)
