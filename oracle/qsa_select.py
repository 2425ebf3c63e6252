"""CPU oracle of block selection over QSAPrepare block keys: compressed
attention scores, selection-block pooling, head-group sum, top-k.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): only the tests,
``__graft_entry__.smoke()`` and the bench's CPU-baseline leg may use it; the
library never imports it and shares no code with it.

Source: aclnnNsaCompressAttentionInfer (Description and Formulas):
    P_cmp      = Softmax(scale * query . key^T)
    P_slc[j]   = sum_{m=0}^{l'/d-1} sum_{n=0}^{l/d-1} P_cmp[(l'/d) * j - m - n]
    P_slc'     = sum over the G query heads that share one key head
    topkIndices = topk(P_slc')
with the block keys of openvino.opset17.qsa_prepare as the compressed keys
(one key per complete block of key_block_size tokens, so d = key_block_size).

Readings (the pages leave these open):
  * single-token inference: one query per sequence and head, which sees
    every complete block of its sequence (nb = key_length // key_block_size
    blocks; no causal mask is needed);
  * one key head per sequence (the block keys have none), so G = H: the
    scores of all H query heads are summed;
  * sel_ratio = l'/d and cmp_ratio = l/d are positive integers; the pooling
    formula is taken as printed, and a term whose compressed index falls
    outside [0, nb) contributes 0; selection block j exists for
    0 <= j < J = (nb + sel_ratio + cmp_ratio - 3) // sel_ratio + 1 (the
    blocks with at least one index in range; J = 0 when nb = 0);
  * precision: float64; the softmax subtracts the row maximum;
  * top-k: the k existing selection blocks of largest score, in descending
    score order, equal scores in ascending index order; positions beyond
    min(k, J) hold -1.

Every function is pinned in ``tests/test_oracle_select.py``.
"""
from __future__ import annotations

import numpy as np


class SelectOracleError(RuntimeError):
    pass


def bf16_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def num_selection_blocks(nb: int, sel_ratio: int, cmp_ratio: int) -> int:
    if nb <= 0:
        return 0
    return (nb + sel_ratio + cmp_ratio - 3) // sel_ratio + 1


def compressed_scores(q, keys, scale):
    """P_cmp [H, nb]: softmax over the blocks of scale * q . k (float64)."""
    s = float(scale) * (q @ keys.T)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def pool(p_cmp_sum, nb, sel_ratio, cmp_ratio):
    """P_slc'[j] = sum_m sum_n Q[sel_ratio * j - m - n] over the existing j,
    with Q the head-summed compressed scores and out-of-range terms 0."""
    J = num_selection_blocks(nb, sel_ratio, cmp_ratio)
    out = np.zeros(J)
    for j in range(J):
        acc = 0.0
        for m in range(sel_ratio):
            for n in range(cmp_ratio):
                i = sel_ratio * j - m - n
                if 0 <= i < nb:
                    acc += p_cmp_sum[i]
        out[j] = acc
    return out


def topk_indices(scores, k):
    """Indices of the k largest scores, descending, ties by ascending index;
    -1 where fewer than k exist."""
    order = sorted(range(len(scores)), key=lambda j: (-scores[j], j))
    out = np.full(k, -1, dtype=np.int64)
    out[: min(k, len(order))] = order[:k]
    return out


def select_sequence(q_bits, keys_bits, key_length, kbs, scale, sel_ratio, cmp_ratio, k):
    """One sequence: q [H, Di] and block keys [Bcap, Di] (bf16 bits).
    Returns (P_slc' [J] float64, top-k indices [k])."""
    if kbs < 1 or sel_ratio < 1 or cmp_ratio < 1 or k < 0:
        raise SelectOracleError("bad argument")
    nb = int(key_length) // kbs
    if nb > keys_bits.shape[0]:
        raise SelectOracleError("key_length beyond the block-key capacity")
    if nb == 0:
        return np.zeros(0), np.full(k, -1, dtype=np.int64)
    q = bf16_to_f64(q_bits)
    keys = bf16_to_f64(keys_bits[:nb])
    p = compressed_scores(q, keys, scale)
    scores = pool(p.sum(axis=0), nb, sel_ratio, cmp_ratio)
    return scores, topk_indices(scores, k)


def run_select_case(case):
    """All sequences of a gen.qsa_select_case: scores [N, Jcap] (0 beyond each
    sequence's J) and indices [N, k]."""
    N = case["N"]
    Jcap = case["Jcap"]
    scores = np.zeros((N, Jcap))
    idx = np.full((N, case["topk"]), -1, dtype=np.int64)
    kl = case["key_length"]
    for n in range(N):
        s, t = select_sequence(case["query"][n], case["block_keys"][n], kl[n % len(kl)],
                               case["kbs"], case["scale"], case["sel_ratio"],
                               case["cmp_ratio"], case["topk"])
        scores[n, : len(s)] = s
        idx[n] = t
    return scores, idx
