"""GPU parity of block selection (qsa_select_topk) against the float64 oracle
(oracle/qsa_select.py) on the same seeded inputs.

Scores: float32 on the device (bf16 products summed on the matrix cores,
expf, sums in fixed orders), float64 in the oracle. The bound per selection
score follows the arithmetic: each logit scale * q . k is within
ds = scale * 2 Di u / (1 - Di u) * sum |q_d k_d| (+ one rounding) of its exact
value (u = 2^-24); a softmax term exp(s - max) / sum then has relative error
at most 4 ds + (nb + 32) u (1 + max |s - max|); the head sum and the pooling
add (H + l'/d * l/d) u. Every score must be within that relative bound, and
the median relative error must stay below 1e-5 (a float32 path gives about
1e-7; the bound itself allows worst cases).

Top-k indices decide integers from floating point, so what is unique is
compared: the count min(topk, J), the padding with -1, distinct in-range
indices, the device's own order (descending score, equal scores by
ascending index), and agreement with the oracle's ranking wherever the
oracle scores are farther apart than the bound; between scores closer than
that, either order is correct.
"""
import numpy as np
import pytest
import torch

import gen
import latent_attention_kv_amd as k
from oracle import qsa_select as S

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
U = 2.0 ** -24


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _native_library_loaded():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert k.lib()._name == k.LIB_PATH
    yield


def dbf(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def run_select_gpu(case, err=None, key_length=None):
    N = case["N"]
    kl = case["key_length"] if key_length is None else key_length
    scores = torch.full((N, case["Jcap"]), -7.0, dtype=torch.float32, device=DEV)
    idx = torch.full((N, case["topk"]), -7, dtype=torch.int32, device=DEV)
    k.qsa_select_topk(dbf(case["query"]), dbf(case["block_keys"]), torch.from_numpy(kl).to(DEV),
                      scores, idx, key_block_size=case["kbs"], sel_ratio=case["sel_ratio"],
                      cmp_ratio=case["cmp_ratio"], scale=case["scale"], err_count=err)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), idx.cpu().numpy()


def score_bound(case, n, scores_ref):
    """Per-score absolute bound for sequence n (see the module docstring)."""
    kl = case["key_length"]
    nb = int(kl[n % len(kl)]) // case["kbs"]
    if nb == 0:
        return np.zeros(0)
    q = S.bf16_to_f64(case["query"][n])
    kk = S.bf16_to_f64(case["block_keys"][n][:nb])
    Di, H = q.shape[1], q.shape[0]
    sc = case["scale"]
    s = sc * (q @ kk.T)
    ds = sc * (2 * Di * U / (1 - Di * U)) * (np.abs(q) @ np.abs(kk).T).max() + np.abs(s).max() * U
    spread = float((s.max(axis=1, keepdims=True) - s).max())
    rel = 4 * ds + (nb + 32) * U * (1 + spread) + (H + case["sel_ratio"] * case["cmp_ratio"]) * U
    return np.abs(scores_ref) * rel * 1.5 + 1e-30


def compare_select(case, got_scores, got_idx, *, kl=None):
    ref_scores, ref_idx = S.run_select_case(case if kl is None else dict(case, key_length=kl))
    kl = case["key_length"] if kl is None else kl
    N, k_ = case["N"], case["topk"]
    rels = []
    for n in range(N):
        nb = int(kl[n % len(kl)]) // case["kbs"]
        J = S.num_selection_blocks(nb, case["sel_ratio"], case["cmp_ratio"])
        g, r = got_scores[n].astype(np.float64), ref_scores[n]
        assert np.all(g[J:] == 0), f"seq {n}: scores beyond J = {J} must be 0"
        tol = score_bound(dict(case, key_length=kl), n, r[:J])
        err = np.abs(g[:J] - r[:J])
        bad = ~(err <= tol)
        assert not bad.any(), (f"seq {n}: {int(bad.sum())} scores beyond the bound, e.g. j="
                               f"{np.flatnonzero(bad)[0]} gpu {g[np.flatnonzero(bad)[0]]!r} "
                               f"oracle {r[np.flatnonzero(bad)[0]]!r}")
        if J:
            rels.append(err / np.maximum(np.abs(r[:J]), 1e-300))
        # top-k: what is unique
        gi = got_idx[n]
        cnt = min(k_, J)
        assert np.all(gi[cnt:] == -1), f"seq {n}: padding"
        sel = gi[:cnt].astype(np.int64)
        assert np.all((sel >= 0) & (sel < J)) and len(set(sel.tolist())) == cnt, f"seq {n}: indices"
        gs = got_scores[n][sel]                       # the device's own order
        for p in range(cnt - 1):
            assert gs[p] > gs[p + 1] or (gs[p] == gs[p + 1] and sel[p] < sel[p + 1]), \
                f"seq {n}: order at {p}"
        if cnt and cnt < J:
            order = np.argsort(-r[:J], kind="stable")
            tau = r[order[cnt - 1]]
            tt = tol[order[cnt - 1]]
            inside = np.zeros(J, bool)
            inside[sel] = True
            assert np.all(r[:J][inside] >= tau - tol[inside] - tt), f"seq {n}: a selected block scores too low"
            assert np.all(r[:J][~inside] <= tau + tol[~inside] + tt), f"seq {n}: a better block left out"
        # the oracle's ranking wherever it is decided beyond the bound
        ro = ref_idx[n][:cnt]
        for p in range(cnt):
            if sel[p] != ro[p]:
                assert abs(r[sel[p]] - r[ro[p]]) <= tol[sel[p]] + tol[ro[p]], \
                    f"seq {n}: rank {p} differs beyond the bound"
    med = float(np.median(np.concatenate(rels))) if rels else 0.0
    assert med < 1e-5, f"median relative error {med}"
    return med


def test_select_named_workload_full_size():
    say("[select] workload qsa_select")
    case = gen.make_config("qsa_select")
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    scores, idx = run_select_gpu(case, err=err)
    assert int(err.item()) == 0
    med = compare_select(case, scores, idx)
    say(f"[select] median relative score error {med:.2e}")


# Both kernels: Di in {64, 128}, H in {16, 32, 64, 128} and Bcap <= 512 (up to
# 128 Bcap for H = 128) run on the compile-time fast path, the rest (Di 32,
# 96, 256, H 48, Bcap 1000, and keys beyond one LDS chunk) on the general one.
@pytest.mark.parametrize("N,H,Di,Bcap,kbs,sel,cmp,topk", [
    (3, 16, 32, 5, 16, 1, 1, 2), (4, 32, 64, 40, 32, 2, 1, 8), (5, 64, 128, 100, 64, 3, 2, 10),
    (2, 128, 256, 300, 64, 4, 1, 16), (3, 16, 128, 1000, 16, 2, 2, 64), (2, 48, 96, 17, 8, 1, 3, 40),
    (2, 128, 128, 256, 64, 2, 1, 16), (3, 16, 64, 512, 16, 1, 1, 32), (2, 64, 128, 500, 64, 2, 2, 24),
    (2, 128, 64, 200, 32, 1, 4, 12), (4, 32, 128, 129, 16, 1, 1, 130),
    (2, 16, 2048, 64, 16, 2, 1, 8),                             # Di near the LDS limit
])
def test_select_shapes(N, H, Di, Bcap, kbs, sel, cmp, topk):
    say(f"[select] N={N} H={H} Di={Di} Bcap={Bcap} kbs={kbs} sel={sel} cmp={cmp} topk={topk}")
    case = gen.qsa_select_case(700 + Bcap + H, N=N, H=H, Di=Di, Bcap=Bcap, kbs=kbs, sel_ratio=sel,
                               cmp_ratio=cmp, topk=topk)
    compare_select(case, *run_select_gpu(case))


def test_select_more_sequences_than_the_chip_holds_at_once():
    """600 sequences on the compile-time kernel: more workgroups than are
    resident at once (LDS and registers hold two per compute unit), so
    compute units run several in turn on the same LDS."""
    say("[select] N=600 H=64 Di=128 Bcap=256")
    case = gen.qsa_select_case(719, N=600, H=64, Di=128, Bcap=256, kbs=64, sel_ratio=2, cmp_ratio=1,
                               topk=16, kl_lo=64)
    compare_select(case, *run_select_gpu(case))


def test_select_graph_replays_match_eager():
    """Block selection captured in a HIP graph: every replay, with the outputs
    reset eagerly in between, gives the eager call's scores and indices bit
    for bit (the kernel is deterministic), and those meet the oracle's bar."""
    case = gen.qsa_select_case(720, N=20, H=64, Di=128, Bcap=256, kbs=64, sel_ratio=2, cmp_ratio=1,
                               topk=16, kl_lo=64)
    want_scores, want_idx = run_select_gpu(case)
    compare_select(case, want_scores, want_idx)
    N = case["N"]
    q, keys = dbf(case["query"]), dbf(case["block_keys"])
    kl = torch.from_numpy(case["key_length"]).to(DEV)
    scores = torch.full((N, case["Jcap"]), -7.0, dtype=torch.float32, device=DEV)
    idx = torch.full((N, case["topk"]), -7, dtype=torch.int32, device=DEV)

    def call():
        k.qsa_select_topk(q, keys, kl, scores, idx, key_block_size=case["kbs"],
                          sel_ratio=case["sel_ratio"], cmp_ratio=case["cmp_ratio"],
                          scale=case["scale"])

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for rep in range(4):
        scores.fill_(-7.0)                                   # eager reset between replays
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(scores.cpu().numpy().view(np.uint32), want_scores.view(np.uint32)), rep
        assert np.array_equal(idx.cpu().numpy(), want_idx), rep


def test_select_edge_lengths_and_broadcast():
    """key_length below one block (no block), exactly the capacity, a
    broadcast key_length, and topk beyond the block count (padding)."""
    case = gen.qsa_select_case(710, N=4, H=16, Di=64, Bcap=20, kbs=16, sel_ratio=2, cmp_ratio=1,
                               topk=12)
    kl = np.array([15, 20 * 16, 20 * 16 + 15, 40], dtype=np.int64)
    keys = case["block_keys"].copy()
    rng = gen.rng_for(711)
    fresh = gen.bf16_bits(rng.standard_normal(keys.shape, dtype=np.float32))
    for n in range(4):
        nb = int(kl[n]) // 16
        keys[n, :nb] = fresh[n, :nb]
        keys[n, nb:] = gen.BF16_NAN
    case = dict(case, block_keys=keys, key_length=kl)
    compare_select(case, *run_select_gpu(case))
    one = dict(case, key_length=np.array([7 * 16 + 3], dtype=np.int64),
               block_keys=np.where(np.arange(20)[None, :, None] < 7, fresh, gen.BF16_NAN).astype(np.uint16))
    compare_select(one, *run_select_gpu(one))


@pytest.mark.parametrize("H,Di", [(64, 128), (48, 96)])
def test_select_rank_paths_around_128_candidates(H, Di):
    """Up to 128 selection blocks the top-k counts each block's rank on four
    lanes with a quad sum; from 129 on, in segments added with LDS atomics.
    J = nb / 2 + 1 = 127, 128, 129, 130 (sel 2, cmp 1) on both kernels (the
    compile-time kernel at H 64 / Di 128, the general one at H 48 / Di 96);
    the rows past each sequence's blocks are NaN, and the compile-time kernel
    loads the fragments of its first tile before the key length is known."""
    say(f"[select] rank paths around 128 candidates, H={H} Di={Di}")
    case = gen.qsa_select_case(718 + H, N=4, H=H, Di=Di, Bcap=260, kbs=16, sel_ratio=2, cmp_ratio=1,
                               topk=20)
    kl = np.array([252 * 16 + 3, 254 * 16, 256 * 16 + 15, 258 * 16], dtype=np.int64)
    keys = case["block_keys"].copy()
    fresh = gen.bf16_bits(gen.rng_for(719 + H).standard_normal(keys.shape, dtype=np.float32))
    for n in range(4):
        nb = int(kl[n]) // 16
        keys[n, :nb] = fresh[n, :nb]
        keys[n, nb:] = gen.BF16_NAN
    case = dict(case, block_keys=keys, key_length=kl)
    got = run_select_gpu(case)
    compare_select(case, *got)
    assert [S.num_selection_blocks(int(x) // 16, 2, 1) for x in kl] == [127, 128, 129, 130]


def test_select_invalid_lengths_counted():
    case = gen.qsa_select_case(712, N=3, H=16, Di=32, Bcap=8, kbs=16, sel_ratio=1, cmp_ratio=1,
                               topk=4)
    kl = case["key_length"].copy()
    kl[0] = 9 * 16                                # 9 blocks > capacity 8
    kl[2] = -5
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    scores, idx = run_select_gpu(case, err=err, key_length=kl)
    assert int(err.item()) == 2
    assert np.all(scores[[0, 2]] == 0) and np.all(idx[[0, 2]] == -1)
    ok = dict(case, N=1, query=case["query"][1:2], block_keys=case["block_keys"][1:2],
              key_length=case["key_length"][1:2])
    compare_select(ok, scores[1:2], idx[1:2])


def test_select_invalid_lengths_counted_fast_kernel():
    """The same rule on the compile-time kernel (Di = 128, H = 64)."""
    case = gen.qsa_select_case(717, N=3, H=64, Di=128, Bcap=50, kbs=16, sel_ratio=2, cmp_ratio=1,
                               topk=5)
    kl = case["key_length"].copy()
    kl[1] = 51 * 16                               # 51 blocks > capacity 50
    kl[2] = -1
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    scores, idx = run_select_gpu(case, err=err, key_length=kl)
    assert int(err.item()) == 2
    assert np.all(scores[[1, 2]] == 0) and np.all(idx[[1, 2]] == -1)
    ok = dict(case, N=1, query=case["query"][:1], block_keys=case["block_keys"][:1],
              key_length=case["key_length"][:1])
    compare_select(ok, scores[:1], idx[:1])


def test_select_exact_ties_by_ascending_index():
    """Identical key rows give identical scores on both sides: equal scores
    are ranked by ascending block index."""
    case = gen.qsa_select_case(713, N=2, H=32, Di=64, Bcap=24, kbs=8, sel_ratio=1, cmp_ratio=1,
                               topk=10, kl_lo=24 * 8, kl_hi=24 * 8 + 1)
    keys = case["block_keys"].copy()
    keys[:, 5] = keys[:, 2]
    keys[:, 17] = keys[:, 2]
    keys[:, 9] = keys[:, 2]
    case = dict(case, block_keys=keys)
    scores, idx = run_select_gpu(case)
    compare_select(case, scores, idx)
    for n in range(2):
        assert scores[n, 2] == scores[n, 5] == scores[n, 9] == scores[n, 17]
        pos = [list(idx[n]).index(j) for j in (2, 5, 9, 17) if j in idx[n]]
        assert pos == sorted(pos)


def test_select_deterministic():
    case = gen.qsa_select_case(714, N=6, H=64, Di=128, Bcap=64, kbs=64, sel_ratio=2, cmp_ratio=1,
                               topk=8)
    a = run_select_gpu(case)
    b = run_select_gpu(case)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_select_many_candidates_argmax_path():
    """More than 2048 selection blocks: the one-wavefront arg-max top-k, over
    keys staged in several chunks."""
    say("[select] J > 2048, several key chunks")
    case = gen.qsa_select_case(715, N=2, H=16, Di=32, Bcap=2100, kbs=8, sel_ratio=1, cmp_ratio=1,
                               topk=24, kl_lo=2060 * 8, kl_hi=2100 * 8 + 1)
    compare_select(case, *run_select_gpu(case))


def test_select_nan_scores_are_never_selected():
    """A NaN inside a sequence's key rows makes every score of that sequence
    NaN (the softmax sums take it in): no block is selected, every index is
    -1; the other sequences are unaffected."""
    case = gen.qsa_select_case(716, N=3, H=32, Di=64, Bcap=40, kbs=16, sel_ratio=2, cmp_ratio=1,
                               topk=8, kl_lo=30 * 16, kl_hi=40 * 16 + 1)
    keys = case["block_keys"].copy()
    keys[1, 3, 5] = gen.BF16_NAN
    case = dict(case, block_keys=keys)
    scores, idx = run_select_gpu(case)
    nb = int(case["key_length"][1]) // 16
    J = S.num_selection_blocks(nb, 2, 1)
    assert np.all(np.isnan(scores[1, :J])) and np.all(scores[1, J:] == 0)
    assert np.all(idx[1] == -1)
    rest = [0, 2]
    ok = dict(case, N=2, query=case["query"][rest], block_keys=keys[rest],
              key_length=case["key_length"][rest])
    compare_select(ok, scores[rest], idx[rest])


@pytest.mark.parametrize("scale", [2.0, 8.0])
def test_select_wide_score_spread(scale):
    """Logits spread over hundreds of log2 units (a large scale): some or
    most lanes of the fast kernel meet exp2 arguments below -126, whose
    results are subnormal or zero, and take exp2f with its subnormal
    handling instead of the bare v_exp_f32."""
    say(f"[select] wide score spread, scale {scale}")
    case = gen.qsa_select_case(717, N=16, H=64, Di=128, Bcap=256, kbs=64, sel_ratio=2,
                               cmp_ratio=1, topk=16, kl_lo=128 * 64, kl_hi=256 * 64 + 1,
                               scale=scale)
    compare_select(case, *run_select_gpu(case))
