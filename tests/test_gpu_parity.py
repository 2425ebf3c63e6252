"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on
the same seeded inputs.

Bar (per output):
  * placement of every written row, and every byte no token addresses:
    bit-exact;
  * int8 codes: bit-exact; float32 scales and carried rope rows: within
    1e-5 relative;
  * bf16 outputs: within 1 bf16 ulp of bf16(oracle float32).
The five named workloads run at full size in the launch configuration the
bench times; the edge cases cover ragged tails, skipped and invalid indices,
other shapes (generic kernel), extreme magnitudes and QSA state chaining.
"""
import numpy as np
import pytest
import torch

import gen
import latent_attention_kv_amd as k
import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _native_library_loaded():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L = k.lib()
    assert L._name == k.LIB_PATH
    yield


def dbf(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def dt(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def ordered(t):
    """bf16 (as int16 bits) -> int32 ordered like the values; +-0 -> 0."""
    x = t.view(torch.int16).to(torch.int32)
    mag = x & 0x7FFF
    return torch.where(x < 0, -mag, mag)


# ---------------------------------------------------------------------------
# norm-rope-cache helpers
# ---------------------------------------------------------------------------

def run_kvrc_gpu(case, err=None, index_override=None):
    caches = {}
    for name, spec in case["caches"].items():
        a = spec.numpy()
        caches[name] = dbf(a) if spec.dtype == np.uint16 else dt(a)
    args = (dbf(case["kv"]), dbf(case["gamma"]), dbf(case["cos"]), dbf(case["sin"]))
    if case["mode"] == "paged":
        idx = case["slot_mapping"] if index_override is None else index_override
        k.kvrc_paged_norm_rope_cache(*args, dt(idx), caches["k_cache"], caches["ckv_cache"],
                                     caches.get("ckv_scale"), eps=case["eps"], err_count=err)
    elif case["mode"] == "paged_blk":
        idx = case["block_index"] if index_override is None else index_override
        k.kvrc_paged_blk_norm_rope_cache(*args, dt(idx), caches["k_cache"], caches["ckv_cache"],
                                         caches.get("ckv_scale"), eps=case["eps"], err_count=err)
    else:
        idx = case["index"] if index_override is None else index_override
        k.kvrc_norm_rope_cache(*args, dt(idx), caches["k_cache"], caches["ckv_cache"],
                               caches.get("ckv_scale"), eps=case["eps"], err_count=err)
    torch.cuda.synchronize()
    return caches


def written_rows(case):
    if case["mode"] == "paged":
        v = case["slot_mapping"]
        return np.unique(v[v >= 0])
    if case["mode"] == "paged_blk":
        S, bs = case["S"], case["block_size"]
        chunks = -(-S // bs)
        rows = []
        for b in range(case["B"]):
            for s in range(S):
                v = int(case["block_index"][b * chunks + s // bs])
                if v >= 0:
                    rows.append((v // bs) * bs + s % bs)
        return np.unique(np.array(rows, dtype=np.int64))
    idx = case["index"]
    rows = np.arange(case["B"])[:, None] * case["Sc"] + idx
    return np.unique(rows[idx >= 0])


def compare_kvrc(case, got, want, *, exact_bf16=False):
    """Returns (max bf16 ulp, number of bf16 elements off by one)."""
    rows = torch.from_numpy(written_rows(case)).to(DEV)
    max_ulp, off = 0, 0
    for name, g in got.items():
        w = want[name]
        if g.dtype == torch.bfloat16:
            wd = dbf(w)
            d = (ordered(g) - ordered(wd)).abs()
            n_rows = d.shape[0] * (d.shape[2] if case["mode"] == "norm" else d.shape[1])
            per_row = d.reshape(n_rows, -1).amax(dim=1)
            untouched = torch.ones(n_rows, dtype=torch.bool, device=DEV)
            untouched[rows] = False
            assert int(per_row[untouched].max().item() if untouched.any() else 0) == 0, \
                f"{name}: bytes outside the written rows changed"
            m = int(d.max().item())
            assert m <= (0 if exact_bf16 else 1), f"{name}: {m} bf16 ulps from the oracle"
            max_ulp = max(max_ulp, m)
            off += int((d > 0).sum().item())
            del d, wd
        elif g.dtype in (torch.int8, torch.uint8):
            assert torch.equal(g, dt(w)), f"{name}: int8 / E4M3FN codes differ"
        else:
            wd = dt(w)
            assert torch.equal(torch.isnan(g), torch.isnan(wd))
            rel = ((g - wd).abs() / wd.abs().clamp_min(1e-30)).nan_to_num(0.0)
            assert float(rel.max().item()) <= 1e-5, f"{name}: relative error above 1e-5"
    return max_ulp, off


NAMED_KVRC = ["norm_tiny", "decode_paged", "prefill_paged", "quant_paged", "quant_fp8_paged"]
CKV = ["bf16", "int8", "fp8"]


@pytest.mark.parametrize("name", NAMED_KVRC)
def test_named_workload_full_size(name):
    say(f"[parity] workload {name}")
    case = gen.make_config(name)
    want = oracle.run_kvrc_case(case)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = run_kvrc_gpu(case, err=err)
    max_ulp, off = compare_kvrc(case, got, want)
    assert int(err.item()) == 0
    say(f"[parity] {name}: max bf16 ulp {max_ulp}, elements off by one ulp {off}")


@pytest.mark.parametrize("name", NAMED_KVRC)
def test_named_workload_bit_exact(name):
    """Stronger than the bar: this implementation uses IEEE division and
    square root in the oracle's order, so every output is bit-identical."""
    say(f"[exact] workload {name}")
    case = gen.make_config(name)
    want = oracle.run_kvrc_case(case)
    got = run_kvrc_gpu(case)
    compare_kvrc(case, got, want, exact_bf16=True)


GENERIC_SHAPES = [(8, 8), (64, 16), (128, 32), (520, 72), (1024, 128), (512, 128), (256, 64)]


@pytest.mark.parametrize("dv,dk", GENERIC_SHAPES)
@pytest.mark.parametrize("ckv", CKV)
def test_other_shapes_paged(dv, dk, ckv):
    say(f"[parity] paged Dv={dv} Dk={dk} {ckv}")
    case = gen.kvrc_paged_case(100 + dv + dk, B=3, S=37, Dv=dv, Dk=dk, num_blocks=16,
                               block_size=16, slot_kind="random", skip_frac=0.15, ckv_dtype=ckv,
                               max_pos=4096)
    compare_kvrc(case, run_kvrc_gpu(case), oracle.run_kvrc_case(case), exact_bf16=True)


@pytest.mark.parametrize("B,S", [(1, 1), (1, 5), (3, 7), (2, 333), (7, 129)])
@pytest.mark.parametrize("ckv", CKV)
def test_ragged_token_counts_d576(B, S, ckv):
    say(f"[parity] d576 ragged B={B} S={S} {ckv}")
    case = gen.kvrc_paged_case(200 + B * S, B=B, S=S, Dv=512, Dk=64, num_blocks=64,
                               block_size=32, slot_kind="random", skip_frac=0.2, ckv_dtype=ckv)
    compare_kvrc(case, run_kvrc_gpu(case), oracle.run_kvrc_case(case), exact_bf16=True)


@pytest.mark.parametrize("ckv", CKV)
@pytest.mark.parametrize("dv,dk", [(512, 64), (64, 16)])
def test_norm_mode(ckv, dv, dk):
    say(f"[parity] norm mode Dv={dv} Dk={dk} {ckv}")
    case = gen.kvrc_norm_case(300 + dv, B=5, S=21, Dv=dv, Dk=dk, Bc=6, Sc=40, n_skip=9,
                              ckv_dtype=ckv)
    compare_kvrc(case, run_kvrc_gpu(case), oracle.run_kvrc_case(case), exact_bf16=True)


@pytest.mark.parametrize("B,S,Sc", [(4, 1, 3), (3, 7, 7), (2, 33, 50), (1, 5, 9)])
def test_norm_mode_sequence_lengths(B, S, Sc):
    """Token t belongs to batch t // S: lengths 1, odd and prime, and a cache
    row count equal to S."""
    say(f"[parity] norm mode B={B} S={S} Sc={Sc}")
    case = gen.kvrc_norm_case(330 + S, B=B, S=S, Dv=512, Dk=64, Bc=B + 1, Sc=Sc,
                              n_skip=min(2, B * S - 1))
    compare_kvrc(case, run_kvrc_gpu(case), oracle.run_kvrc_case(case), exact_bf16=True)


@pytest.mark.parametrize("sigma", [1e15, 1e-20, 1e-25, 3e-3])
@pytest.mark.parametrize("ckv", CKV)
def test_extreme_magnitudes(sigma, ckv):
    """Large rows, rows whose squares are float32 denormals, small rows."""
    say(f"[parity] sigma={sigma} {ckv}")
    case = gen.kvrc_paged_case(400, B=4, S=50, Dv=512, Dk=64, num_blocks=16, block_size=16,
                               slot_kind="random", sigma=sigma, ckv_dtype=ckv)
    compare_kvrc(case, run_kvrc_gpu(case), oracle.run_kvrc_case(case), exact_bf16=True)


@pytest.mark.parametrize("ckv", CKV)
def test_zero_rows_and_zero_eps(ckv):
    case = gen.kvrc_paged_case(401, B=2, S=40, Dv=512, Dk=64, num_blocks=8, block_size=16,
                               slot_kind="random", ckv_dtype=ckv)
    case["kv"][0, 0, :7] = 0                      # all-zero rows: amax 0 -> scale 0
    case["kv"][1, 0, 3, :100] = 0x8000            # negative zeros
    compare_kvrc(case, run_kvrc_gpu(case), oracle.run_kvrc_case(case), exact_bf16=True)
    case["eps"] = 0.0
    case["kv"][0, 0, :7] = gen.bf16_bits(np.ones((7, 576), np.float32))
    compare_kvrc(case, run_kvrc_gpu(case), oracle.run_kvrc_case(case), exact_bf16=True)


@pytest.mark.parametrize("ckv", CKV)
def test_subnormal_outputs_and_scales(ckv):
    """x ~ 2^-35 with eps = 1 (rms = 1) and gamma = 2^-107 put y near 2^-142:
    bf16 outputs are subnormal, and the int8 / E4M3FN scales RowMax/127 and
    RowMax/448 round to float32 subnormals (or to 0), so quotients pass 127
    or 448 in some rows and the codes saturate."""
    say(f"[parity] subnormal scales {ckv}")
    case = gen.kvrc_paged_case(407, B=4, S=64, Dv=512, Dk=64, num_blocks=16, block_size=32,
                               slot_kind="random", ckv_dtype=ckv)
    rng = gen.rng_for(408)
    x = rng.standard_normal((256, 576)).astype(np.float32) * np.float32(2.0 ** -35)
    x *= np.exp2(rng.uniform(-3, 3, (256, 1))).astype(np.float32)
    case["kv"] = gen.bf16_bits(x).reshape(4, 1, 64, 576)
    case["gamma"] = gen.bf16_bits(np.full(512, 2.0 ** -107, np.float32))
    case["eps"] = 1.0
    want = oracle.run_kvrc_case(case)
    if ckv != "bf16":
        sc = want["ckv_scale"].reshape(-1)[case["slot_mapping"][case["slot_mapping"] >= 0]]
        assert np.any((sc > 0) & (sc < np.float32(2.0 ** -126)))
    compare_kvrc(case, run_kvrc_gpu(case), want, exact_bf16=True)


def test_all_skipped_and_empty():
    case = gen.kvrc_paged_case(402, B=2, S=9, Dv=512, Dk=64, num_blocks=4, block_size=16,
                               slot_kind="random")
    case["slot_mapping"][:] = -1
    got = run_kvrc_gpu(case)
    for name, g in got.items():
        assert torch.equal(g.view(torch.int16) if g.dtype == torch.bfloat16 else g,
                           dbf(case["caches"][name].numpy()).view(torch.int16))
    empty = gen.kvrc_paged_case(403, B=0, S=9, Dv=512, Dk=64, num_blocks=4, block_size=16,
                                slot_kind="random")
    got = run_kvrc_gpu(empty)
    assert torch.all(got["k_cache"].view(torch.int16) == gen.BF16_SENTINEL)


@pytest.mark.parametrize("mode", ["paged", "norm"])
def test_invalid_indices_are_skipped_and_counted(mode):
    if mode == "paged":
        case = gen.kvrc_paged_case(404, B=3, S=20, Dv=512, Dk=64, num_blocks=8, block_size=16,
                                   slot_kind="random", skip_frac=0.1)
        idx = case["slot_mapping"].copy()
        limit = 8 * 16
        flat = idx
    else:
        case = gen.kvrc_norm_case(405, B=3, S=20, Dv=512, Dk=64, Bc=3, Sc=32, n_skip=5)
        idx = case["index"].copy()
        limit = 32
        flat = idx.reshape(-1)
    bad_pos = [1, 7, 30]
    flat[bad_pos[0]] = limit
    flat[bad_pos[1]] = -2
    flat[bad_pos[2]] = 1 << 40
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = run_kvrc_gpu(case, err=err, index_override=idx)
    assert int(err.item()) == 3
    clean = dict(case)
    fixed = idx.copy()
    fixed.reshape(-1)[bad_pos] = -1
    clean["slot_mapping" if mode == "paged" else "index"] = fixed
    compare_kvrc(clean, got, oracle.run_kvrc_case(clean), exact_bf16=True)


def test_async_on_caller_stream():
    """The launch goes to the given stream, ordered with the caller's work."""
    case = gen.kvrc_paged_case(406, B=4, S=64, Dv=512, Dk=64, num_blocks=16, block_size=32,
                               slot_kind="random")
    want = oracle.run_kvrc_case(case)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        kc = dbf(case["caches"]["k_cache"].numpy())
        ck = dbf(case["caches"]["ckv_cache"].numpy())
        kv = dbf(case["kv"])
        k.kvrc_paged_norm_rope_cache(kv, dbf(case["gamma"]), dbf(case["cos"]), dbf(case["sin"]),
                                     dt(case["slot_mapping"]), kc, ck, eps=case["eps"], stream=s)
    s.synchronize()
    compare_kvrc(case, {"k_cache": kc, "ckv_cache": ck}, want, exact_bf16=True)


# ---------------------------------------------------------------------------
# QSA
# ---------------------------------------------------------------------------

def run_qsa_gpu(case, err=None):
    N, Di, kbs, Dr = case["N"], case["Di"], case["kbs"], case["Dr"]
    rope = case["rope_cos"] is not None
    bk = dbf(case["caches"]["block_keys"].numpy())
    nraw = dbf(np.full((N, kbs - 1, Di), 0x7FC0, dtype=np.uint16))
    nrope = torch.full((N, 2 * Dr), float("nan"), device=DEV) if rope else None
    w = case["k_norm_weight"]
    k.qsa_prepare(dbf(case["raw_index_keys"]), bk, dt(case["key_length"]),
                  dt(case["rope_cos"]) if rope else None, dt(case["rope_sin"]) if rope else None,
                  dbf(w) if w is not None else None, dbf(case["past_incomplete_raw_keys"]),
                  dt(case["past_incomplete_rope"]) if rope else None, nraw, nrope,
                  key_block_size=kbs, eps=case["eps"], err_count=err)
    torch.cuda.synchronize()
    return bk, nraw, nrope


def compare_qsa(got, want, *, exact=False):
    bk, nraw, nrope = got
    wbk, wraw, wrope = want
    d = (ordered(bk) - ordered(dbf(wbk))).abs()
    m = int(d.max().item())
    assert m <= (0 if exact else 1), f"block keys: {m} bf16 ulps"
    # rows never written keep the sentinel exactly
    written = torch.from_numpy(wbk != gen.BF16_SENTINEL).to(DEV)
    assert torch.equal(bk.view(torch.int16)[~written],
                       torch.full_like(bk.view(torch.int16)[~written], gen.BF16_SENTINEL))
    assert torch.equal(nraw.view(torch.int16), dbf(wraw).view(torch.int16)), "carried rows"
    if wrope is not None:
        assert torch.equal(nrope.view(torch.int32), dt(wrope).view(torch.int32)), "carried rope"
    return m


def test_qsa_named_workload_full_size():
    say("[parity] workload qsa")
    case = gen.make_config("qsa")
    want = oracle.run_qsa_case(case)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    m = compare_qsa(run_qsa_gpu(case, err=err), want)
    assert int(err.item()) == 0
    say(f"[parity] qsa: max bf16 ulp {m}")


def test_qsa_named_workload_bit_exact():
    case = gen.make_config("qsa")
    compare_qsa(run_qsa_gpu(case), oracle.run_qsa_case(case), exact=True)


# Di = 128 with blocks of at most 64 rows runs on the one-wavefront kernel,
# every other shape on the general one.
@pytest.mark.parametrize("N,L,Di,Dr,kbs", [
    (4, 100, 128, 64, 16), (3, 7, 64, 16, 16), (5, 1, 32, 8, 4), (2, 300, 1024, 128, 24),
    (6, 65, 8, 2, 3), (1, 2048, 256, 256, 64), (3, 50, 136, 40, 2),
    (3, 130, 128, 128, 64), (2, 70, 128, 2, 33), (2, 90, 128, 64, 65),
    (1, 70, 4096, 64, 32),                                     # the largest Di accepted
    # one-wavefront kernel: the smallest block (one carried row at most),
    # blocks whose last load group is partial, the largest partial block
    (3, 150, 128, 64, 2), (2, 77, 128, 64, 5), (2, 200, 128, 32, 63),
])
@pytest.mark.parametrize("variant", ["full", "no_norm", "no_rope", "plain", "broadcast"])
def test_qsa_shapes_and_features(N, L, Di, Dr, kbs, variant):
    say(f"[parity] qsa N={N} L={L} Di={Di} Dr={Dr} kbs={kbs} {variant}")
    case = gen.qsa_case(500 + N + L + Di, N=N, L=L, Di=Di, Dr=Dr, kbs=kbs, past_max=3 * kbs + 5,
                        key_length_count=1 if variant == "broadcast" else None)
    if variant in ("no_norm", "plain"):
        case["k_norm_weight"] = None
    if variant in ("no_rope", "plain"):
        case["rope_cos"] = case["rope_sin"] = case["past_incomplete_rope"] = None
    compare_qsa(run_qsa_gpu(case), oracle.run_qsa_case(case), exact=True)


def test_qsa_more_blocks_than_the_chip_holds_at_once():
    """100 sequences x 2048 tokens on the one-wavefront kernel: 3300
    workgroups, more than are resident at once (16 KiB of LDS each, ten per
    compute unit), so compute units run several in turn on the same LDS."""
    say("[parity] qsa N=100 L=2048 Di=128 Dr=64 kbs=64")
    case = gen.qsa_case(620, N=100, L=2048, Di=128, Dr=64, kbs=64, past_max=8192)
    compare_qsa(run_qsa_gpu(case), oracle.run_qsa_case(case), exact=True)


def test_qsa_invalid_lengths_counted():
    case = gen.qsa_case(600, N=4, L=40, Di=64, Dr=16, kbs=8, past_max=30)
    kl = case["key_length"].copy()
    kl[1] = 10                                   # K < L
    kl[3] = 10_000                               # blocks past Bcap
    case["key_length"] = kl
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    bk, _, _ = run_qsa_gpu(case, err=err)
    assert int(err.item()) == 2
    assert torch.all(bk[1].view(torch.int16) == gen.BF16_SENTINEL)
    assert torch.all(bk[3].view(torch.int16) == gen.BF16_SENTINEL)


def test_qsa_invalid_lengths_counted_one_wavefront_kernel():
    """The same error rule on the Di = 128 kernel: a sequence with K < L or
    with blocks past Bcap writes nothing and counts once; the others are
    exact."""
    case = gen.qsa_case(601, N=4, L=70, Di=128, Dr=64, kbs=32, past_max=100)
    kl = case["key_length"].copy()
    kl[0] = 50                                   # K < L
    kl[2] = 100_000                              # blocks past Bcap
    case["key_length"] = kl
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    bk, _, _ = run_qsa_gpu(case, err=err)
    assert int(err.item()) == 2
    assert torch.all(bk[0].view(torch.int16) == gen.BF16_SENTINEL)
    assert torch.all(bk[2].view(torch.int16) == gen.BF16_SENTINEL)
    ok = [1, 3]
    sub = dict(case, N=2, raw_index_keys=case["raw_index_keys"][ok], key_length=kl[ok],
               rope_cos=case["rope_cos"][ok], rope_sin=case["rope_sin"][ok],
               past_incomplete_raw_keys=case["past_incomplete_raw_keys"][ok],
               past_incomplete_rope=case["past_incomplete_rope"][ok],
               caches={"block_keys": gen.CacheSpec((2,) + case["caches"]["block_keys"].shape[1:],
                                                   np.uint16, gen.BF16_SENTINEL)})
    want_bk, _, _ = oracle.run_qsa_case(sub)
    got = bk[ok].view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want_bk)


@pytest.mark.parametrize("seed,kbs", [(700, 16), (701, 16), (702, 64), (703, 5)])
def test_qsa_chained_calls_match_whole_history(seed, kbs):
    """Random chunking of each sequence's token stream across calls, with the
    state carried by the library itself, equals (bit for bit) the oracle's
    single call over the whole stream."""
    rng = gen.rng_for(seed)
    N, T, Di, Dr = 3, 400, 128, 64
    Bcap = T // kbs + 1
    raw = gen.bf16_bits(rng.standard_normal((N, T, Di)).astype(np.float32))
    pos = np.broadcast_to(np.arange(T), (N, T))
    rc, rs = gen.rope_table_f32(pos, Dr)
    w = gen.bf16_bits(rng.uniform(0.5, 1.5, Di).astype(np.float32))
    full = dict(raw_index_keys=raw, key_length=np.full(N, T, np.int64), rope_cos=rc, rope_sin=rs,
                k_norm_weight=w,
                past_incomplete_raw_keys=np.full((N, kbs - 1, Di), gen.BF16_NAN, np.uint16),
                past_incomplete_rope=np.full((N, 2 * Dr), np.nan, np.float32),
                caches={"block_keys": gen.CacheSpec((N, Bcap, Di), np.uint16, gen.BF16_SENTINEL)},
                N=N, L=T, Di=Di, Dr=Dr, kbs=kbs, Bcap=Bcap, eps=1e-6)
    want_bk, _, _ = oracle.run_qsa_case(full)
    bk = dbf(full["caches"]["block_keys"].numpy())
    st_raw = dbf(full["past_incomplete_raw_keys"])
    st_rope = dt(full["past_incomplete_rope"])
    done = 0
    while done < T:
        L = min(int(rng.choice([1, 3, kbs - 1, kbs, kbs + 1, 5 * kbs + 3])), T - done)
        nraw = dbf(np.full((N, kbs - 1, Di), gen.BF16_NAN, np.uint16))
        nrope = torch.full((N, 2 * Dr), float("nan"), device=DEV)
        k.qsa_prepare(dbf(raw[:, done:done + L]), bk, dt(np.full(N, done + L, np.int64)),
                      dt(rc[:, done:done + L]), dt(rs[:, done:done + L]), dbf(w), st_raw, st_rope,
                      nraw, nrope, key_block_size=kbs, eps=1e-6)
        st_raw, st_rope = nraw, nrope
        done += L
    torch.cuda.synchronize()
    assert torch.equal(bk.view(torch.int16), dbf(want_bk).view(torch.int16))


def test_qsa_graph_replays_match_the_oracle():
    """QSAPrepare captured in a HIP graph: every replay, with the outputs reset
    eagerly in between, writes the block keys and the next carry state the
    oracle gives, bit for bit."""
    case = gen.qsa_case(630, N=6, L=300, Di=128, Dr=64, kbs=64, past_max=500)
    want = oracle.run_qsa_case(case)
    N, Di, kbs, Dr = case["N"], case["Di"], case["kbs"], case["Dr"]
    ins = (dbf(case["raw_index_keys"]), None, dt(case["key_length"]), dt(case["rope_cos"]),
           dt(case["rope_sin"]), dbf(case["k_norm_weight"]), dbf(case["past_incomplete_raw_keys"]),
           dt(case["past_incomplete_rope"]))
    bk = dbf(case["caches"]["block_keys"].numpy())
    nraw = dbf(np.full((N, kbs - 1, Di), 0x7FC0, dtype=np.uint16))
    nrope = torch.full((N, 2 * Dr), float("nan"), device=DEV)

    def call():
        k.qsa_prepare(ins[0], bk, *ins[2:], nraw, nrope, key_block_size=kbs, eps=case["eps"])

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for rep in range(4):
        bk.view(torch.int16).fill_(gen.BF16_SENTINEL)       # eager reset between replays
        nraw.view(torch.int16).fill_(0x7FC0)
        nrope.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        compare_qsa((bk, nraw, nrope), want, exact=True)


def test_graph_replays_match_eager():
    """The bench replays captured launches: every replay, with eager work and
    synchronisation in between, must give the eager (oracle-equal) result."""
    case = gen.kvrc_paged_case(800, B=2, S=300, Dv=512, Dk=64, num_blocks=16, block_size=64,
                               slot_kind="random", skip_frac=0.05, ckv_dtype="int8")
    want = oracle.run_kvrc_case(case)
    ins = (dbf(case["kv"]), dbf(case["gamma"]), dbf(case["cos"]), dbf(case["sin"]),
           dt(case["slot_mapping"]))
    kc = dbf(case["caches"]["k_cache"].numpy())
    ck = dt(case["caches"]["ckv_cache"].numpy())
    sc = dt(case["caches"]["ckv_scale"].numpy())
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        k.kvrc_paged_norm_rope_cache(*ins, kc, ck, sc, eps=case["eps"])
    s.synchronize()
    with torch.cuda.graph(g, stream=s):
        k.kvrc_paged_norm_rope_cache(*ins, kc, ck, sc, eps=case["eps"])
    for rep in range(4):
        kc.view(torch.int16).fill_(gen.BF16_SENTINEL)      # eager reset between replays
        ck.fill_(gen.INT8_SENTINEL)
        sc.fill_(gen.SCALE_SENTINEL)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        compare_kvrc(case, {"k_cache": kc, "ckv_cache": ck, "ckv_scale": sc}, want,
                     exact_bf16=True)


@pytest.mark.parametrize("ckv", CKV)
@pytest.mark.parametrize("T", [96, 4096])
@pytest.mark.parametrize("span", ["over_4gib", "3gib"])
def test_large_cache_offsets(ckv, T, span):
    """Caches of 4 GiB or more take the plain-global-store path (with both the
    small-batch and the large-batch launch shapes): rows beyond the 32-bit
    byte offset must land exactly. A 3 GiB cache takes the buffer stores,
    whose 32-bit offsets pass 2^31 there: rows beyond 2 GiB must land too.
    Nothing else may change."""
    Dv, Dk, BS = 512, 64, 128
    row_bytes = Dv * (2 if ckv == "bf16" else 1)
    if span == "over_4gib":
        split = 2 ** 32 // row_bytes                          # first row past the 4 GiB offset
        NB = split // BS + 64                                 # just over 4 GiB of ckv rows
    else:
        split = 2 ** 31 // row_bytes                          # first row past the 2 GiB offset
        NB = (3 * 2 ** 30 // row_bytes) // BS                 # 3 GiB of ckv rows
    say(f"[parity] large cache ({span}): {ckv}, {NB} blocks, {T} tokens")
    small = gen.kvrc_paged_case(900, B=2, S=T // 2, Dv=Dv, Dk=Dk, num_blocks=1, block_size=T,
                                slot_kind="random", ckv_dtype=ckv)
    # real slots: half below the split offset, half above it
    rng = gen.rng_for(901)
    lo = rng.choice(split - 1, size=T // 2, replace=False)
    hi = split + rng.choice(NB * BS - split, size=T // 2, replace=False)
    slots = np.concatenate([lo, hi]).astype(np.int64)
    rng.shuffle(slots)
    want = oracle.run_kvrc_case(small)                        # slot t -> compact row small[t]
    compact = small["slot_mapping"]
    caches = {"k_cache": torch.full((NB, BS, 1, Dk), gen.BF16_SENTINEL, dtype=torch.int16,
                                    device=DEV).view(torch.bfloat16)}
    if ckv == "bf16":
        caches["ckv_cache"] = torch.full((NB, BS, 1, Dv), gen.BF16_SENTINEL, dtype=torch.int16,
                                         device=DEV).view(torch.bfloat16)
        scale = None
    else:
        caches["ckv_cache"] = torch.from_numpy(gen.ckv_cache_spec((1,), ckv).numpy()).to(DEV) \
            .expand(NB, BS, 1, Dv).contiguous()
        scale = torch.full((NB, BS, 1), gen.SCALE_SENTINEL, dtype=torch.float32, device=DEV)
    ckv_sentinel = gen.ckv_cache_spec((1,), ckv).fill
    k.kvrc_paged_norm_rope_cache(dbf(small["kv"]), dbf(small["gamma"]), dbf(small["cos"]),
                                 dbf(small["sin"]), dt(slots), caches["k_cache"],
                                 caches["ckv_cache"], scale, eps=small["eps"])
    torch.cuda.synchronize()
    idx = torch.from_numpy(slots).to(DEV)
    for name, d in (("k_cache", Dk), ("ckv_cache", Dv)):
        g = caches[name].view(NB * BS, d)
        w = want[name].reshape(-1, d)[compact]
        if g.dtype == torch.bfloat16:
            assert torch.equal(g[idx].view(torch.int16), dbf(w).view(torch.int16)), name
            sentinel = gen.BF16_SENTINEL
            changed = int((g.view(torch.int16) != sentinel).sum().item())
            in_rows = int((g[idx].view(torch.int16) != sentinel).sum().item())
        else:
            assert torch.equal(g[idx], dt(w)), name
            changed = int((g != ckv_sentinel).sum().item())
            in_rows = int((g[idx] != ckv_sentinel).sum().item())
        assert changed == in_rows, f"{name}: bytes outside the written rows changed"
    if scale is not None:
        sv = scale.view(-1)
        assert torch.equal(sv[idx], dt(want["ckv_scale"].reshape(-1)[compact]))
        assert int((sv != gen.SCALE_SENTINEL).sum().item()) == int((sv[idx] != gen.SCALE_SENTINEL).sum().item())


def test_int8_exact_ties():
    """Rows whose quotients y/scale are exact half-integers: eps is chosen so
    that mean(x^2) + eps = 64^2 (rms = 64 exactly), gamma = 1, max|x| = 127,
    hence y = x/64, scale = 1/64 and y/scale = x; codes must be
    rint half-to-even(x). (All squares are multiples of 1/4 and the sums stay
    below 2^21, so every partial sum is exact in float32.)"""
    rng = gen.rng_for(950)
    Dv, Dk, T = 512, 64, 64
    base = np.zeros(Dv, np.float32)
    base[0] = 127.0
    halves = np.arange(-126.5, 127.0, 1.0, dtype=np.float32)       # -126.5 .. 126.5
    base[1:1 + 180] = rng.choice(halves, 180, replace=False)
    ss = float(np.sum(base.astype(np.float64) ** 2))
    ms = np.float32(ss / Dv)
    assert float(ms) * Dv == ss and ms < 4096
    eps = float(np.float32(4096.0) - ms)
    assert np.float32(ms + np.float32(eps)) == 4096.0
    rows = np.stack([rng.permutation(base) for _ in range(T)])
    kv = np.concatenate([rows, rng.standard_normal((T, Dk)).astype(np.float32)], axis=1)
    case = gen.kvrc_paged_case(951, B=1, S=T, Dv=Dv, Dk=Dk, num_blocks=4, block_size=32,
                               slot_kind="random", ckv_dtype="int8")
    case["kv"] = gen.bf16_bits(kv).reshape(1, 1, T, Dv + Dk)
    case["gamma"] = gen.bf16_bits(np.ones(Dv, np.float32))
    case["eps"] = eps
    want = oracle.run_kvrc_case(case)
    got = run_kvrc_gpu(case)
    compare_kvrc(case, got, want, exact_bf16=True)
    slots = case["slot_mapping"]
    codes = got["ckv_cache"].cpu().numpy().reshape(-1, Dv)[slots]
    np.testing.assert_array_equal(codes, np.rint(rows).astype(np.int8))     # rint: half to even
    assert np.all(got["ckv_scale"].cpu().numpy().reshape(-1)[slots] == np.float32(1 / 64))



def test_fp8_exact_ties():
    """Rows whose quotients y/scale are exact midpoints between neighbouring
    E4M3FN values: eps makes mean(x^2) + eps = 64^2 (rms = 64 exactly),
    gamma = 1 and max|x| = 448, hence y = x/64, scale = 7/448 = 1/64 and
    y/scale = x; each midpoint must take the even code. (All squares are
    multiples of 1/4 and the sums stay below 2^21, so every partial sum is
    exact in float32.)"""
    rng = gen.rng_for(952)
    Dv, Dk, T = 512, 64, 64
    mids = [k + 0.5 for k in range(8, 16)] + list(range(17, 32, 2)) + list(range(34, 64, 4)) + \
        list(range(68, 128, 8)) + list(range(136, 256, 16))
    vals = np.array(mids + [-m for m in mids] + list(range(272, 448, 32)), np.float32)
    base = np.zeros(Dv, np.float32)
    base[0] = 448.0
    base[1:1 + len(vals)] = vals
    ss = float(np.sum(base.astype(np.float64) ** 2))
    ms = np.float32(ss / Dv)
    assert ss < 2.0 ** 21 and float(ms) * Dv == ss and ms < 4096
    eps = float(np.float32(4096.0) - ms)
    assert np.float32(ms + np.float32(eps)) == 4096.0
    rows = np.stack([rng.permutation(base) for _ in range(T)])
    kv = np.concatenate([rows, rng.standard_normal((T, Dk)).astype(np.float32)], axis=1)
    case = gen.kvrc_paged_case(953, B=1, S=T, Dv=Dv, Dk=Dk, num_blocks=4, block_size=32,
                               slot_kind="random", ckv_dtype="fp8")
    case["kv"] = gen.bf16_bits(kv).reshape(1, 1, T, Dv + Dk)
    assert np.array_equal(gen.bits_to_f32(case["kv"]).reshape(T, -1)[:, :Dv], rows)
    case["gamma"] = gen.bf16_bits(np.ones(Dv, np.float32))
    case["eps"] = eps
    want = oracle.run_kvrc_case(case)
    got = run_kvrc_gpu(case)
    compare_kvrc(case, got, want, exact_bf16=True)
    slots = case["slot_mapping"]
    codes = got["ckv_cache"].cpu().numpy().reshape(-1, Dv)[slots]
    np.testing.assert_array_equal(codes, oracle.e4m3_encode_array(rows.reshape(-1)).reshape(T, Dv))
    assert np.all(codes[rows == 8.5] == 0x50) and np.all(codes[rows == 17.0] == 0x58)
    assert np.all(got["ckv_scale"].cpu().numpy().reshape(-1)[slots] == np.float32(1 / 64))


@pytest.mark.parametrize("ckv", CKV)
@pytest.mark.parametrize("B,S,BS,offsets", [(8, 4096, 128, False), (3, 300, 64, True),
                                             (2, 37, 16, False), (5, 1, 16, False),
                                             (2, 13, 1, False), (4, 97, 7, True),
                                             (3, 1000, 999, True), (3, 50, 1000, True)])
def test_paged_blk_mode(ckv, B, S, BS, offsets):
    """Block-indexed mode (PA_BLK_BNSD): one entry per chunk of BS tokens,
    ragged last chunks, skipped chunks, entries with offsets inside the block."""
    say(f"[parity] paged blk {ckv} B={B} S={S} BS={BS}")
    chunks = B * (-(-S // BS))
    case = gen.kvrc_paged_blk_case(960 + S, B=B, S=S, Dv=512, Dk=64,
                                   num_blocks=max(2 * chunks, 64), block_size=BS, ckv_dtype=ckv,
                                   n_skip=min(2, chunks - 1), entry_offsets=offsets)
    compare_kvrc(case, run_kvrc_gpu(case), oracle.run_kvrc_case(case), exact_bf16=True)


def test_paged_blk_named_workload_and_invalid_entries():
    case = gen.make_config("prefill_paged_blk")
    compare_kvrc(case, run_kvrc_gpu(case), oracle.run_kvrc_case(case), exact_bf16=True)
    small = gen.kvrc_paged_blk_case(970, B=2, S=100, Dv=512, Dk=64, num_blocks=16,
                                    block_size=32)
    idx = small["block_index"].copy()
    idx[1] = 16 * 32                   # out of range: its 32 tokens are skipped and counted
    idx[3] = -7                        # out of range: batch 0's last chunk has 100 - 96 = 4 tokens
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = run_kvrc_gpu(small, err=err, index_override=idx)
    assert int(err.item()) == 32 + 4
    fixed = idx.copy()
    fixed[[1, 3]] = -1
    clean = dict(small, block_index=fixed)
    compare_kvrc(clean, got, oracle.run_kvrc_case(clean), exact_bf16=True)


# Above 2048 tokens the Dv = 512 / Dk = 64 kernel runs two rows per wavefront
# in 256-thread workgroups (8 rows per workgroup). Token counts that are not a
# multiple of 8 leave the last workgroup partial: its last wavefront may hold
# one row, whose upper 32 lanes exit before the lower half folds its sums and
# maxima over 32 lanes. Odd sequence lengths put batch boundaries inside
# workgroups and wavefronts.
RAGGED_LARGE = [(1, 2049), (2, 1025), (5, 411), (17, 241), (7, 4681), (15, 4369)]


_RAGGED_BASE = {}


def _ragged_case(mode, B, S, ckv):
    """The inputs depend on (mode, B, S) only; the ckv cache type changes the
    caches alone, so the drawn inputs are shared across the three types."""
    key = (mode, B, S)
    if key not in _RAGGED_BASE:
        _RAGGED_BASE.clear()
        T = B * S
        seed = 1000 + T
        if mode == "paged":
            bs = 128
            base = gen.kvrc_paged_case(seed, B=B, S=S, Dv=512, Dk=64,
                                       num_blocks=-(-T // bs) + 8, block_size=bs,
                                       slot_kind="random", skip_frac=0.03)
        elif mode == "paged_blk":
            bs = 64
            base = gen.kvrc_paged_blk_case(seed, B=B, S=S, Dv=512, Dk=64,
                                           num_blocks=B * -(-S // bs) + 5, block_size=bs,
                                           n_skip=1, entry_offsets=True)
        else:
            base = gen.kvrc_norm_case(seed, B=B, S=S, Dv=512, Dk=64, Bc=B, Sc=S + 3,
                                      n_skip=max(1, T // 50))
        _RAGGED_BASE[key] = base
    base = _RAGGED_BASE[key]
    case = dict(base, ckv_dtype=ckv)
    rows = base["caches"]["ckv_cache"].shape
    case["caches"] = {"k_cache": base["caches"]["k_cache"],
                      "ckv_cache": gen.ckv_cache_spec(rows, ckv)}
    if ckv != "bf16":
        case["caches"]["ckv_scale"] = gen.CacheSpec(rows[:-1], np.float32, gen.SCALE_SENTINEL)
    return case


@pytest.mark.parametrize("ckv", CKV)
@pytest.mark.parametrize("B,S", RAGGED_LARGE)
@pytest.mark.parametrize("mode", ["paged", "paged_blk", "norm"])
def test_large_batch_ragged_tail(ckv, B, S, mode):
    T = B * S
    assert T > 2048 and T % 8
    say(f"[parity] large-batch ragged tail: {mode} {ckv} B={B} S={S} T={T}")
    case = _ragged_case(mode, B, S, ckv)
    want = oracle.run_kvrc_case(case)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = run_kvrc_gpu(case, err=err)
    compare_kvrc(case, got, want, exact_bf16=True)
    assert int(err.item()) == 0
    del got, want
