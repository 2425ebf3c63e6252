"""GPU parity of the MLA kv-path head (kvrc_mla_kv_head_paged) against the
float64 oracle (oracle/mla_kv_head.py) on the same seeded inputs.

The projection runs on the matrix cores with float32 accumulation in an order
of its own, so the bar is derived from the arithmetic instead of bit
equality. With He products per output, each exact (bf16 x bf16), any float32
summation order (round to nearest or toward zero) keeps
    |c_gpu - c| <= e = 2 He u / (1 - He u) * sum_k |x_k w_k|,   u = 2^-24;
propagated through the mean square (512 float32 squares and adds), the
square root and the division, the scaling by alpha * gamma and the RoPE
products, it bounds |y_gpu - y| by dy; the bf16 output then lies within
dy + 1/2 bf16 ulp of the float64 value. Every written element must meet that
bound, and, because the bound is loose (it allows for worst-case cancellation
in the sums), at least 99.5 % of the outputs must equal the float64 value
rounded to bf16 (a correct float32 path misses it only where its error of
about 1e-6 relative straddles a bf16 rounding boundary). Placement and every
byte no token addresses: bit-exact.

A quantised ckv cache (int8 codes with scale RowMax/127, E4M3FN codes with
RowMax/448) is held to the same dy: with dA the largest dy of the row, the
quotient t = y * d / RowMax the kernel rounds lies within
    dt = (dy * d / RowMax + |t| * dA / RowMax) * 1.01 + 4 u |t|
of the float64 one, so its code must lie between the codes of t - dt and
t + dt (rounding is monotone), the scale within dA / d * 1.01 + 8 u scale
(the kernel takes the row maximum before the norm and scales it: a few
roundings more than the maximum of its rounded y);
each row's largest code is exactly 127 (448), a zero row stores scale 0 and
code bytes 0, and at least 99.5 % of the codes equal the float64 oracle's.
"""
import numpy as np
import pytest
import torch

import gen
import latent_attention_kv_amd as k
from oracle import mla_kv_head as M

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


def new_workspace(T):
    return torch.zeros(max(1, k.kvrc_mla_kv_head_workspace_bytes(T)), dtype=torch.uint8,
                       device=DEV)


def dev_cache(arr):
    """Device copy of a cache array: bf16 bits (uint16), int8 or E4M3FN codes
    (uint8), float32 scales."""
    if arr.dtype == np.uint16:
        return dbf(arr)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


def host_cache(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def run_mla_gpu(case, slots=None, err=None, workspace=None):
    """One call; the workspace (fresh unless given) must be all zero again
    afterwards."""
    caches = {n: dev_cache(spec.numpy()) for n, spec in case["caches"].items()}
    slots = case["slot_mapping"] if slots is None else slots
    T = case["x"].shape[0]
    ws = new_workspace(T) if workspace is None else workspace
    k.kvrc_mla_kv_head_paged(dbf(case["x"]), dbf(case["w"]), dbf(case["gamma"]), dbf(case["cos"]),
                             dbf(case["sin"]), torch.from_numpy(slots).to(DEV),
                             caches["k_cache"], caches["ckv_cache"], caches.get("ckv_scale"),
                             workspace=ws, alpha_kv=case["alpha"], eps=case["eps"],
                             err_count=err)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws)) == 0, "workspace not left zero"
    return {n: host_cache(t) for n, t in caches.items()}


def ulp_bf16(v):
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def head_bounds(case):
    """float64 outputs (oracle) and the per-element bounds dy, dk on the
    float32 values of the kernel before any rounding of the outputs."""
    y, kr = M.kv_head_rows(case["x"], case["w"], case["gamma"], case["alpha"], case["cos"],
                           case["sin"], case["eps"])
    X, W = M.bf16_to_f64(case["x"]), M.bf16_to_f64(case["w"])
    C = X @ W.T
    A = np.abs(X) @ np.abs(W).T
    He = X.shape[1]
    e = (2 * He * U / (1 - He * U)) * A
    cv, ev = C[:, :512], e[:, :512]
    ssq = np.sum(cv * cv, axis=1)
    dss = np.sum(2 * np.abs(cv) * ev + ev * ev, axis=1) + 520 * U * np.sum((np.abs(cv) + ev) ** 2, axis=1)
    ms = ssq / 512
    den = ms + case["eps"]
    drel = np.divide(dss / 512, 2 * den, out=np.full_like(den, np.inf), where=den > 0) + 4 * U
    rms = np.sqrt(den)
    g = np.abs(M.bf16_to_f64(case["gamma"]))[None, :]
    a = abs(case["alpha"])
    with np.errstate(divide="ignore", invalid="ignore"):
        dy = a * g * (ev / rms[:, None] + np.abs(cv) / rms[:, None] * drel[:, None]) * 1.01 \
            + 4 * U * np.abs(y)
    r, er = C[:, 512:], e[:, 512:]
    cs, sn = np.abs(M.bf16_to_f64(case["cos"])), np.abs(M.bf16_to_f64(case["sin"]))
    ev_, od_ = np.concatenate([er[:, 0::2], er[:, 1::2]], 1), np.concatenate([er[:, 1::2], er[:, 0::2]], 1)
    rv_, ro_ = np.concatenate([r[:, 0::2], r[:, 1::2]], 1), np.concatenate([r[:, 1::2], r[:, 0::2]], 1)
    dk = (cs * ev_ + sn * od_) * 1.01 + 3 * U * (np.abs(rv_) * cs + np.abs(ro_) * sn)
    return y, kr, dy, dk


def compare_quant(kind, codes, scales, y, dy):
    """Quantised rows (codes [n, 512], scales [n]) against the float64 rows y
    with bounds dy; returns the fraction of codes equal to the oracle's."""
    d = 127.0 if kind == "int8" else 448.0
    amax = np.max(np.abs(y), axis=1)
    dA = np.max(dy, axis=1)
    zero = amax == 0
    assert np.all(scales[zero] == 0) and np.all(codes[zero].view(np.uint8) == 0), \
        "zero rows must store scale 0 and code bytes 0"
    nz = ~zero
    y, dy, amax, dA, codes, scales = y[nz], dy[nz], amax[nz], dA[nz], codes[nz], scales[nz]
    want_s = amax / d
    bad = ~(np.abs(scales.astype(np.float64) - want_s) <= dA / d * 1.01 + 8 * U * want_s)
    assert not bad.any(), f"{int(bad.sum())} scales beyond the bound"
    t = y * (d / amax)[:, None]
    dt = (dy * (d / amax)[:, None] + np.abs(t) * (dA / amax)[:, None]) * 1.01 + 4 * U * np.abs(t)
    if kind == "int8":
        rnd = lambda v: np.rint(np.clip(v, -d, d))
        gv = codes.astype(np.float64)
    else:
        rnd = lambda v: M.e4m3_round(np.clip(v, -d, d))
        gv = M.e4m3_decode(codes.view(np.uint8))
    bad = ~((rnd(t - dt) <= gv) & (gv <= rnd(t + dt)))
    if bad.any():
        i = np.argwhere(bad)[0]
        pytest.fail(f"{int(bad.sum())} codes beyond the bound, e.g. row {i[0]} col {i[1]}: "
                    f"gpu {gv[tuple(i)]!r} want {rnd(t)[tuple(i)]!r} (t {t[tuple(i)]!r} +- "
                    f"{dt[tuple(i)]!r})")
    assert np.all(np.max(np.abs(gv), axis=1) == d), "a row's largest code must be the maximum"
    q, _ = M.quantize_rows(y, kind)
    want = q.astype(np.int8) if kind == "int8" else M.e4m3_encode(q)
    equal = int(np.sum(codes.view(np.uint8) == want.view(np.uint8)))
    assert codes.size - equal <= max(3, int(0.005 * codes.size)), \
        f"only {equal / codes.size:.5f} of the codes equal the oracle's"
    return equal / codes.size if codes.size else 1.0


def compare_mla(case, got, slots=None, bounds=None):
    """Returns (fraction of outputs equal to the rounded float64 value, worst
    error / bound)."""
    slots = case["slot_mapping"] if slots is None else slots
    kind = case.get("ckv_dtype", "bf16")
    y, kr, dy, dk = head_bounds(case) if bounds is None else bounds
    tol_k = dk + 0.5 * ulp_bf16(np.abs(kr) + dk)
    ck, kc = got["ckv_cache"].reshape(-1, 512), got["k_cache"].reshape(-1, 64)
    t_idx = np.flatnonzero(slots >= 0)
    rows = slots[t_idx]
    checks = [(kc[rows], kr[t_idx], tol_k[t_idx])]
    if kind == "bf16":
        tol_y = dy + 0.5 * ulp_bf16(np.abs(y) + dy)
        checks.insert(0, (ck[rows], y[t_idx], tol_y[t_idx]))
    equal, total, worst = 0, 0, 0.0
    for gbits, want, tol in checks:
        gv = M.bf16_to_f64(gbits)
        err = np.abs(gv - want)
        bad = ~(err <= tol)
        if bad.any():
            i = np.argwhere(bad)[0]
            pytest.fail(f"{int(bad.sum())} outputs beyond the bound, e.g. token "
                        f"{t_idx[i[0]]} col {i[1]}: gpu {gv[tuple(i)]!r} want {want[tuple(i)]!r} "
                        f"bound {tol[tuple(i)]!r}")
        worst = max(worst, float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0)
        wbits = M.f64_to_bf16(want)
        same = (gbits == wbits) | (((gbits & 0x7FFF) == 0) & ((wbits & 0x7FFF) == 0))
        equal += int(np.sum(same))
        total += gbits.size
    frac = equal / max(total, 1)
    assert total - equal <= max(3, int(0.005 * total)), \
        f"only {frac:.5f} of the outputs equal the float64 value rounded to bf16"
    untouched = np.setdiff1d(np.arange(ck.shape[0]), rows)
    sentinel = {"bf16": gen.BF16_SENTINEL, "int8": gen.INT8_SENTINEL, "fp8": gen.FP8_SENTINEL}[kind]
    assert np.all(ck[untouched] == sentinel) and np.all(kc[untouched] == gen.BF16_SENTINEL), \
        "bytes outside the written rows changed"
    if kind != "bf16":
        sc = got["ckv_scale"].reshape(-1)
        assert np.all(sc[untouched] == gen.SCALE_SENTINEL), "scales outside the written rows changed"
        frac = compare_quant(kind, ck[rows], sc[rows], y[t_idx], dy[t_idx])
    return frac, worst


def test_mla_named_workload_full_size():
    say("[mla] workload mla_kv_head (T=32768, He=7168)")
    case = gen.make_config("mla_kv_head")
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = run_mla_gpu(case, err=err)
    assert int(err.item()) == 0
    frac, worst = compare_mla(case, got)
    say(f"[mla] equal to the rounded float64 value: {frac:.6f}; worst error / bound {worst:.3f}")


@pytest.mark.parametrize("B,S,He", [(1, 1, 32), (1, 5, 64), (2, 100, 96), (1, 129, 512),
                                    (3, 257, 1024), (2, 300, 7168), (1, 128, 2048),
                                    (1, 70, 16384)])
def test_mla_shapes_and_ragged_tails(B, S, He):
    say(f"[mla] B={B} S={S} He={He}")
    case = gen.mla_kv_head_case(500 + S + He, B=B, S=S, He=He, num_blocks=64, block_size=32,
                                slot_kind="random", skip_frac=0.1)
    frac, worst = compare_mla(case, run_mla_gpu(case))
    say(f"[mla] equal fraction {frac:.5f}, worst error / bound {worst:.3f}")


@pytest.mark.parametrize("alpha,eps,x_sigma", [(0.0, 1e-6, 1.0), (-1.5, 1e-6, 1.0),
                                               (3.0, 1.0, 1.0), (1.0, 1e-6, 1e-3),
                                               (1.0, 1e-6, 300.0)])
def test_mla_alpha_eps_magnitudes(alpha, eps, x_sigma):
    say(f"[mla] alpha={alpha} eps={eps} x_sigma={x_sigma}")
    case = gen.mla_kv_head_case(520, B=2, S=200, He=1024, num_blocks=32, block_size=32,
                                slot_kind="random", alpha=alpha, eps=eps, x_sigma=x_sigma)
    compare_mla(case, run_mla_gpu(case))


def test_mla_zero_rows():
    case = gen.mla_kv_head_case(521, B=1, S=150, He=512, num_blocks=16, block_size=16,
                                slot_kind="random")
    case["x"][:7] = 0
    case["x"][140:] = 0x8000                       # negative zeros
    compare_mla(case, run_mla_gpu(case))


def test_mla_invalid_slots_are_skipped_and_counted():
    case = gen.mla_kv_head_case(522, B=1, S=300, He=256, num_blocks=32, block_size=16,
                                slot_kind="random", skip_frac=0.05)
    slots = case["slot_mapping"].copy()
    slots[[3, 130, 299]] = [32 * 16, -2, 1 << 40]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = run_mla_gpu(case, slots=slots, err=err)
    assert int(err.item()) == 3
    fixed = slots.copy()
    fixed[[3, 130, 299]] = -1
    compare_mla(case, got, slots=fixed)


def test_mla_deterministic_across_launch_sizes():
    """A token's outputs do not depend on T or on its position in the batch
    (same He): the first 130 tokens of a batch equal the same tokens alone."""
    case = gen.mla_kv_head_case(523, B=1, S=400, He=1024, num_blocks=32, block_size=16,
                                slot_kind="random")
    full = run_mla_gpu(case)
    part = dict(case, x=case["x"][:130], cos=case["cos"][:130], sin=case["sin"][:130],
                slot_mapping=case["slot_mapping"][:130], T=130, S=130)
    sub = run_mla_gpu(part)
    rows = case["slot_mapping"][:130]
    np.testing.assert_array_equal(full["ckv_cache"].reshape(-1, 512)[rows],
                                  sub["ckv_cache"].reshape(-1, 512)[rows])
    np.testing.assert_array_equal(full["k_cache"].reshape(-1, 64)[rows],
                                  sub["k_cache"].reshape(-1, 64)[rows])


@pytest.mark.parametrize("S", [255, 256, 257, 2049, 2305])
def test_mla_pair_boundaries(S):
    """256 rows per pair of workgroups, pairs in groups of 8: partial pairs,
    a padded grid and a ragged last pair."""
    say(f"[mla] pair boundaries T={S}")
    case = gen.mla_kv_head_case(530 + S, B=1, S=S, He=64, num_blocks=160, block_size=16,
                                slot_kind="random", skip_frac=0.05)
    compare_mla(case, run_mla_gpu(case))


def test_mla_many_pairs_beyond_one_dispatch_wave():
    """More workgroups than the chip holds at once (640 pairs): pairs start
    while earlier ones still run; no wait times out (err stays 0)."""
    say("[mla] T=163840 (1280 workgroups)")
    case = gen.mla_kv_head_case(540, B=4, S=40960, He=64, num_blocks=1400, block_size=128,
                                slot_kind="random", skip_frac=0.01)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    compare_mla(case, run_mla_gpu(case, err=err))
    assert int(err.item()) == 0


def test_mla_workspace_reused_across_calls_and_graph_replays():
    """One workspace for consecutive calls and for replays of a captured
    graph (eager work in between): every result equals the eager call's and
    the workspace ends zero each time."""
    say("[mla] workspace reuse and graph replays")
    a = gen.mla_kv_head_case(550, B=1, S=600, He=256, num_blocks=64, block_size=16,
                             slot_kind="random")
    b = gen.mla_kv_head_case(551, B=1, S=600, He=256, num_blocks=64, block_size=16,
                             slot_kind="random")
    ws = new_workspace(600)
    got_a = run_mla_gpu(a, workspace=ws)
    got_b = run_mla_gpu(b, workspace=ws)
    compare_mla(a, got_a)
    compare_mla(b, got_b)

    x, w, gm = dbf(a["x"]), dbf(a["w"]), dbf(a["gamma"])
    cs, sn = dbf(a["cos"]), dbf(a["sin"])
    sl = torch.from_numpy(a["slot_mapping"]).to(DEV)
    kc = dbf(a["caches"]["k_cache"].numpy())
    ck = dbf(a["caches"]["ckv_cache"].numpy())
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        k.kvrc_mla_kv_head_paged(x, w, gm, cs, sn, sl, kc, ck, workspace=ws,
                                 alpha_kv=a["alpha"], eps=a["eps"], stream=stream)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        k.kvrc_mla_kv_head_paged(x, w, gm, cs, sn, sl, kc, ck, workspace=ws,
                                 alpha_kv=a["alpha"], eps=a["eps"], stream=stream)
    want_k = got_a["k_cache"]
    want_c = got_a["ckv_cache"]
    sentinel = int(np.array([gen.BF16_SENTINEL], dtype=np.uint16).view(np.int16)[0])
    for rep in range(3):
        kc.view(torch.int16).fill_(sentinel)
        ck.view(torch.int16).fill_(sentinel)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        stream.synchronize()
        assert int(torch.count_nonzero(ws)) == 0, f"replay {rep}: workspace not left zero"
        np.testing.assert_array_equal(kc.view(torch.int16).cpu().numpy().view(np.uint16), want_k)
        np.testing.assert_array_equal(ck.view(torch.int16).cpu().numpy().view(np.uint16), want_c)


def test_mla_workspace_too_small_is_rejected():
    case = gen.mla_kv_head_case(552, B=1, S=300, He=64, num_blocks=32, block_size=16,
                                slot_kind="random")
    need = k.kvrc_mla_kv_head_workspace_bytes(300)
    ws = torch.zeros(need - 8, dtype=torch.uint8, device=DEV)
    caches = {n: dbf(spec.numpy()) for n, spec in case["caches"].items()}
    with pytest.raises(k.KvrcError):
        k.kvrc_mla_kv_head_paged(dbf(case["x"]), dbf(case["w"]), dbf(case["gamma"]),
                                 dbf(case["cos"]), dbf(case["sin"]),
                                 torch.from_numpy(case["slot_mapping"]).to(DEV),
                                 caches["k_cache"], caches["ckv_cache"], workspace=ws)
    torch.cuda.synchronize()
    assert np.all(caches["ckv_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
                  == gen.BF16_SENTINEL)


@pytest.mark.parametrize("span", ["over_4gib", "3gib"])
def test_mla_large_cache_offsets(span):
    """Caches of 4 GiB or more take the plain-store path of the scatter (the
    sc1 buffer stores need 32-bit offsets): rows beyond the 32-bit byte
    offset land exactly. A 3 GiB cache takes the buffer stores, whose offsets
    pass 2^31 there: rows beyond 2 GiB land too. Nothing else in the caches
    changes."""
    T, He, BS = 300, 256, 128
    if span == "over_4gib":
        rows_4g = 2 ** 32 // 1024                              # ckv rows below the 4 GiB offset
        NB = rows_4g // BS + 64
    else:
        rows_4g = 2 ** 31 // 1024                              # ckv rows below the 2 GiB offset
        NB = (3 * 2 ** 30 // 1024) // BS
    say(f"[mla] large cache ({span}): {NB} blocks")
    case = gen.mla_kv_head_case(560, B=1, S=T, He=He, num_blocks=1, block_size=T,
                                slot_kind="random", skip_frac=0.05)   # compact slots 0..T-1
    rng = gen.rng_for(561)
    lo = rng.choice(rows_4g - 1, size=T // 2, replace=False)
    hi = rows_4g + rng.choice(NB * BS - rows_4g, size=T - T // 2, replace=False)
    big = np.concatenate([lo, hi]).astype(np.int64)
    rng.shuffle(big)
    big[case["slot_mapping"] < 0] = -1
    sentinel = int(np.array([gen.BF16_SENTINEL], dtype=np.uint16).view(np.int16)[0])
    kc = torch.full((NB, BS, 1, 64), sentinel, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    ck = torch.full((NB, BS, 1, 512), sentinel, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    ws = new_workspace(T)
    k.kvrc_mla_kv_head_paged(dbf(case["x"]), dbf(case["w"]), dbf(case["gamma"]), dbf(case["cos"]),
                             dbf(case["sin"]), torch.from_numpy(big).to(DEV), kc, ck,
                             workspace=ws, alpha_kv=case["alpha"], eps=case["eps"])
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws)) == 0
    valid = big >= 0
    idx = torch.from_numpy(big[valid]).to(DEV)
    compact = case["slot_mapping"][valid]
    got = {"ckv_cache": np.full((T, 512), gen.BF16_SENTINEL, np.uint16),
           "k_cache": np.full((T, 64), gen.BF16_SENTINEL, np.uint16)}
    for name, t, d in (("ckv_cache", ck, 512), ("k_cache", kc, 64)):
        rows = t.view(-1, d)[idx].view(torch.int16).cpu().numpy().view(np.uint16)
        got[name][compact] = rows
        changed = int((t.view(torch.int16) != sentinel).sum().item())
        in_rows = int((t.view(-1, d)[idx].view(torch.int16) != sentinel).sum().item())
        assert changed == in_rows, f"{name}: bytes outside the written rows changed"
    compare_mla(case, got)


def run_mla_blk_gpu(case, index=None, err=None):
    """One block-indexed call (x, cos, sin as [B, S, ...]); the workspace
    must be zero again afterwards."""
    B, S = case["B"], case["S"]
    caches = {n: dev_cache(spec.numpy()) for n, spec in case["caches"].items()}
    idx = case["block_index"] if index is None else index
    ws = new_workspace(B * S)
    k.kvrc_mla_kv_head_paged_blk(dbf(case["x"]).view(B, S, -1), dbf(case["w"]), dbf(case["gamma"]),
                                 dbf(case["cos"]).view(B, S, 64), dbf(case["sin"]).view(B, S, 64),
                                 torch.from_numpy(idx).to(DEV), caches["k_cache"],
                                 caches["ckv_cache"], caches.get("ckv_scale"), workspace=ws,
                                 alpha_kv=case["alpha"], eps=case["eps"], err_count=err)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws)) == 0, "workspace not left zero"
    return {n: host_cache(t) for n, t in caches.items()}


@pytest.mark.parametrize("B,S,BS,offsets,He", [(2, 300, 64, True, 256), (3, 37, 16, False, 64),
                                               (1, 1, 16, False, 64), (4, 129, 128, True, 512),
                                               (2, 13, 1, False, 64), (2, 4096, 128, False, 1024)])
def test_mla_paged_blk(B, S, BS, offsets, He):
    """Block-indexed placement (PA_BLK_BSND): one entry per chunk of BS
    tokens, ragged last chunks, skipped chunks, entries with offsets inside
    the block; the rows come from the oracle's placement."""
    say(f"[mla] blk B={B} S={S} BS={BS} He={He}")
    chunks = B * (-(-S // BS))
    case = gen.mla_kv_head_blk_case(570 + S + BS, B=B, S=S, He=He,
                                    num_blocks=max(2 * chunks, 16), block_size=BS,
                                    n_skip=min(2, chunks - 1), entry_offsets=offsets)
    rows = case["num_blocks"] * BS
    slots = M.block_index_slots(case["block_index"], B, S, BS, rows)
    compare_mla(case, run_mla_blk_gpu(case), slots=slots)


def test_mla_paged_blk_invalid_entries_counted_per_token():
    case = gen.mla_kv_head_blk_case(580, B=2, S=100, He=64, num_blocks=16, block_size=32)
    idx = case["block_index"].copy()                 # 4 chunks per sequence: 32, 32, 32, 4 tokens
    idx[1] = 16 * 32                                 # out of range: 32 tokens skipped and counted
    idx[3] = -7                                      # out of range: the 4-token last chunk
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = run_mla_blk_gpu(case, index=idx, err=err)
    assert int(err.item()) == 32 + 4
    fixed = idx.copy()
    fixed[[1, 3]] = -1
    slots = M.block_index_slots(fixed, 2, 100, 32, 16 * 32)
    compare_mla(case, got, slots=slots)


# ---------------------------------------------------------------------------
# quantised ckv cache (int8 RowMax/127, E4M3FN RowMax/448)
# ---------------------------------------------------------------------------

def test_mla_quantised_named_workload_full_size():
    """The named workload's shape (T=32768, He=7168) into int8 and E4M3FN ckv
    caches; one float64 evaluation serves both."""
    say("[mla-q] workload mla_kv_head (T=32768, He=7168), int8 and fp8")
    base = gen.make_config("mla_kv_head")
    bounds = None
    for kind in ("int8", "fp8"):
        case = dict(base, ckv_dtype=kind, caches=dict(
            base["caches"], ckv_cache=gen.ckv_cache_spec(base["caches"]["ckv_cache"].shape, kind),
            ckv_scale=gen.CacheSpec(base["caches"]["ckv_cache"].shape[:3], np.float32,
                                    gen.SCALE_SENTINEL)))
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        got = run_mla_gpu(case, err=err)
        assert int(err.item()) == 0
        if bounds is None:
            bounds = head_bounds(case)
        frac, _ = compare_mla(case, got, bounds=bounds)
        say(f"[mla-q] {kind}: codes equal to the oracle's {frac:.6f}")


@pytest.mark.parametrize("kind", ["int8", "fp8"])
@pytest.mark.parametrize("B,S,He", [(1, 1, 32), (1, 5, 64), (2, 300, 7168), (3, 257, 1024),
                                    (1, 2305, 64)])
def test_mla_quantised_shapes(kind, B, S, He):
    say(f"[mla-q] {kind} B={B} S={S} He={He}")
    case = gen.mla_kv_head_case(600 + S + He, B=B, S=S, He=He, num_blocks=160, block_size=32,
                                slot_kind="random", skip_frac=0.1, ckv_dtype=kind)
    frac, _ = compare_mla(case, run_mla_gpu(case))
    say(f"[mla-q] codes equal {frac:.5f}")


@pytest.mark.parametrize("kind", ["int8", "fp8"])
@pytest.mark.parametrize("alpha,x_sigma", [(0.0, 1.0), (-1.5, 1.0), (1.0, 1e-3), (1.0, 300.0),
                                           (2.0 ** 70, 1.0), (2.0 ** -80, 1.0)])
def test_mla_quantised_alpha_and_magnitudes(kind, alpha, x_sigma):
    """alpha = 0: every row zero (scale 0, code bytes 0); a negative alpha;
    tiny and large inputs (the norm makes the codes scale-free); alpha 2^70
    and 2^-80 put the scales above 2^60 and below 2^-60, outside the fast
    reciprocal's domain (IEEE division there)."""
    say(f"[mla-q] {kind} alpha={alpha} x_sigma={x_sigma}")
    case = gen.mla_kv_head_case(620, B=2, S=200, He=1024, num_blocks=32, block_size=32,
                                slot_kind="random", alpha=alpha, x_sigma=x_sigma, ckv_dtype=kind)
    compare_mla(case, run_mla_gpu(case))


def test_mla_quantised_many_pairs_and_shared_workspace():
    """1280 workgroups (two exchanges per pair, pairs starting while others
    run) with no timed-out wait; then a bf16 call and an fp8 call on the same
    workspace, each leaving it zero."""
    say("[mla-q] T=163840 int8, then bf16 and fp8 on one workspace")
    case = gen.mla_kv_head_case(630, B=4, S=40960, He=64, num_blocks=1400, block_size=128,
                                slot_kind="random", skip_frac=0.01, ckv_dtype="int8")
    ws = new_workspace(163840)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    compare_mla(case, run_mla_gpu(case, err=err, workspace=ws))
    assert int(err.item()) == 0
    for kind in ("bf16", "fp8"):
        c = gen.mla_kv_head_case(631, B=1, S=700, He=128, num_blocks=64, block_size=16,
                                 slot_kind="random", ckv_dtype=kind)
        compare_mla(c, run_mla_gpu(c, err=err, workspace=ws))
    assert int(err.item()) == 0


@pytest.mark.parametrize("kind", ["int8", "fp8"])
@pytest.mark.parametrize("B,S,BS,offsets,He", [(2, 300, 64, True, 256), (3, 37, 16, False, 64)])
def test_mla_quantised_paged_blk(kind, B, S, BS, offsets, He):
    say(f"[mla-q] blk {kind} B={B} S={S} BS={BS} He={He}")
    chunks = B * (-(-S // BS))
    case = gen.mla_kv_head_blk_case(640 + S + BS, B=B, S=S, He=He,
                                    num_blocks=max(2 * chunks, 16), block_size=BS,
                                    n_skip=min(2, chunks - 1), entry_offsets=offsets,
                                    ckv_dtype=kind)
    slots = M.block_index_slots(case["block_index"], B, S, BS, case["num_blocks"] * BS)
    compare_mla(case, run_mla_blk_gpu(case), slots=slots)


def test_mla_quantised_invalid_slots_are_skipped_and_counted():
    case = gen.mla_kv_head_case(650, B=1, S=300, He=256, num_blocks=32, block_size=16,
                                slot_kind="random", skip_frac=0.05, ckv_dtype="fp8")
    slots = case["slot_mapping"].copy()
    slots[[3, 130, 299]] = [32 * 16, -2, 1 << 40]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = run_mla_gpu(case, slots=slots, err=err)
    assert int(err.item()) == 3
    fixed = slots.copy()
    fixed[[3, 130, 299]] = -1
    compare_mla(case, got, slots=fixed)


@pytest.mark.parametrize("span", ["over_4gib", "3gib"])
def test_mla_quantised_large_cache_offsets(span):
    """An int8 ckv cache of 4 GiB or more (2^23 rows) takes the plain-store
    path: rows beyond the 32-bit byte offset land exactly, with their scales;
    a 3 GiB one takes the buffer stores with offsets past 2^31. Nothing else
    changes."""
    T, He, BS = 300, 256, 128
    if span == "over_4gib":
        rows_4g = 2 ** 32 // 512
        NB = rows_4g // BS + 64
    else:
        rows_4g = 2 ** 31 // 512
        NB = (3 * 2 ** 30 // 512) // BS
    say(f"[mla-q] int8 large cache ({span}): {NB} blocks")
    case = gen.mla_kv_head_case(660, B=1, S=T, He=He, num_blocks=1, block_size=T,
                                slot_kind="random", skip_frac=0.05, ckv_dtype="int8")
    rng = gen.rng_for(661)
    lo = rng.choice(rows_4g - 1, size=T // 2, replace=False)
    hi = rows_4g + rng.choice(NB * BS - rows_4g, size=T - T // 2, replace=False)
    big = np.concatenate([lo, hi]).astype(np.int64)
    rng.shuffle(big)
    big[case["slot_mapping"] < 0] = -1
    sentinel = int(np.array([gen.BF16_SENTINEL], dtype=np.uint16).view(np.int16)[0])
    kc = torch.full((NB, BS, 1, 64), sentinel, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    ck = torch.full((NB, BS, 1, 512), gen.INT8_SENTINEL, dtype=torch.int8, device=DEV)
    sc = torch.full((NB, BS, 1), gen.SCALE_SENTINEL, dtype=torch.float32, device=DEV)
    ws = new_workspace(T)
    k.kvrc_mla_kv_head_paged(dbf(case["x"]), dbf(case["w"]), dbf(case["gamma"]), dbf(case["cos"]),
                             dbf(case["sin"]), torch.from_numpy(big).to(DEV), kc, ck, sc,
                             workspace=ws, alpha_kv=case["alpha"], eps=case["eps"])
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws)) == 0
    valid = big >= 0
    idx = torch.from_numpy(big[valid]).to(DEV)
    compact = case["slot_mapping"][valid]
    got = {"ckv_cache": np.full((T, 512), gen.INT8_SENTINEL, np.int8),
           "k_cache": np.full((T, 64), gen.BF16_SENTINEL, np.uint16),
           "ckv_scale": np.full(T, gen.SCALE_SENTINEL, np.float32)}
    got["ckv_cache"][compact] = ck.view(-1, 512)[idx].cpu().numpy()
    got["k_cache"][compact] = kc.view(-1, 64)[idx].view(torch.int16).cpu().numpy().view(np.uint16)
    got["ckv_scale"][compact] = sc.view(-1)[idx].cpu().numpy()
    for t, d, s_ in ((ck, 512, gen.INT8_SENTINEL), (kc.view(torch.int16), 64, sentinel),
                     (sc, 1, gen.SCALE_SENTINEL)):
        changed = int((t != s_).sum().item())
        in_rows = int((t.reshape(-1, d)[idx] != s_).sum().item())
        assert changed == in_rows, "bytes outside the written rows changed"
    compare_mla(case, got)


def test_mla_quantised_graph_replays_reuse_the_workspace():
    """The two-exchange quantised head captured in a HIP graph: three
    replays (eager work in between) on one workspace, each equal to the
    eager call bit for bit, the workspace zero after each."""
    say("[mla-q] fp8 graph replays")
    case = gen.mla_kv_head_case(670, B=1, S=600, He=256, num_blocks=64, block_size=16,
                                slot_kind="random", ckv_dtype="fp8")
    ws = new_workspace(600)
    eager = run_mla_gpu(case, workspace=ws)
    compare_mla(case, eager)
    x, w, gm = dbf(case["x"]), dbf(case["w"]), dbf(case["gamma"])
    cs, sn = dbf(case["cos"]), dbf(case["sin"])
    sl = torch.from_numpy(case["slot_mapping"]).to(DEV)
    caches = {n: dev_cache(spec.numpy()) for n, spec in case["caches"].items()}
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        k.kvrc_mla_kv_head_paged(x, w, gm, cs, sn, sl, caches["k_cache"], caches["ckv_cache"],
                                 caches["ckv_scale"], workspace=ws, alpha_kv=case["alpha"],
                                 eps=case["eps"], stream=stream)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        k.kvrc_mla_kv_head_paged(x, w, gm, cs, sn, sl, caches["k_cache"], caches["ckv_cache"],
                                 caches["ckv_scale"], workspace=ws, alpha_kv=case["alpha"],
                                 eps=case["eps"], stream=stream)
    for rep in range(3):
        for n, spec in case["caches"].items():
            caches[n].copy_(dev_cache(spec.numpy()))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        stream.synchronize()
        assert int(torch.count_nonzero(ws)) == 0, f"replay {rep}: workspace not left zero"
        for n, t in caches.items():
            np.testing.assert_array_equal(host_cache(t), eager[n], err_msg=f"replay {rep}: {n}")


@pytest.mark.parametrize("kind", ["bf16", "int8", "fp8"])
def test_mla_all_tokens_skipped(kind):
    """Every slot -1 (a ragged 300-token batch: two pairs, the second
    partial): the kernel runs and its pairs still exchange, but no cache
    byte changes, nothing is counted and the workspace ends zero."""
    case = gen.mla_kv_head_case(680, B=1, S=300, He=128, num_blocks=16, block_size=32,
                                slot_kind="random", ckv_dtype=kind)
    slots = np.full(300, -1, dtype=np.int64)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = run_mla_gpu(case, slots=slots, err=err)
    assert int(err.item()) == 0
    for name, spec in case["caches"].items():
        np.testing.assert_array_equal(got[name], spec.numpy(), err_msg=name)


# ---------------------------------------------------------------------------
# The pair exchange without any co-residency assumption
# ---------------------------------------------------------------------------

def _mla_device_inputs(case):
    return (dbf(case["x"]), dbf(case["w"]), dbf(case["gamma"]), dbf(case["cos"]),
            dbf(case["sin"]), torch.from_numpy(case["slot_mapping"]).to(DEV))


@pytest.mark.parametrize("kind", ["bf16", "int8", "fp8"])
def test_mla_takeover_gives_the_same_bits(kind):
    """The second workgroup of every pair is held back (3 ms) before it
    claims its half: the first one finds neither partials nor a claim, takes
    the partner's half over and computes both halves itself; the outputs are
    bit-identical to the paired computation, every pair was taken over, the
    partner left without writing, and the workspace ends zero."""
    say(f"[mla] takeover {kind}")
    case = gen.mla_kv_head_case(560, B=1, S=2305, He=256, num_blocks=160, block_size=16,
                                slot_kind="random", skip_frac=0.05, ckv_dtype=kind)
    want = run_mla_gpu(case)
    T = case["x"].shape[0]
    caches = {n: dev_cache(spec.numpy()) for n, spec in case["caches"].items()}
    ws = new_workspace(T)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    steals = torch.zeros(1, dtype=torch.int32, device=DEV)
    k.kvrc_mla_kv_head_paged(*_mla_device_inputs(case), caches["k_cache"], caches["ckv_cache"],
                             caches.get("ckv_scale"), workspace=ws, alpha_kv=case["alpha"],
                             eps=case["eps"], err_count=err, _stall_us=3000, _steals=steals)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws)) == 0, "workspace not left zero"
    assert int(err.item()) == 0
    assert int(steals.item()) == -(-T // 256), "every pair's second half was taken over"
    got = {n: host_cache(t) for n, t in caches.items()}
    for n in want:
        np.testing.assert_array_equal(got[n], want[n], err_msg=n)
    compare_mla(case, got)


def test_mla_overlapping_calls_on_two_streams():
    """Two MLA head calls in flight at once on two streams, each with its own
    workspace and with more workgroups than the chip holds (1280 each): pairs
    may be split by the other call's workgroups. Both end with err_count 0,
    workspaces zero, and outputs bit-identical to the same calls made one
    after the other (which meet the oracle bound)."""
    say("[mla] two overlapping calls, 1280 workgroups each")
    cases = [gen.mla_kv_head_case(541, B=4, S=40960, He=64, num_blocks=1400, block_size=128,
                                  slot_kind="random", skip_frac=0.01),
             gen.mla_kv_head_case(542, B=4, S=40960, He=64, num_blocks=1400, block_size=128,
                                  slot_kind="random", skip_frac=0.01, ckv_dtype="int8")]
    want = [run_mla_gpu(c) for c in cases]
    compare_mla(cases[0], want[0])
    ins = [_mla_device_inputs(c) for c in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        caches = [{n: dev_cache(spec.numpy()) for n, spec in c["caches"].items()} for c in cases]
        ws = [new_workspace(c["x"].shape[0]) for c in cases]
        errs = [torch.zeros(1, dtype=torch.int32, device=DEV) for _ in cases]
        torch.cuda.synchronize()
        for c, i, ca, w, e, s in zip(cases, ins, caches, ws, errs, streams):
            k.kvrc_mla_kv_head_paged(*i, ca["k_cache"], ca["ckv_cache"], ca.get("ckv_scale"),
                                     workspace=w, alpha_kv=c["alpha"], eps=c["eps"],
                                     err_count=e, stream=s)
        torch.cuda.synchronize()
        for c, ca, w, e, wt in zip(cases, caches, ws, errs, want):
            assert int(e.item()) == 0
            assert int(torch.count_nonzero(w)) == 0, "workspace not left zero"
            for n, t in ca.items():
                np.testing.assert_array_equal(host_cache(t), wt[n], err_msg=f"rep {rep} {n}")
        say(f"[mla] overlap rep {rep}: both calls equal the sequential ones")


@pytest.mark.parametrize("kind", ["bf16", "int8"])
def test_mla_workspace_left_dirty_is_counted_and_ignored(kind):
    """Flags and claim words left in the workspace by another call (written
    here from the host: each call marks its own with a fresh tag, so these
    can never match) are counted in err_count, and the outputs are still the
    clean call's."""
    case = gen.mla_kv_head_case(543, B=1, S=700, He=128, num_blocks=64, block_size=16,
                                slot_kind="random", ckv_dtype=kind)
    want = run_mla_gpu(case)
    T = case["x"].shape[0]
    npairs = -(-T // 256)
    ws = new_workspace(T)
    words = ws.view(torch.int32)
    flags0 = npairs * 4 * 256                       # after the sums and maxima areas
    words[:flags0] = 0x7F7F7F7F                     # stale partials
    words[flags0:flags0 + 2 * npairs] = 0x7FFFFFFF   # flags of no call (tags are below 2^30)
    words[flags0 + 2 * npairs:flags0 + 4 * npairs] = -1   # claim words of no call
    caches = {n: dev_cache(spec.numpy()) for n, spec in case["caches"].items()}
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    k.kvrc_mla_kv_head_paged(*_mla_device_inputs(case), caches["k_cache"], caches["ckv_cache"],
                             caches.get("ckv_scale"), workspace=ws, alpha_kv=case["alpha"],
                             eps=case["eps"], err_count=err)
    torch.cuda.synchronize()
    assert int(err.item()) > 0, "a workspace that was not zero must be reported"
    for n, t in caches.items():
        np.testing.assert_array_equal(host_cache(t), want[n], err_msg=n)
