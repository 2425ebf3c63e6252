"""C-ABI boundary tests that run without a GPU.

* The library loads and exports exactly the functions include/kvrc.h declares.
* Host-side validation returns the documented status before any HIP call.
  Every call below is INVALID on purpose (or empty), so nothing is launched and
  the fake device addresses are never dereferenced.
* The Python binding refuses CPU tensors and a missing library (no fallback).
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import latent_attention_kv_amd as k

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, HIP, WORKSPACE = range(8)


def header_functions():
    src = "\n".join(open(h).read() for h in HEADERS)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int32_t|int64_t)\s*\*?\s*(\w+)\s*\(", src,
                                 re.M)))


def test_exports_match_header():
    names = header_functions()
    assert names == sorted(k.EXPORTED_SYMBOLS)
    L = k.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", k.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported
    assert k.lib().kvrc_version() == 106


def test_status_strings():
    L = k.lib()
    for s in range(8):
        assert L.kvrc_status_string(s) != b"unknown status"
    assert L.kvrc_status_string(99) == b"unknown status"


# fake, 256-byte aligned, non-overlapping "device" addresses (never touched)
A = {name: (i + 1) << 32 for i, name in enumerate(
    ["kv", "gamma", "cos", "sin", "idx", "kc", "ckv", "scale", "err"])}


def paged(**over):
    a = dict(kv=A["kv"], gamma=A["gamma"], cos=A["cos"], sin=A["sin"], idx=A["idx"], kc=A["kc"],
             ckv=A["ckv"], scale=None, B=2, S=3, Dv=512, Dk=64, NB=4, BS=16, dt=0, eps=1e-6,
             err=None, stream=None)
    a.update(over)
    return k.lib().kvrc_paged_norm_rope_cache(a["kv"], a["gamma"], a["cos"], a["sin"], a["idx"],
                                              a["kc"], a["ckv"], a["scale"], a["B"], a["S"],
                                              a["Dv"], a["Dk"], a["NB"], a["BS"], a["dt"],
                                              a["eps"], a["err"], a["stream"])


def norm(**over):
    a = dict(kv=A["kv"], gamma=A["gamma"], cos=A["cos"], sin=A["sin"], idx=A["idx"], kc=A["kc"],
             ckv=A["ckv"], scale=None, B=2, S=3, Dv=512, Dk=64, Bc=2, Sc=16, dt=0, eps=1e-6,
             err=None, stream=None)
    a.update(over)
    return k.lib().kvrc_norm_rope_cache(a["kv"], a["gamma"], a["cos"], a["sin"], a["idx"],
                                        a["kc"], a["ckv"], a["scale"], a["B"], a["S"], a["Dv"],
                                        a["Dk"], a["Bc"], a["Sc"], a["dt"], a["eps"], a["err"],
                                        a["stream"])


@pytest.mark.parametrize("over,want", [
    (dict(kv=None), NULL), (dict(gamma=None), NULL), (dict(idx=None), NULL),
    (dict(kc=None), NULL), (dict(ckv=None), NULL),
    (dict(Dv=510), SHAPE), (dict(Dk=4), SHAPE), (dict(Dk=60), SHAPE), (dict(Dv=0), SHAPE),
    (dict(B=-1), SHAPE), (dict(S=-2), SHAPE), (dict(NB=-1), SHAPE), (dict(BS=0), SHAPE),
    (dict(B=1 << 20, S=1 << 20), SHAPE),
    (dict(dt=3), DTYPE), (dict(dt=-1), DTYPE), (dict(dt=1), DTYPE), (dict(dt=2), DTYPE),
    (dict(scale=A["scale"]), DTYPE), (dict(dt=3, scale=A["scale"]), DTYPE),
    (dict(dt=2, scale=A["scale"] + 2), ALIGN),
    # an E4M3FN cache holds one byte per element: 64 rows * 512 B
    (dict(dt=2, scale=A["ckv"] + 64 * 512 - 16), ALIAS),
    (dict(kv=A["kv"] + 8), ALIGN), (dict(cos=A["cos"] + 2), ALIGN), (dict(idx=A["idx"] + 4), ALIGN),
    (dict(kc=A["kc"] + 8), ALIGN), (dict(dt=1, scale=A["scale"] + 2), ALIGN),
    (dict(err=A["err"] + 2), ALIGN),
    (dict(kc=A["kv"]), ALIAS), (dict(ckv=A["kc"] + 4096), ALIAS), (dict(ckv=A["sin"]), ALIAS),
    (dict(dt=1, scale=A["ckv"] + 16), ALIAS), (dict(err=A["kc"]), ALIAS),
    (dict(B=0), OK), (dict(S=0), OK), (dict(B=0, kv=None, kc=None), OK),
])
def test_paged_validation(over, want):
    assert paged(**over) == want


@pytest.mark.parametrize("over", [
    # row widths above the library's bound of 2^20 elements
    dict(Dv=(1 << 20) + 8), dict(Dk=(1 << 20) + 8), dict(Dv=1 << 32),
    # 2^31 - 1 tokens of 2^20 + 2^20 elements with one cache row: every size
    # passes alone, but kv spans 2^31 * 2^21 * 2 bytes (beyond int64's range
    # before the cap, 2^53 with it); here the cache product overflows instead
    dict(B=(1 << 31) - 1, S=1, Dv=1 << 20, Dk=1 << 20, NB=1 << 45, BS=1 << 10),
    # the cache byte span rows * Dv * 2 passes 2^63
    dict(NB=1 << 40, BS=1 << 10, Dv=1 << 20),
    dict(NB=1 << 62, BS=1, Dk=64),
])
def test_paged_validation_at_the_caps(over):
    """Sizes at and past the bounds: every byte span is formed with checked
    products, so extreme sizes give a shape error, never an overflow (run
    under the host sanitizer build as well)."""
    assert paged(**over) == SHAPE


def test_norm_and_blk_validation_at_the_caps():
    assert norm(Dv=(1 << 20) + 8) == SHAPE
    assert norm(Bc=1 << 40, Sc=1 << 20, Dv=1 << 20) == SHAPE
    assert paged_blk(Dk=(1 << 20) + 8) == SHAPE
    assert paged_blk(B=1 << 30, S=2, BS=1, NB=1 << 62) == SHAPE


def paged_blk(**over):
    a = dict(kv=A["kv"], gamma=A["gamma"], cos=A["cos"], sin=A["sin"], idx=A["idx"], kc=A["kc"],
             ckv=A["ckv"], scale=None, B=2, S=300, Dv=512, Dk=64, NB=64, BS=128, dt=0, eps=1e-6,
             err=None, stream=None)
    a.update(over)
    return k.lib().kvrc_paged_blk_norm_rope_cache(a["kv"], a["gamma"], a["cos"], a["sin"],
                                                  a["idx"], a["kc"], a["ckv"], a["scale"], a["B"],
                                                  a["S"], a["Dv"], a["Dk"], a["NB"], a["BS"],
                                                  a["dt"], a["eps"], a["err"], a["stream"])


@pytest.mark.parametrize("over,want", [
    (dict(idx=None), NULL), (dict(BS=0), SHAPE), (dict(NB=-1), SHAPE), (dict(BS=1 << 32), SHAPE),
    (dict(Dk=12), SHAPE), (dict(dt=1), DTYPE), (dict(idx=A["idx"] + 4), ALIGN),
    # the index holds B*ceil(S/BS) = 6 entries (48 bytes): a cache starting inside it aliases
    (dict(kc=A["idx"] + 32), ALIAS),
    (dict(B=0), OK), (dict(S=0, idx=None), OK),
])
def test_paged_blk_validation(over, want):
    assert paged_blk(**over) == want


@pytest.mark.parametrize("over,want", [
    (dict(Bc=1), SHAPE), (dict(Sc=-1), SHAPE), (dict(sin=None), NULL), (dict(Dv=12), SHAPE),
    (dict(dt=1), DTYPE), (dict(ckv=A["ckv"] + 8), ALIGN), (dict(ckv=A["kc"]), ALIAS),
    (dict(B=0), OK),
])
def test_norm_validation(over, want):
    assert norm(**over) == want


M = {name: (i + 40) << 32 for i, name in enumerate(
    ["x", "w", "gamma", "cos", "sin", "slot", "kc", "ckv", "err", "ws", "sc"])}
WS_300 = 2 * (4 * 256 * 4 + 4 * 4)      # 300 tokens: two pairs of workgroups


def mla(**over):
    a = dict(x=M["x"], w=M["w"], gamma=M["gamma"], alpha=1.0, cos=M["cos"], sin=M["sin"],
             slot=M["slot"], kc=M["kc"], ckv=M["ckv"], sc=None, T=300, He=7168, NB=64, BS=128,
             dt=0, eps=1e-6, ws=M["ws"], wsb=WS_300, err=None, stream=None)
    a.update(over)
    return k.lib().kvrc_mla_kv_head_paged(a["x"], a["w"], a["gamma"], a["alpha"], a["cos"],
                                          a["sin"], a["slot"], a["kc"], a["ckv"], a["sc"], a["T"],
                                          a["He"], a["NB"], a["BS"], a["dt"], a["eps"], a["ws"],
                                          a["wsb"], a["err"], a["stream"])


def mla_blk(**over):
    a = dict(x=M["x"], w=M["w"], gamma=M["gamma"], alpha=1.0, cos=M["cos"], sin=M["sin"],
             idx=M["slot"], kc=M["kc"], ckv=M["ckv"], sc=None, B=3, S=100, He=7168, NB=64,
             BS=128, dt=0, eps=1e-6, ws=M["ws"], wsb=WS_300, err=None, stream=None)
    a.update(over)
    return k.lib().kvrc_mla_kv_head_paged_blk(a["x"], a["w"], a["gamma"], a["alpha"], a["cos"],
                                              a["sin"], a["idx"], a["kc"], a["ckv"], a["sc"],
                                              a["B"], a["S"], a["He"], a["NB"], a["BS"], a["dt"],
                                              a["eps"], a["ws"], a["wsb"], a["err"], a["stream"])


@pytest.mark.parametrize("over,want", [
    (dict(idx=None), NULL), (dict(B=-1), SHAPE), (dict(S=-1), SHAPE), (dict(BS=0), SHAPE),
    (dict(He=16), SHAPE), (dict(B=1 << 20, S=1 << 12), SHAPE),       # T = 2^32 > 2^31 - 1
    (dict(idx=M["slot"] + 4), ALIGN), (dict(ws=None), NULL), (dict(wsb=WS_300 - 1), WORKSPACE),
    # 3 * ceil(100 / 128) = 3 index entries (24 bytes): an output 16 bytes in overlaps
    (dict(kc=M["slot"] + 16), ALIAS),
    (dict(dt=2), DTYPE), (dict(dt=2, sc=M["sc"] + 2), ALIGN), (dict(dt=-1), DTYPE),
    # no blocks and a block size near 2^63: one chunk per sequence, 3 entries (24 bytes),
    # so a workspace 16 bytes into the index aliases (the chunk count must not overflow;
    # the caches hold no rows, so only the workspace can overlap)
    (dict(NB=0, BS=(1 << 63) - 1, ws=M["slot"] + 16), ALIAS),
    (dict(B=0), OK), (dict(S=0, idx=None), OK),
])
def test_mla_blk_validation(over, want):
    assert mla_blk(**over) == want


def test_mla_workspace_bytes():
    """One pair of workgroups per 256 tokens: 256 partial sums and 256
    partial maxima per half, two flags and two claim words."""
    f = k.lib().kvrc_mla_kv_head_workspace_bytes
    assert f(0) == 0
    assert f(1) == f(256) == 4112
    assert f(257) == 2 * 4112
    assert f(32768) == 128 * 4112
    assert f(-1) == -1 and f(1 << 31) == -1
    assert f(300) == WS_300


@pytest.mark.parametrize("over,want", [
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(gamma=None), NULL), (dict(cos=None), NULL),
    (dict(sin=None), NULL), (dict(slot=None), NULL), (dict(kc=None), NULL), (dict(ckv=None), NULL),
    (dict(He=0), SHAPE), (dict(He=16), SHAPE), (dict(He=7160), SHAPE), (dict(T=-1), SHAPE),
    (dict(T=1 << 31), SHAPE), (dict(NB=-1), SHAPE), (dict(BS=0), SHAPE),
    (dict(x=M["x"] + 8), ALIGN), (dict(w=M["w"] + 2), ALIGN), (dict(slot=M["slot"] + 4), ALIGN),
    (dict(ckv=M["ckv"] + 8), ALIGN), (dict(err=M["err"] + 1), ALIGN),
    # x holds 300 * 7168 * 2 bytes: a cache starting inside it aliases
    (dict(kc=M["x"] + 4096), ALIAS), (dict(ckv=M["w"]), ALIAS), (dict(kc=M["ckv"] + 16), ALIAS),
    (dict(err=M["kc"]), ALIAS),
    (dict(ws=None), NULL), (dict(ws=M["ws"] + 8), ALIGN), (dict(ws=M["ckv"] + 64), ALIAS),
    (dict(ws=M["x"]), ALIAS), (dict(wsb=WS_300 - 1), WORKSPACE), (dict(wsb=0), WORKSPACE),
    (dict(T=0), OK), (dict(T=0, x=None, kc=None), OK), (dict(T=0, ws=None, wsb=0), OK),
    # quantised ckv: the scale pointer goes with the type; [rows] float32
    (dict(dt=3), DTYPE), (dict(dt=1), DTYPE), (dict(dt=2), DTYPE), (dict(sc=M["sc"]), DTYPE),
    (dict(dt=1, sc=M["sc"] + 2), ALIGN), (dict(dt=1, sc=M["ckv"] + 64), ALIAS),
    (dict(dt=2, sc=M["kc"]), ALIAS), (dict(dt=1, sc=M["ws"]), ALIAS), (dict(dt=1, sc=M["x"]), ALIAS),
    # an int8 ckv cache of 64 * 128 rows holds 4 MiB: a scale array 4 bytes before its end
    # overlaps it
    (dict(dt=1, sc=M["ckv"] + 64 * 128 * 512 - 4), ALIAS),
])
def test_mla_validation(over, want):
    assert mla(**over) == want


@pytest.mark.parametrize("over", [
    dict(He=(1 << 20) + 32), dict(He=1 << 62), dict(NB=1 << 62, BS=2),
    dict(NB=1 << 55, BS=1 << 8),                   # rows * 512 * 2 passes 2^63
])
def test_mla_validation_at_the_caps(over):
    assert mla(**over) == SHAPE
    assert mla(dt=1, sc=M["sc"], **over) == SHAPE


SL = {name: (i + 60) << 32 for i, name in enumerate(["q", "k", "kl", "sc", "ix", "err"])}


def select(**over):
    a = dict(q=SL["q"], k=SL["k"], kl=SL["kl"], klc=4, scale=0.1, N=4, H=64, Di=128, Bcap=256,
             kbs=64, sel=2, cmp=1, topk=16, sc=SL["sc"], ix=SL["ix"], err=None, stream=None)
    a.update(over)
    return k.lib().qsa_select_topk(a["q"], a["k"], a["kl"], a["klc"], a["scale"], a["N"], a["H"],
                                   a["Di"], a["Bcap"], a["kbs"], a["sel"], a["cmp"], a["topk"],
                                   a["sc"], a["ix"], a["err"], a["stream"])


@pytest.mark.parametrize("over,want", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(kl=None), NULL), (dict(sc=None), NULL),
    (dict(ix=None), NULL),
    (dict(H=8), SHAPE), (dict(H=40), SHAPE), (dict(Di=48), SHAPE), (dict(Di=0), SHAPE),
    (dict(kbs=0), SHAPE), (dict(sel=0), SHAPE), (dict(cmp=0), SHAPE), (dict(topk=-1), SHAPE),
    (dict(klc=2), SHAPE), (dict(N=-1), SHAPE), (dict(Bcap=-1), SHAPE),
    (dict(H=1024, Di=4096), SHAPE),                   # working set beyond one workgroup's LDS
    (dict(q=SL["q"] + 8), ALIGN), (dict(kl=SL["kl"] + 4), ALIGN), (dict(sc=SL["sc"] + 2), ALIGN),
    (dict(ix=SL["ix"] + 1), ALIGN),
    (dict(sc=SL["q"] + 64), ALIAS), (dict(ix=SL["sc"] + 16), ALIAS), (dict(err=SL["ix"]), ALIAS),
    (dict(N=0, klc=1), OK), (dict(N=0, klc=0, q=None, sc=None), OK),
])
def test_select_validation(over, want):
    assert select(**over) == want


Q = {name: (i + 20) << 32 for i, name in enumerate(
    ["raw", "bk", "kl", "rc", "rs", "w", "praw", "prope", "nraw", "nrope", "err"])}


def qsa(**over):
    a = dict(raw=Q["raw"], bk=Q["bk"], kl=Q["kl"], klc=3, rc=Q["rc"], rs=Q["rs"], w=Q["w"],
             praw=Q["praw"], prope=Q["prope"], nraw=Q["nraw"], nrope=Q["nrope"], N=3, L=100,
             Di=128, Dr=64, Bcap=10, kbs=64, eps=1e-6, err=None, stream=None)
    a.update(over)
    return k.lib().qsa_prepare(a["raw"], a["bk"], a["kl"], a["klc"], a["rc"], a["rs"], a["w"],
                               a["praw"], a["prope"], a["nraw"], a["nrope"], a["N"], a["L"],
                               a["Di"], a["Dr"], a["Bcap"], a["kbs"], a["eps"], a["err"],
                               a["stream"])


@pytest.mark.parametrize("over,want", [
    (dict(raw=None), NULL), (dict(bk=None), NULL), (dict(kl=None), NULL), (dict(praw=None), NULL),
    (dict(nraw=None), NULL), (dict(rs=None), NULL), (dict(prope=None), NULL),
    (dict(nrope=None), NULL), (dict(rc=None, rs=None, prope=None), NULL),
    (dict(Di=12), SHAPE), (dict(Di=0), SHAPE), (dict(Di=8192), SHAPE), (dict(kbs=1), SHAPE),
    (dict(Dr=63), SHAPE), (dict(Dr=0), SHAPE), (dict(Dr=256), SHAPE), (dict(klc=2), SHAPE),
    (dict(N=-1), SHAPE), (dict(L=-1), SHAPE), (dict(Bcap=-1), SHAPE),
    (dict(raw=Q["raw"] + 8), ALIGN), (dict(kl=Q["kl"] + 4), ALIGN), (dict(rc=Q["rc"] + 2), ALIGN),
    (dict(nraw=Q["praw"]), ALIAS), (dict(bk=Q["raw"] + 64), ALIAS), (dict(nrope=Q["prope"]), ALIAS),
    (dict(nraw=Q["bk"] + 1024), ALIAS), (dict(err=Q["bk"]), ALIAS),
    (dict(N=0), OK), (dict(L=0), OK), (dict(L=0, raw=None), OK),
])
def test_qsa_validation(over, want):
    assert qsa(**over) == want


@pytest.mark.parametrize("over", [
    dict(L=1 << 31), dict(kbs=1 << 31), dict(kbs=(1 << 62) + 1),
    # N * Bcap * Di * 2 passes 2^63
    dict(N=3, klc=3, Bcap=1 << 62), dict(N=1, klc=1, L=(1 << 31) - 1, Bcap=1 << 50, Di=4096),
])
def test_qsa_validation_at_the_caps(over):
    assert qsa(**over) == SHAPE



@pytest.mark.parametrize("x,code,n,want", [
    (A["kv"], A["ckv"], 3, SHAPE), (A["kv"], A["ckv"], -4, SHAPE), (None, A["ckv"], 4, NULL),
    (A["kv"], None, 4, NULL), (A["kv"] + 4, A["ckv"], 4, ALIGN), (A["kv"], A["ckv"] + 2, 4, ALIGN),
    (A["kv"], A["kv"] + 12, 4, ALIAS), (A["kv"] + 16, A["kv"], 64, ALIAS),
    (A["kv"], A["ckv"], 0, OK), (None, None, 0, OK),
])
def test_selftest_e4m3_validation(x, code, n, want):
    assert k.lib().kvrc_selftest_e4m3(x, code, n, None) == want


def test_mla_noalloc_validation():
    """The allocation-free MLA head: the MLA head's checks, T up to 2^17 (its
    static workspace), and no workspace arguments."""
    L = k.lib()

    def call(**over):
        a = dict(x=M["x"], w=M["w"], gamma=M["gamma"], alpha=1.0, cos=M["cos"], sin=M["sin"],
                 slot=M["slot"], kc=M["kc"], ckv=M["ckv"], sc=None, T=300, He=7168, NB=64,
                 BS=128, dt=0, eps=1e-6, err=None, stream=None)
        a.update(over)
        return L.kvrc_mla_kv_head_paged_noalloc(
            a["x"], a["w"], a["gamma"], a["alpha"], a["cos"], a["sin"], a["slot"], a["kc"],
            a["ckv"], a["sc"], a["T"], a["He"], a["NB"], a["BS"], a["dt"], a["eps"], a["err"],
            a["stream"])

    assert k.MLA_NOALLOC_MAX_TOKENS == 1 << 17
    assert call(T=(1 << 17) + 1, He=64) == WORKSPACE
    assert call(T=-1) == SHAPE
    assert call(He=16) == SHAPE
    assert call(x=None) == NULL
    assert call(slot=M["slot"] + 4) == ALIGN
    assert call(dt=1) == DTYPE
    assert call(kc=M["x"] + 4096) == ALIAS
    assert call(T=0) == OK and call(T=0, x=None) == OK


def test_selftest_mla_stalled_validation():
    """The stalled selftest takes the MLA head's checks, plus its own."""
    L = k.lib()

    def call(**over):
        a = dict(x=M["x"], w=M["w"], gamma=M["gamma"], alpha=1.0, cos=M["cos"], sin=M["sin"],
                 slot=M["slot"], kc=M["kc"], ckv=M["ckv"], sc=None, T=300, He=7168, NB=64,
                 BS=128, dt=0, eps=1e-6, ws=M["ws"], wsb=WS_300, err=None, stall=100,
                 steals=None, stream=None)
        a.update(over)
        return L.kvrc_selftest_mla_kv_head_stalled(
            a["x"], a["w"], a["gamma"], a["alpha"], a["cos"], a["sin"], a["slot"], a["kc"],
            a["ckv"], a["sc"], a["T"], a["He"], a["NB"], a["BS"], a["dt"], a["eps"], a["ws"],
            a["wsb"], a["err"], a["stall"], a["steals"], a["stream"])

    assert call(stall=-1) == SHAPE
    assert call(stall=10 ** 7 + 1) == SHAPE
    assert call(steals=M["err"] + 2) == ALIGN
    assert call(He=16) == SHAPE
    assert call(wsb=WS_300 - 1) == WORKSPACE
    assert call(ws=M["x"]) == ALIAS
    assert call(T=0) == OK


@pytest.mark.parametrize("wg,threads,want", [
    (0, 256, SHAPE), (-1, 64, SHAPE), (1 << 31, 64, SHAPE), (1, 0, SHAPE), (1, 1025, SHAPE),
])
def test_selftest_empty_validation(wg, threads, want):
    assert k.lib().kvrc_selftest_empty(wg, threads, None) == want


@pytest.mark.parametrize("src,dst,n,want", [
    (A["kv"], A["ckv"], 8, SHAPE), (A["kv"], A["ckv"], -16, SHAPE),
    (A["kv"], A["ckv"], (1 << 40) + 16, SHAPE), (None, A["ckv"], 16, NULL),
    (A["kv"], None, 16, NULL), (A["kv"] + 8, A["ckv"], 16, ALIGN), (A["kv"], A["ckv"] + 4, 16, ALIGN),
    (A["kv"], A["kv"] + 16, 32, ALIAS), (A["kv"] + 16, A["kv"], 32, ALIAS),
    (A["kv"], A["ckv"], 0, OK), (None, None, 0, OK),
])
def test_selftest_copy_validation(src, dst, n, want):
    assert k.lib().kvrc_selftest_copy(src, dst, n, None) == want


def test_binding_refuses_cpu_tensors():
    bf = torch.bfloat16
    kv = torch.zeros(1, 1, 2, 576, dtype=bf)
    with pytest.raises(ValueError, match="GPU"):
        k.kvrc_paged_norm_rope_cache(kv, torch.zeros(512, dtype=bf), torch.zeros(1, 1, 2, 64, dtype=bf),
                                     torch.zeros(1, 1, 2, 64, dtype=bf),
                                     torch.zeros(2, dtype=torch.int64),
                                     torch.zeros(4, 4, 1, 64, dtype=bf),
                                     torch.zeros(4, 4, 1, 512, dtype=bf))


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(k, "_lib", None)
    monkeypatch.setattr(k, "LIB_PATH", "/nonexistent/libkvrc.so")
    with pytest.raises(RuntimeError, match="not built"):
        k.lib()


def test_product_does_not_import_oracle():
    """The library package never reaches the oracle (no CPU fallback)."""
    pkg = os.path.join(ROOT, "latent_attention_kv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", src, re.M), f
                assert "liboracle" not in src and "kvrc_oracle" not in src, f
