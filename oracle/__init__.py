"""ctypes binding of the CPU oracle (``oracle/kvrc_oracle.c``); the MLA
kv-path head and block-selection oracles (float64, numpy) are
``oracle/mla_kv_head.py`` and ``oracle/qsa_select.py``.

TEST INFRASTRUCTURE ONLY: the plain CPU definition that the HIP library is
checked against. Only the tests, ``__graft_entry__.smoke()`` and the bench's
CPU-baseline leg may import this module. The library (``latent_attention_kv_amd``)
never imports it and shares no code with it.

Every function is pinned by ``tests/test_oracle_*.py``; none is parity
unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvrc_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_kvrc.so")
_lib = None

STATUS = {0: "ok", 1: "bad argument", 2: "index out of range", 3: "duplicate index",
          4: "bad key_length"}


class OracleError(RuntimeError):
    pass


# Host sanitizers for a checking build of the oracle: address errors and
# undefined behaviour abort the process (no recovery).
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]


def build(verbose: bool = False, sanitize: bool = False, out: str | None = None) -> str:
    """Compile the oracle with gcc (float32, no contraction, OpenMP over rows).
    sanitize=True builds a checking copy with SANITIZE_FLAGS at `out` (it must
    be loaded into a process that preloads the sanitizer runtimes)."""
    path = out or _LIB_PATH
    opt = SANITIZE_FLAGS if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-fopenmp", "-o", path + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(path + ".tmp", path)
    return path


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    F = ctypes.c_float
    I = ctypes.c_int
    lib.orc_sumsq_canonical.argtypes = [P, I64]
    lib.orc_sumsq_canonical.restype = F
    lib.orc_rmsnorm_f32.argtypes = [P, P, I64, F, P]
    lib.orc_rope_f32.argtypes = [P, P, P, I64, P]
    lib.orc_quant_row.argtypes = [P, I64, P, P]
    lib.orc_token_outputs.argtypes = [P, P, P, P, I64, I64, F, P, P]
    lib.orc_paged_norm_rope_cache.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I64,
                                              I64, I64, I, F, I]
    lib.orc_norm_rope_cache.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64,
                                        I64, I, F, I]
    lib.orc_paged_blk_norm_rope_cache.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I64,
                                                  I64, I64, I, F, I]
    lib.orc_qsa_prepare.argtypes = [P, P, P, I64, P, P, P, P, P, P, P, I64, I64, I64, I64,
                                    I64, I64, F, I]
    lib.orc_qsa_block_key.argtypes = [P, I64, I64, P, P, P, I64, F, P, P]
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_decode.restype = F
    lib.orc_e4m3_encode.argtypes = [F]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_quant_row_fp8.argtypes = [P, I64, P, P]
    lib.orc_e4m3_encode_array.argtypes = [P, P, I64, I]
    lib.orc_f32_to_bf16_array.argtypes = [P, P, I64]
    lib.orc_bf16_to_f32_array.argtypes = [P, P, I64]
    lib.orc_max_threads.restype = I
    _lib = lib
    return lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def max_threads() -> int:
    return int(_load().orc_max_threads())


# ----------------------------------------------------------------- formats

def f32_to_bf16(a) -> np.ndarray:
    a = _f32(a)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().orc_f32_to_bf16_array(_p(a), _p(out), a.size)
    return out


def bf16_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    _load().orc_bf16_to_f32_array(_p(b), _p(out), b.size)
    return out


# ---------------------------------------------------------- row building blocks

def sumsq(v) -> np.float32:
    v = _f32(v)
    return np.float32(_load().orc_sumsq_canonical(_p(v), v.size))


def rmsnorm(x, w=None, eps=1e-6) -> np.ndarray:
    x = _f32(x)
    w = None if w is None else _f32(w)
    y = np.empty_like(x)
    _load().orc_rmsnorm_f32(_p(x), _p(w), x.size, eps, _p(y))
    return y


def rope(x, c, s) -> np.ndarray:
    x, c, s = _f32(x), _f32(c), _f32(s)
    assert x.size % 2 == 0 and c.size == x.size and s.size == x.size
    y = np.empty_like(x)
    _load().orc_rope_f32(_p(x), _p(c), _p(s), x.size, _p(y))
    return y


def quant_row(y):
    y = _f32(y)
    code = np.empty(y.shape, dtype=np.int8)
    scale = np.zeros(1, dtype=np.float32)
    _load().orc_quant_row(_p(y), y.size, _p(code), _p(scale))
    return code, np.float32(scale[0])


def e4m3_decode(code) -> np.float32:
    return np.float32(_load().orc_e4m3_decode(int(code) & 0xFF))


def e4m3_encode(v) -> int:
    return int(_load().orc_e4m3_encode(float(np.float32(v))))


def e4m3_encode_array(v, nthreads=None) -> np.ndarray:
    v = _f32(v)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().orc_e4m3_encode_array(_p(v), _p(out), v.size, nthreads or max_threads())
    return out


def quant_row_fp8(y):
    y = _f32(y)
    code = np.empty(y.shape, dtype=np.uint8)
    scale = np.zeros(1, dtype=np.float32)
    _load().orc_quant_row_fp8(_p(y), y.size, _p(code), _p(scale))
    return code, np.float32(scale[0])


def token_outputs(kv_row, gamma, cos_row, sin_row, Dv, Dk, eps=1e-6):
    """float32 (pre-rounding) outputs of one token: rmsnorm(Dv) and rope(Dk)."""
    kv_row = np.ascontiguousarray(kv_row, dtype=np.uint16)
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    cos_row = np.ascontiguousarray(cos_row, dtype=np.uint16)
    sin_row = np.ascontiguousarray(sin_row, dtype=np.uint16)
    yn = np.empty(Dv, dtype=np.float32)
    yr = np.empty(Dk, dtype=np.float32)
    _load().orc_token_outputs(_p(kv_row), _p(gamma), _p(cos_row), _p(sin_row), Dv, Dk, eps,
                              _p(yn), _p(yr))
    return yn, yr


def qsa_block_key(rows, w=None, c=None, s=None, eps=1e-6):
    """One block key from rows [kbs, Di] (bf16 bits): returns (mean, key) float32."""
    rows = np.ascontiguousarray(rows, dtype=np.uint16)
    kbs, Di = rows.shape
    w = None if w is None else _f32(w)
    Dr = 0
    if c is not None:
        c, s = _f32(c), _f32(s)
        Dr = c.size
    m = np.empty(Di, dtype=np.float32)
    z = np.empty(Di, dtype=np.float32)
    _load().orc_qsa_block_key(_p(rows), kbs, Di, _p(w), _p(c), _p(s), Dr, eps, _p(m), _p(z))
    return m, z


# ------------------------------------------------------------------ whole ops

def _check(rc):
    if rc != 0:
        raise OracleError(f"oracle status {rc}: {STATUS.get(rc, '?')}")


def _ckv_kind(ckv_cache) -> int:
    """0: bf16 bits (uint16), 1: int8 codes, 2: FLOAT8 E4M3FN codes (uint8)."""
    return {np.dtype(np.uint16): 0, np.dtype(np.int8): 1, np.dtype(np.uint8): 2}[ckv_cache.dtype]


def paged_norm_rope_cache(kv, gamma, cos, sin, slot_mapping, k_cache, ckv_cache,
                          ckv_scale=None, *, eps=1e-6, nthreads=None):
    """Update k_cache / ckv_cache (/ ckv_scale) in place. Shapes:
    kv [B,1,S,Dv+Dk] u16; cos/sin [B,1,S,Dk] u16; slot_mapping [B*S] i64;
    k_cache [NB,BS,1,Dk] u16; ckv_cache [NB,BS,1,Dv] u16 or i8; ckv_scale [NB,BS,1] f32."""
    B, _, S, D = kv.shape
    Dk = cos.shape[-1]
    Dv = D - Dk
    NB, BS = k_cache.shape[0], k_cache.shape[1]
    int8 = _ckv_kind(ckv_cache)
    rc = _load().orc_paged_norm_rope_cache(
        _p(kv), _p(gamma), _p(cos), _p(sin), _p(slot_mapping), _p(k_cache), _p(ckv_cache),
        _p(ckv_scale), B, S, Dv, Dk, NB, BS, int(int8), eps,
        nthreads or max_threads())
    _check(rc)


def paged_blk_norm_rope_cache(kv, gamma, cos, sin, block_index, k_cache, ckv_cache,
                              ckv_scale=None, *, eps=1e-6, nthreads=None):
    """Block-indexed paged mode: block_index [B * ceil(S / block_size)]."""
    B, _, S, D = kv.shape
    Dk = cos.shape[-1]
    Dv = D - Dk
    NB, BS = k_cache.shape[0], k_cache.shape[1]
    int8 = _ckv_kind(ckv_cache)
    rc = _load().orc_paged_blk_norm_rope_cache(
        _p(kv), _p(gamma), _p(cos), _p(sin), _p(block_index), _p(k_cache), _p(ckv_cache),
        _p(ckv_scale), B, S, Dv, Dk, NB, BS, int(int8), eps, nthreads or max_threads())
    _check(rc)


def norm_rope_cache(kv, gamma, cos, sin, index, k_cache, ckv_cache, ckv_scale=None, *,
                    eps=1e-6, nthreads=None):
    """Norm mode: index [B,S]; caches [Bc,1,Sc,d]; ckv_scale [Bc,1,Sc]."""
    B, _, S, D = kv.shape
    Dk = cos.shape[-1]
    Dv = D - Dk
    Bc, Sc = k_cache.shape[0], k_cache.shape[2]
    int8 = _ckv_kind(ckv_cache)
    rc = _load().orc_norm_rope_cache(
        _p(kv), _p(gamma), _p(cos), _p(sin), _p(index), _p(k_cache), _p(ckv_cache),
        _p(ckv_scale), B, S, Dv, Dk, Bc, Sc, int(int8), eps, nthreads or max_threads())
    _check(rc)


def qsa_prepare(raw_index_keys, block_keys, key_length, rope_cos, rope_sin, k_norm_weight,
                past_incomplete_raw_keys, past_incomplete_rope, next_incomplete_raw_keys,
                next_incomplete_rope, *, key_block_size, eps=1e-6, nthreads=None):
    """Writes block_keys [N,Bcap,Di] rows of the completed blocks and the next
    carry state, in place."""
    N, L, Di = raw_index_keys.shape
    Bcap = block_keys.shape[1]
    Dr = 0 if rope_cos is None else rope_cos.shape[-1]
    rc = _load().orc_qsa_prepare(
        _p(raw_index_keys), _p(block_keys), _p(key_length), key_length.size, _p(rope_cos),
        _p(rope_sin), _p(k_norm_weight), _p(past_incomplete_raw_keys),
        _p(past_incomplete_rope), _p(next_incomplete_raw_keys), _p(next_incomplete_rope),
        N, L, Di, Dr, Bcap, key_block_size, eps, nthreads or max_threads())
    _check(rc)


# ------------------------------------------------------- convenience drivers

def run_kvrc_case(case, nthreads=None):
    """Run a gen.kvrc_*_case dict through the oracle; returns the cache arrays."""
    caches = {k: spec.numpy() for k, spec in case["caches"].items()}
    args = (case["kv"], case["gamma"], case["cos"], case["sin"])
    if case["mode"] == "paged":
        paged_norm_rope_cache(*args, case["slot_mapping"], caches["k_cache"],
                              caches["ckv_cache"], caches.get("ckv_scale"), eps=case["eps"],
                              nthreads=nthreads)
    elif case["mode"] == "paged_blk":
        paged_blk_norm_rope_cache(*args, case["block_index"], caches["k_cache"],
                                  caches["ckv_cache"], caches.get("ckv_scale"),
                                  eps=case["eps"], nthreads=nthreads)
    else:
        norm_rope_cache(*args, case["index"], caches["k_cache"], caches["ckv_cache"],
                        caches.get("ckv_scale"), eps=case["eps"], nthreads=nthreads)
    return caches


def run_qsa_case(case, nthreads=None):
    """Run a gen.qsa_case dict through the oracle; returns (block_keys,
    next_raw, next_rope) with next_* pre-filled like the generator's state."""
    N, Di, kbs, Dr = case["N"], case["Di"], case["kbs"], case["Dr"]
    bk = case["caches"]["block_keys"].numpy()
    next_raw = np.full((N, kbs - 1, Di), 0x7FC0, dtype=np.uint16)
    next_rope = None
    if case["rope_cos"] is not None:
        next_rope = np.full((N, 2 * Dr), np.nan, dtype=np.float32)
    qsa_prepare(case["raw_index_keys"], bk, case["key_length"], case["rope_cos"],
                case["rope_sin"], case["k_norm_weight"], case["past_incomplete_raw_keys"],
                case["past_incomplete_rope"], next_raw, next_rope,
                key_block_size=kbs, eps=case["eps"], nthreads=nthreads)
    return bk, next_raw, next_rope
