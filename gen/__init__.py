"""Seeded synthetic inputs for the KV preprocessing path and QSA block keys.

This module only *draws* inputs. It holds none of the method's arithmetic:
no normalisation, no rotation, no quantisation and no scatter. Both the CPU
oracle (``oracle/``) and the HIP library are fed from here, and nothing here
imports either of them.

Conventions
-----------
* Random numbers come from ``numpy.random.Generator(PCG64(seed))``; the draw
  order inside each builder is fixed, so a (builder, seed) pair always yields
  the same bytes.
* bf16 tensors are stored as ``uint16`` bit patterns, rounded from float32
  with round-to-nearest-even (``bf16_bits``).
* RoPE tables follow the usual angle rule ``angle_i = pos * 10000^(-2i/d)``
  for pair index ``i < d/2``; the table row has full width ``d`` with the two
  halves duplicated (``tab[j] = f(angle_{j mod d/2})``), which is the layout
  under which the interleaved RoPE of the aclnnKvRmsNormRopeCache page
  (Formulas (1) interleaveRope) rotates each (x[2i], x[2i+1]) pair.
  Angles and cos/sin are evaluated in float64, rounded to float32, and (where
  a bf16 table is wanted) rounded again to bf16.
* Caches are pre-filled with sentinels that the method never produces:
  bf16 7.0, int8 -128, FLOAT8 E4M3FN code 0x7f (NaN), scale -1.0.
"""
from __future__ import annotations

import numpy as np

BF16_SENTINEL = 0x40E0          # 7.0 in bf16
BF16_NAN = 0x7FC0
INT8_SENTINEL = -128
FP8_SENTINEL = 0x7F             # E4M3FN NaN code
SCALE_SENTINEL = -1.0

CONFIG_NAMES = ("norm_tiny", "decode_paged", "prefill_paged", "quant_paged", "qsa")
EXTRA_NAMES = ("prefill_paged_blk", "quant_fp8_paged", "mla_kv_head", "qsa_select")


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even; NaN kept quiet."""
    u = np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bits_to_f32(b) -> np.ndarray:
    """bf16 bit pattern -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def rope_table_f64(pos, d: int):
    """cos and sin tables, float64, shape pos.shape + (d,), duplicated halves."""
    pos = np.asarray(pos, dtype=np.float64)
    h = d // 2
    i = np.arange(d) % h
    inv = np.power(10000.0, -2.0 * i / d)
    ang = np.ascontiguousarray(pos[..., None] * inv)
    return np.ascontiguousarray(np.cos(ang)), np.ascontiguousarray(np.sin(ang))


def rope_table_bf16(pos, d: int):
    c, s = rope_table_f64(pos, d)
    return bf16_bits(c.astype(np.float32)), bf16_bits(s.astype(np.float32))


def rope_table_f32(pos, d: int):
    c, s = rope_table_f64(pos, d)
    return (np.ascontiguousarray(c, dtype=np.float32), np.ascontiguousarray(s, dtype=np.float32))


class CacheSpec:
    """Shape, numpy dtype and fill value of a cache the caller allocates."""

    def __init__(self, shape, dtype, fill):
        self.shape = tuple(int(x) for x in shape)
        self.dtype = np.dtype(dtype)
        self.fill = fill

    def numpy(self) -> np.ndarray:
        return np.full(self.shape, self.fill, dtype=self.dtype)

    @property
    def nbytes(self) -> int:
        return int(np.prod(self.shape)) * self.dtype.itemsize


# ---------------------------------------------------------------------------
# Norm-rope-cache cases
# ---------------------------------------------------------------------------

def ckv_cache_spec(shape, ckv_dtype):
    """ckv cache of the given element type ("bf16", "int8" or "fp8" = E4M3FN codes)."""
    if ckv_dtype == "bf16":
        return CacheSpec(shape, np.uint16, BF16_SENTINEL)
    if ckv_dtype == "int8":
        return CacheSpec(shape, np.int8, INT8_SENTINEL)
    if ckv_dtype == "fp8":
        return CacheSpec(shape, np.uint8, FP8_SENTINEL)
    raise ValueError(ckv_dtype)


def _kv_common(g, B, S, Dv, Dk, sigma):
    kv = bf16_bits(g.standard_normal((B, 1, S, Dv + Dk), dtype=np.float32) * np.float32(sigma))
    gamma = bf16_bits(g.uniform(0.5, 1.5, size=(Dv,)).astype(np.float32))
    return kv, gamma


def kvrc_norm_case(seed, B, S, Dv, Dk, Bc, Sc, n_skip, *, eps=1e-6, sigma=1.0,
                   ckv_dtype="bf16", positions=None):
    """Norm (contiguous) cache mode: index[b, s] in [-1, Sc), distinct per row."""
    g = rng_for(seed)
    kv, gamma = _kv_common(g, B, S, Dv, Dk, sigma)
    if positions is None:
        positions = np.broadcast_to(np.arange(S), (B, S))
    cos, sin = rope_table_bf16(np.asarray(positions).reshape(B, 1, S), Dk)
    index = np.stack([g.permutation(Sc)[:S] for _ in range(B)]).astype(np.int64)
    if n_skip:
        flat = g.choice(B * S, size=n_skip, replace=False)
        index.reshape(-1)[flat] = -1
    caches = {
        "k_cache": CacheSpec((Bc, 1, Sc, Dk), np.uint16, BF16_SENTINEL),
        "ckv_cache": ckv_cache_spec((Bc, 1, Sc, Dv), ckv_dtype),
    }
    if ckv_dtype != "bf16":
        caches["ckv_scale"] = CacheSpec((Bc, 1, Sc), np.float32, SCALE_SENTINEL)
    return dict(mode="norm", kv=kv, gamma=gamma, cos=cos, sin=sin, index=index,
                caches=caches, B=B, S=S, Dv=Dv, Dk=Dk, Bc=Bc, Sc=Sc, eps=float(eps),
                ckv_dtype=ckv_dtype)


def kvrc_paged_case(seed, B, S, Dv, Dk, num_blocks, block_size, *, eps=1e-6, sigma=1.0,
                    ckv_dtype="bf16", slot_kind="table", skip_frac=0.0, positions=None,
                    max_pos=32768):
    """Paged (PA_BNSD, N=1) cache mode.

    slot_kind "table": every sequence owns ceil(S/block_size) distinct random
    blocks and slot = block*block_size + s % block_size (prefill layout).
    slot_kind "random": B*S unique random slots over the whole pool, with
    round(skip_frac*B*S) of them set to -1; positions ~ U{0..max_pos-1}
    (decode layout).
    """
    g = rng_for(seed)
    kv, gamma = _kv_common(g, B, S, Dv, Dk, sigma)
    T = B * S
    if slot_kind == "table":
        per_seq = -(-S // block_size)
        blocks = g.choice(num_blocks, size=B * per_seq, replace=False).reshape(B, per_seq)
        s = np.arange(S)
        slots = (blocks[:, s // block_size] * block_size + (s % block_size)[None, :]).reshape(T)
        if positions is None:
            positions = np.broadcast_to(np.arange(S), (B, S))
    elif slot_kind == "random":
        slots = g.choice(num_blocks * block_size, size=T, replace=False)
        if positions is None:
            positions = g.integers(0, max_pos, size=(B, S))
        blocks = None
    else:
        raise ValueError(slot_kind)
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    n_skip = int(round(skip_frac * T))
    if n_skip:
        slots[g.choice(T, size=n_skip, replace=False)] = -1
    cos, sin = rope_table_bf16(np.asarray(positions).reshape(B, 1, S), Dk)
    caches = {
        "k_cache": CacheSpec((num_blocks, block_size, 1, Dk), np.uint16, BF16_SENTINEL),
        "ckv_cache": ckv_cache_spec((num_blocks, block_size, 1, Dv), ckv_dtype),
    }
    if ckv_dtype != "bf16":
        caches["ckv_scale"] = CacheSpec((num_blocks, block_size, 1), np.float32, SCALE_SENTINEL)
    return dict(mode="paged", kv=kv, gamma=gamma, cos=cos, sin=sin, slot_mapping=slots,
                caches=caches, B=B, S=S, Dv=Dv, Dk=Dk, num_blocks=num_blocks,
                block_size=block_size, eps=float(eps), ckv_dtype=ckv_dtype,
                block_table=blocks)


def kvrc_paged_blk_case(seed, B, S, Dv, Dk, num_blocks, block_size, *, eps=1e-6, sigma=1.0,
                        ckv_dtype="bf16", n_skip=0, entry_offsets=False):
    """Block-indexed paged mode (PA_BLK_BNSD): one index entry per chunk of
    block_size tokens of a sequence, B * ceil(S/block_size) entries naming
    distinct random blocks (entry = block*block_size, plus a random offset in
    [0, block_size) when entry_offsets), n_skip entries set to -1;
    positions 0..S-1 per sequence."""
    g = rng_for(seed)
    kv, gamma = _kv_common(g, B, S, Dv, Dk, sigma)
    chunks = -(-S // block_size)
    blocks = g.choice(num_blocks, size=B * chunks, replace=False)
    entries = (blocks * block_size).astype(np.int64)
    if entry_offsets:
        entries += g.integers(0, block_size, size=entries.shape)
    if n_skip:
        entries[g.choice(B * chunks, size=n_skip, replace=False)] = -1
    positions = np.broadcast_to(np.arange(S), (B, S))
    cos, sin = rope_table_bf16(np.asarray(positions).reshape(B, 1, S), Dk)
    caches = {
        "k_cache": CacheSpec((num_blocks, block_size, 1, Dk), np.uint16, BF16_SENTINEL),
        "ckv_cache": ckv_cache_spec((num_blocks, block_size, 1, Dv), ckv_dtype),
    }
    if ckv_dtype != "bf16":
        caches["ckv_scale"] = CacheSpec((num_blocks, block_size, 1), np.float32, SCALE_SENTINEL)
    return dict(mode="paged_blk", kv=kv, gamma=gamma, cos=cos, sin=sin,
                block_index=np.ascontiguousarray(entries), caches=caches, B=B, S=S, Dv=Dv,
                Dk=Dk, num_blocks=num_blocks, block_size=block_size, eps=float(eps),
                ckv_dtype=ckv_dtype)


# ---------------------------------------------------------------------------
# MLA kv-path head cases
# ---------------------------------------------------------------------------

def mla_kv_head_case(seed, B, S, He, num_blocks, block_size, *, eps=1e-6, alpha=0.875,
                     slot_kind="table", skip_frac=0.0, max_pos=32768, x_sigma=1.0,
                     ckv_dtype="bf16"):
    """Inputs of the MLA kv-path head for T = B*S tokens of hidden size He.

    x [T, He] bf16 ~ N(0, x_sigma); the fused projection weight
    w [576, He] bf16 ~ N(0, 1/He) (random init, row j produces output
    column j: rows 0..511 the compressed kv, rows 512..575 the rope key);
    gamma ~ U(0.5, 1.5); alpha a float32 scalar; cos/sin [T, 64] bf16 and the
    slot mapping as in kvrc_paged_case (table or random slots); bf16 paged
    caches [num_blocks, block_size, 1, d].
    """
    Dv, Dk = 512, 64
    g = rng_for(seed)
    T = B * S
    x = bf16_bits(g.standard_normal((T, He), dtype=np.float32) * np.float32(x_sigma))
    w = bf16_bits(g.standard_normal((Dv + Dk, He), dtype=np.float32)
                  * np.float32(1.0 / np.sqrt(He)))
    gamma = bf16_bits(g.uniform(0.5, 1.5, size=(Dv,)).astype(np.float32))
    if slot_kind == "table":
        per_seq = -(-S // block_size)
        blocks = g.choice(num_blocks, size=B * per_seq, replace=False).reshape(B, per_seq)
        s = np.arange(S)
        slots = (blocks[:, s // block_size] * block_size + (s % block_size)[None, :]).reshape(T)
        positions = np.broadcast_to(np.arange(S), (B, S))
    elif slot_kind == "random":
        slots = g.choice(num_blocks * block_size, size=T, replace=False)
        positions = g.integers(0, max_pos, size=(B, S))
    else:
        raise ValueError(slot_kind)
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    n_skip = int(round(skip_frac * T))
    if n_skip:
        slots[g.choice(T, size=n_skip, replace=False)] = -1
    cos, sin = rope_table_bf16(np.asarray(positions).reshape(B, 1, S), Dk)
    caches = {
        "k_cache": CacheSpec((num_blocks, block_size, 1, Dk), np.uint16, BF16_SENTINEL),
        "ckv_cache": ckv_cache_spec((num_blocks, block_size, 1, Dv), ckv_dtype),
    }
    if ckv_dtype != "bf16":
        caches["ckv_scale"] = CacheSpec((num_blocks, block_size, 1), np.float32, SCALE_SENTINEL)
    return dict(mode="mla_paged", ckv_dtype=ckv_dtype, x=x, w=w, gamma=gamma,
                alpha=float(np.float32(alpha)),
                cos=np.ascontiguousarray(cos.reshape(T, Dk)),
                sin=np.ascontiguousarray(sin.reshape(T, Dk)), slot_mapping=slots,
                caches=caches, B=B, S=S, T=T, He=He, Dv=Dv, Dk=Dk, num_blocks=num_blocks,
                block_size=block_size, eps=float(eps))


def mla_kv_head_blk_case(seed, B, S, He, num_blocks, block_size, *, eps=1e-6, alpha=0.875,
                         n_skip=0, entry_offsets=False, x_sigma=1.0, ckv_dtype="bf16"):
    """The MLA kv-path head with the block-indexed placement: x [B*S, He]
    (batch-major), positions 0..S-1 per sequence, one cache-index entry per
    chunk of block_size tokens (B * ceil(S/block_size) entries naming
    distinct random blocks: entry = block*block_size, plus a random offset in
    [0, block_size) when entry_offsets), n_skip entries set to -1."""
    Dv, Dk = 512, 64
    g = rng_for(seed)
    T = B * S
    x = bf16_bits(g.standard_normal((T, He), dtype=np.float32) * np.float32(x_sigma))
    w = bf16_bits(g.standard_normal((Dv + Dk, He), dtype=np.float32)
                  * np.float32(1.0 / np.sqrt(He)))
    gamma = bf16_bits(g.uniform(0.5, 1.5, size=(Dv,)).astype(np.float32))
    chunks = -(-S // block_size)
    blocks = g.choice(num_blocks, size=B * chunks, replace=False)
    entries = (blocks * block_size).astype(np.int64)
    if entry_offsets:
        entries += g.integers(0, block_size, size=entries.shape)
    if n_skip:
        entries[g.choice(B * chunks, size=n_skip, replace=False)] = -1
    positions = np.broadcast_to(np.arange(S), (B, S))
    cos, sin = rope_table_bf16(np.asarray(positions).reshape(B, 1, S), Dk)
    caches = {
        "k_cache": CacheSpec((num_blocks, block_size, 1, Dk), np.uint16, BF16_SENTINEL),
        "ckv_cache": ckv_cache_spec((num_blocks, block_size, 1, Dv), ckv_dtype),
    }
    if ckv_dtype != "bf16":
        caches["ckv_scale"] = CacheSpec((num_blocks, block_size, 1), np.float32, SCALE_SENTINEL)
    return dict(mode="mla_paged_blk", ckv_dtype=ckv_dtype, x=x, w=w, gamma=gamma,
                alpha=float(np.float32(alpha)),
                cos=np.ascontiguousarray(cos.reshape(T, Dk)),
                sin=np.ascontiguousarray(sin.reshape(T, Dk)),
                block_index=np.ascontiguousarray(entries), caches=caches, B=B, S=S, T=T, He=He,
                Dv=Dv, Dk=Dk, num_blocks=num_blocks, block_size=block_size, eps=float(eps))


# ---------------------------------------------------------------------------
# Block selection over QSA block keys
# ---------------------------------------------------------------------------

def qsa_select_case(seed, N, H, Di, Bcap, kbs, sel_ratio, cmp_ratio, topk, *, kl_lo=None,
                    kl_hi=None, key_length_count=None, scale=None, key_sigma=1.0):
    """One query per sequence and head, q [N, H, Di] ~ N(0,1) bf16, scored
    against block keys [N, Bcap, Di] ~ N(0, key_sigma) bf16; the rows at or
    beyond a sequence's block count are NaN (never to be read).
    key_length ~ U{kl_lo .. kl_hi - 1} (default: 0 .. Bcap * kbs), so a
    sequence has key_length // kbs complete blocks. scale defaults to
    1 / sqrt(Di)."""
    g = rng_for(seed)
    if kl_lo is None:
        kl_lo = 0
    if kl_hi is None:
        kl_hi = Bcap * kbs + 1
    q = bf16_bits(g.standard_normal((N, H, Di), dtype=np.float32))
    keys = bf16_bits(g.standard_normal((N, Bcap, Di), dtype=np.float32) * np.float32(key_sigma))
    kl = g.integers(kl_lo, kl_hi, size=N).astype(np.int64)
    if key_length_count == 1:
        kl = kl[:1].copy()
    for n in range(N):
        nb = int(kl[n % len(kl)]) // kbs
        keys[n, nb:] = BF16_NAN
    Jcap = (Bcap + sel_ratio + cmp_ratio - 3) // sel_ratio + 1 if Bcap > 0 else 0
    if scale is None:
        scale = 1.0 / np.sqrt(Di)
    return dict(query=q, block_keys=keys, key_length=kl, N=N, H=H, Di=Di, Bcap=Bcap, kbs=kbs,
                sel_ratio=sel_ratio, cmp_ratio=cmp_ratio, topk=topk, Jcap=Jcap,
                scale=float(np.float32(scale)))


# ---------------------------------------------------------------------------
# QSA block-key cases
# ---------------------------------------------------------------------------

def qsa_case(seed, N, L, Di, Dr, kbs, *, past_max=8192, Bcap=None, eps=1e-6,
             rope=True, norm=True, key_length_count=None):
    """QSAPrepare inputs for N sequences of L new tokens each.

    past ~ U{0..past_max-1}; key_length = past + L. The carried raw rows
    (past % kbs of them) are N(0,1); invalid carried rows and an unused
    carried rope row are NaN, so a reader of invalid state shows up.
    RoPE tables are float32 at absolute positions past + j; the carried rope
    row is cos || sin at the first position of the incomplete block.
    """
    g = rng_for(seed)
    raw = bf16_bits(g.standard_normal((N, L, Di), dtype=np.float32))
    if key_length_count == 1:
        past = np.full(N, int(g.integers(0, past_max)), dtype=np.int64)
    else:
        past = g.integers(0, past_max, size=N).astype(np.int64)
    key_length = (past + L).astype(np.int64)
    if key_length_count == 1:
        key_length = key_length[:1].copy()
    r = past % kbs
    pinc = np.full((N, kbs - 1, Di), BF16_NAN, dtype=np.uint16)
    cand = bf16_bits(g.standard_normal((N, kbs - 1, Di), dtype=np.float32))
    for n in range(N):
        pinc[n, : r[n]] = cand[n, : r[n]]
    w = bf16_bits(g.uniform(0.5, 1.5, size=(Di,)).astype(np.float32)) if norm else None
    if rope:
        pos = past[:, None] + np.arange(L)[None, :]
        rc, rs = rope_table_f32(pos, Dr)
        start = past - r
        sc, ss = rope_table_f32(start, Dr)
        prope = np.concatenate([sc, ss], axis=1).astype(np.float32)
        prope[r == 0] = np.nan
    else:
        rc = rs = prope = None
    if Bcap is None:
        Bcap = int((past.max() + L) // kbs) + 1 if N else 1
    caches = {"block_keys": CacheSpec((N, Bcap, Di), np.uint16, BF16_SENTINEL)}
    return dict(raw_index_keys=raw, key_length=key_length, past=past, rope_cos=rc,
                rope_sin=rs, k_norm_weight=w, past_incomplete_raw_keys=pinc,
                past_incomplete_rope=prope, caches=caches, N=N, L=L, Di=Di, Dr=Dr,
                kbs=kbs, Bcap=Bcap, eps=float(eps))


# ---------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------

def make_config(name: str, seed: int | None = None):
    """The named workloads, each with its own default seed."""
    if name == "norm_tiny":
        return kvrc_norm_case(1 if seed is None else seed, B=2, S=16, Dv=512, Dk=64,
                              Bc=2, Sc=32, n_skip=3)
    if name == "decode_paged":
        return kvrc_paged_case(2 if seed is None else seed, B=256, S=1, Dv=512, Dk=64,
                               num_blocks=4096, block_size=128, slot_kind="random",
                               skip_frac=0.05, max_pos=32768)
    if name == "prefill_paged":
        return kvrc_paged_case(3 if seed is None else seed, B=8, S=4096, Dv=512, Dk=64,
                               num_blocks=8192, block_size=128, slot_kind="table")
    if name == "quant_paged":
        return kvrc_paged_case(4 if seed is None else seed, B=64, S=1024, Dv=512, Dk=64,
                               num_blocks=4096, block_size=128, slot_kind="table",
                               sigma=2.0, ckv_dtype="int8")
    if name == "qsa":
        return qsa_case(5 if seed is None else seed, N=32, L=2048, Di=128, Dr=64, kbs=64,
                        past_max=8192, Bcap=160)
    if name == "quant_fp8_paged":
        # the quantised-cache batch with a FLOAT8 E4M3FN ckv cache
        return kvrc_paged_case(7 if seed is None else seed, B=64, S=1024, Dv=512, Dk=64,
                               num_blocks=4096, block_size=128, slot_kind="table",
                               sigma=2.0, ckv_dtype="fp8")
    if name == "mla_kv_head":
        # the prefill batch through the MLA kv-path head (DeepSeek-V3 hidden 7168)
        return mla_kv_head_case(8 if seed is None else seed, B=8, S=4096, He=7168,
                                num_blocks=8192, block_size=128)
    if name in ("mla_kv_head_int8", "mla_kv_head_fp8"):
        # the same head into an int8 (RowMax/127) or E4M3FN (RowMax/448) ckv cache
        kind = name.rsplit("_", 1)[1]
        return mla_kv_head_case((10 if kind == "int8" else 11) if seed is None else seed, B=8,
                                S=4096, He=7168, num_blocks=8192, block_size=128, ckv_dtype=kind)
    if name == "qsa_select":
        # decode-time block selection: 128 sequences, 64 query heads, up to
        # 256 blocks of 64 tokens, selection blocks of 128 tokens, top 16
        return qsa_select_case(9 if seed is None else seed, N=128, H=64, Di=128, Bcap=256,
                               kbs=64, sel_ratio=2, cmp_ratio=1, topk=16, kl_lo=4096,
                               kl_hi=16385)
    if name == "prefill_paged_blk":
        # the prefill batch in block-indexed form: one entry per 128-token chunk
        return kvrc_paged_blk_case(6 if seed is None else seed, B=8, S=4096, Dv=512, Dk=64,
                                   num_blocks=8192, block_size=128)
    raise KeyError(name)


def kvrc_bytes_per_written_token(Dv: int, Dk: int, ckv_dtype: str) -> int:
    """Algorithmic bytes one written token moves: kv + cos/sin + slot + outputs
    (a quantised ckv row is one byte per value plus its float32 scale)."""
    reads = 2 * (Dv + Dk) + 2 * 2 * Dk + 8
    writes = (2 * Dv if ckv_dtype == "bf16" else Dv + 4) + 2 * Dk
    return reads + writes
