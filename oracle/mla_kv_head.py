"""CPU oracle of the MLA kv-path head: projection, RmsNorm scaled by alpha_kv,
RoPE, paged cache scatter.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): only the tests,
``__graft_entry__.smoke()`` and the bench's CPU-baseline leg may use it; the
library never imports it and shares no code with it.

Source: aclnnMlaPrologV3WeightNz (Interface function: the third path, x times
W^DKV, RmsNorm, times the key scale factor alpha_kv, into the cache; the
fourth path, x times W^KR, ROPE, into the other cache; Formula: RmsNorm
formula, c^KV = alpha_kv * RmsNorm(x W^DKV), k^C = Cache(c^KV),
k^R = Cache(ROPE(x W^KR))), with the interleaved RoPE of
aclnnKvRmsNormRopeCache (Formula (1) interleaveRope) and its paged cache
placement (restrictions on index, PA_BNSD: slot -1 skips the token), or the
block-indexed placement (PA_BLK_BSND: one cache-index entry per chunk of
BlockSize tokens of a sequence).

Readings (the pages fix none of these):
  * precision: float64 throughout; the bf16 inputs widen exactly, the
    products x_k * w_kj of two bf16 values are exact, the projection is one
    float64 matrix product (a library routine), and each output is rounded to
    bf16 (nearest, ties to even) once, directly from float64;
  * the projection output is not rounded before the norm (the head is one
    fused step, as in the pages' formula);
  * alpha_kv is a scalar applied to the RmsNorm output, gamma included:
    y = alpha_kv * (gamma * c / RMS(c)) with RMS(c) = sqrt(mean(c^2) + eps);
  * the weight is one [576, He] matrix: row j < 512 is column j of W^DKV,
    row 512 + i is column i of W^KR (the rope key input);
  * RoPE is the interleaved one, with per-token cos / sin rows [T, 64];
  * a quantised ckv cache takes the per-row rule of the norm-rope-cache
    operator (RowMax/127 and round for int8, RowMax/448 and the nearest
    E4M3FN value for FLOAT8 E4M3FN) applied to the float64 y.

Every function is pinned in ``tests/test_oracle_mla.py``.
"""
from __future__ import annotations

import numpy as np

DV, DK = 512, 64


class MlaOracleError(RuntimeError):
    pass


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(v) -> np.ndarray:
    """float64 -> bf16 bit patterns, round to nearest, ties to even, in one
    step (no float32 intermediate, which could round twice)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float64)
    fin = np.isfinite(v)
    a = np.abs(v)
    normal = fin & (a >= 2.0 ** -126)
    # normal range: 8 significant bits
    m, e = np.frexp(np.where(normal, v, 1.0))          # v = m * 2^e, 0.5 <= |m| < 1
    out[normal] = np.ldexp(np.rint(m * 256.0), e - 8)[normal]
    # subnormal range: multiples of 2^-133
    sub = fin & ~normal
    out[sub] = np.rint(v[sub] * 2.0 ** 133) * 2.0 ** -133
    out[~fin] = v[~fin]
    # largest finite bf16 is (2 - 2^-7) * 2^127; anything rounding above it is inf
    big = fin & (np.abs(out) >= 2.0 ** 128)
    out[big] = np.copysign(np.inf, v[big])
    with np.errstate(over="ignore"):
        f = out.astype(np.float32)                       # exact: out is a bf16 value
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    bits[np.isnan(v)] = 0x7FC0
    return bits


def kv_project(x, w) -> np.ndarray:
    """c = x @ W^T in float64: x [T, He], w [576, He] bf16 -> [T, 576]."""
    return bf16_to_f64(x) @ bf16_to_f64(w).T


def kv_head_rows(x, w, gamma, alpha, cos, sin, eps):
    """Per-token float64 outputs: y [T, 512] = alpha * RmsNorm(c[:, :512]) and
    kr [T, 64] = RoPE(c[:, 512:]) with the token's cos / sin rows."""
    c = kv_project(x, w)
    if c.shape[1] != DV + DK:
        raise MlaOracleError("the weight must have 576 rows")
    cv, cr = c[:, :DV], c[:, DV:]
    ms = np.sum(cv * cv, axis=1) / DV
    rms = np.sqrt(ms + float(eps))
    g = bf16_to_f64(gamma)
    y = float(alpha) * ((cv / rms[:, None]) * g[None, :])
    x1, x2 = cr[:, 0::2], cr[:, 1::2]
    cs, sn = bf16_to_f64(cos), bf16_to_f64(sin)
    kr = np.concatenate([x1, x2], axis=1) * cs + np.concatenate([-x2, x1], axis=1) * sn
    return y, kr


def check_slots(slot_mapping, rows):
    v = np.asarray(slot_mapping, dtype=np.int64)
    if np.any((v < -1) | (v >= rows)):
        raise MlaOracleError("slot out of range")
    valid = v[v >= 0]
    if np.unique(valid).size != valid.size:
        raise MlaOracleError("duplicate slot")


def mla_kv_head_paged(x, w, gamma, alpha, cos, sin, slot_mapping, k_cache, ckv_cache, eps,
                      ckv_scale=None, kind="bf16"):
    """Writes the ckv row of y and bf16(kr) of every token with slot v >= 0 to
    row v of ckv_cache [NB, BS, 1, 512] and k_cache [NB, BS, 1, 64] (in
    place); -1 skips the token; other rows keep their bytes. kind "bf16":
    bf16(y) (uint16 bits); "int8" / "fp8": the quantize_rows codes (int8, or
    E4M3FN code bytes) and the float32 of the scale into ckv_scale
    [NB, BS, 1]."""
    kc = k_cache.reshape(-1, DK)
    ck = ckv_cache.reshape(-1, DV)
    check_slots(slot_mapping, ck.shape[0])
    v = np.asarray(slot_mapping, dtype=np.int64)
    if v.size == 0:
        return
    y, kr = kv_head_rows(x, w, gamma, alpha, cos, sin, eps)
    keep = v >= 0
    if kind == "bf16":
        ck[v[keep]] = f64_to_bf16(y[keep])
    else:
        q, scale = quantize_rows(y[keep], kind)
        ck[v[keep]] = q.astype(np.int8) if kind == "int8" else e4m3_encode(q)
        ckv_scale.reshape(-1)[v[keep]] = scale.astype(np.float32)
    kc[v[keep]] = f64_to_bf16(kr[keep])


E4M3_MAX = 448.0


def e4m3_round(v):
    """Nearest FLOAT8 E4M3FN value of float64 v (|v| <= 464), ties to the
    even code. The format: sign, 4 exponent bits (bias 7), 3 mantissa bits;
    normal values (1 + m/8) * 2^(E - 7), E = 1..15 (E = 15, m = 7 is NaN, so
    448 is the largest); subnormals (m/8) * 2^-6. In the binade
    [2^e, 2^(e+1)) the values are spaced 2^(e-3); below 2^-6 the spacing is
    2^-9, as in [2^-6, 2^-5)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(np.maximum(a, 2.0 ** -6))        # a = f * 2^ex, f in [0.5, 1)
    step = np.ldexp(1.0, ex - 1 - 3)
    return np.copysign(np.rint(a / step) * step, v)


def e4m3_encode(q):
    """Code bytes of E4M3FN values q (as e4m3_round returns them); the sign
    bit follows the sign of q, also for zeros."""
    q = np.asarray(q, dtype=np.float64)
    a = np.abs(q)
    sign = np.signbit(q).astype(np.uint8) << 7
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = ex - 1                                          # a in [2^e, 2^(e+1))
    normal = a >= 2.0 ** -6
    field = np.where(normal, e + 7, 0)
    mant = np.where(normal, a / np.ldexp(1.0, e - 3) - 8, a / 2.0 ** -9)
    return (sign | (field.astype(np.uint8) << 3) | mant.astype(np.uint8)).astype(np.uint8)


def e4m3_decode(code):
    """Values of E4M3FN code bytes (the format definition above; NaN codes
    0x7F / 0xFF give NaN)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    field, mant = (c >> 3) & 0xF, c & 7
    val = np.where(field > 0, np.ldexp(1.0 + mant / 8.0, field - 7), np.ldexp(mant / 8.0, -6))
    val = np.where((field == 15) & (mant == 7), np.nan, val)
    return sign * val


def quantize_rows(y, kind):
    """Per-row quantisation of the ckv rows y [T, 512] (float64), the rule of
    the norm-rope-cache oracle taken to float64: scale = RowMax(|y|) / 127
    and code = round(y / scale), half to even (int8; the RowMax/127 + round
    rule of aclnnMlaPrologV3WeightNz, Dequant Scale Query Nope formula), or
    scale = RowMax(|y|) / 448 and the nearest E4M3FN value of y / scale
    (FLOAT8 E4M3FN). A zero row has scale 0 and codes 0. Returns (codes as
    float64 values, scale). The zero codes of a zero row are +0 (byte 0x00),
    as in the norm-rope-cache rule; elsewhere a zero keeps its sign."""
    amax = np.max(np.abs(y), axis=1)
    scale = amax / (127.0 if kind == "int8" else E4M3_MAX)
    safe = np.where(scale > 0, scale, 1.0)[:, None]
    qv = y / safe
    q = np.rint(qv) if kind == "int8" else e4m3_round(qv)
    q = np.where(scale[:, None] > 0, q, 0.0)
    return q, scale


def block_index_slots(block_index, B, S, block_size, rows):
    """Per-token cache rows of the block-indexed placement (PA_BLK_BSND:
    aclnnMlaPrologV3WeightNz, cacheIndex of shape (B, Ceil(S/BlockSize));
    aclnnKvRmsNormRopeCache, restrictions on index for PA_BLK_BNSD: each entry
    is -1 or in [0, BlockNum*BlockSize), entry / BlockSize must not repeat).
    READING (as for the norm-rope-cache operator): entry (b, c) covers tokens
    s = c*BS .. c*BS + BS - 1 of batch b and names block entry // BS; token
    (b, s) goes to row (entry // BS) * BS + s % BS; -1 skips the chunk."""
    chunks = -(-S // block_size) if S > 0 else 0
    e = np.asarray(block_index, dtype=np.int64).reshape(-1)
    if e.size != B * chunks:
        raise MlaOracleError("block_index must hold B * ceil(S / block_size) entries")
    if np.any((e < -1) | (e >= rows)):
        raise MlaOracleError("block index entry out of range")
    blocks = e[e >= 0] // block_size
    if np.unique(blocks).size != blocks.size:
        raise MlaOracleError("a block is named twice")
    slots = np.full(B * S, -1, dtype=np.int64)
    for b in range(B):
        for s in range(S):
            v = e[b * chunks + s // block_size]
            if v >= 0:
                slots[b * S + s] = (v // block_size) * block_size + s % block_size
    return slots


def mla_kv_head_paged_blk(x, w, gamma, alpha, cos, sin, block_index, B, S, k_cache, ckv_cache,
                          eps, ckv_scale=None, kind="bf16"):
    """The same head with the block-indexed placement: x, cos, sin hold the
    B * S tokens batch-major; one block_index entry per chunk of
    block_size tokens of a sequence (block_size = k_cache.shape[1])."""
    rows = k_cache.reshape(-1, DK).shape[0]
    slots = block_index_slots(block_index, B, S, k_cache.shape[1], rows)
    mla_kv_head_paged(x, w, gamma, alpha, cos, sin, slots, k_cache, ckv_cache, eps, ckv_scale,
                      kind)


def run_mla_case(case):
    """Runs a gen.mla_kv_head_case (per-token slots) or a
    gen.mla_kv_head_blk_case (block index) on fresh sentinel-filled caches."""
    caches = {k: spec.numpy() for k, spec in case["caches"].items()}
    kind = case.get("ckv_dtype", "bf16")
    scale = caches.get("ckv_scale")
    if case.get("mode") == "mla_paged_blk":
        mla_kv_head_paged_blk(case["x"], case["w"], case["gamma"], case["alpha"], case["cos"],
                              case["sin"], case["block_index"], case["B"], case["S"],
                              caches["k_cache"], caches["ckv_cache"], case["eps"], scale, kind)
    else:
        mla_kv_head_paged(case["x"], case["w"], case["gamma"], case["alpha"], case["cos"],
                          case["sin"], case["slot_mapping"], caches["k_cache"],
                          caches["ckv_cache"], case["eps"], scale, kind)
    return caches
