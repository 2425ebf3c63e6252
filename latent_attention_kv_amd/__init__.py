"""Python binding of libkvrc.so: MI355X (gfx950) latent-attention KV preprocessing.

Argument marshalling only. Every step of the computation runs in the HIP
kernels of ``libkvrc.so``; PyTorch supplies device memory and the stream.
There is no CPU or PyTorch fallback: if the library is missing, or a tensor
is not on the GPU, the call raises.

Entry points (same names as the C ABI in ``include/kvrc.h``):
  * kvrc_paged_norm_rope_cache - RMSNorm + interleaved RoPE + scatter into
    paged caches [num_blocks, block_size, 1, d] (aclnnKvRmsNormRopeCache,
    PA_BNSD cache mode); the ckv cache holds bf16 rows, or int8 / FLOAT8
    E4M3FN codes with a float32 scale per row
  * kvrc_paged_blk_norm_rope_cache - the same with one index entry per block
    of tokens (PA_BLK_BNSD cache mode)
  * kvrc_norm_rope_cache       - the same into contiguous caches
    [Bc, 1, Sc, d] (Norm cache mode)
  * kvrc_mla_kv_head_paged     - the MLA kv-path head: x [T, He] times the
    fused [576, He] projection on the matrix cores, then alpha_kv * RMSNorm,
    RoPE and the paged scatter (aclnnMlaPrologV3WeightNz, third and fourth
    paths); it takes a caller-owned workspace of
    kvrc_mla_kv_head_workspace_bytes(T) bytes
  * qsa_prepare                - block keys (openvino.opset17.qsa_prepare)
  * qsa_select_topk            - block selection over those keys: softmax
    scores, selection pooling, head sum, top-k (aclnnNsaCompressAttentionInfer)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["kvrc_paged_norm_rope_cache", "kvrc_paged_blk_norm_rope_cache",
           "kvrc_norm_rope_cache", "kvrc_mla_kv_head_workspace_bytes", "kvrc_mla_kv_head_paged",
           "kvrc_mla_kv_head_paged_blk",
           "qsa_prepare", "qsa_select_topk", "kvrc_selftest_arith", "kvrc_selftest_recip",
           "kvrc_selftest_e4m3", "kvrc_selftest_empty", "kvrc_selftest_copy",
           "kvrc_selftest_mla_kv_head_stalled", "kvrc_mla_kv_head_paged_noalloc",
           "MLA_NOALLOC_MAX_TOKENS",
           "select_blocks_capacity", "KvrcError", "lib", "LIB_PATH", "CACHE_BF16", "CACHE_INT8", "CACHE_FP8_E4M3",
           "EXPORTED_SYMBOLS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvrc.so")
CACHE_BF16 = 0
CACHE_INT8 = 1
CACHE_FP8_E4M3 = 2
# largest T of kvrc_mla_kv_head_paged_noalloc (its static workspace)
MLA_NOALLOC_MAX_TOKENS = 1 << 17
EXPORTED_SYMBOLS = ("kvrc_status_string", "kvrc_version", "kvrc_paged_norm_rope_cache",
                    "kvrc_paged_blk_norm_rope_cache", "kvrc_norm_rope_cache",
                    "kvrc_mla_kv_head_workspace_bytes", "kvrc_mla_kv_head_paged",
                    "kvrc_mla_kv_head_paged_blk", "qsa_prepare", "qsa_select_topk",
                    "kvrc_selftest_arith", "kvrc_selftest_recip", "kvrc_selftest_e4m3",
                    "kvrc_selftest_empty", "kvrc_selftest_copy",
                    "kvrc_selftest_mla_kv_head_stalled", "kvrc_mla_kv_head_paged_noalloc")

_lib = None


class KvrcError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({_status_string(status)})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libkvrc.so (built by ``__graft_entry__.build()``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    L.kvrc_status_string.argtypes = [I32]
    L.kvrc_status_string.restype = ctypes.c_char_p
    L.kvrc_version.restype = I32
    L.kvrc_paged_norm_rope_cache.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I64,
                                             I32, F, P, P]
    L.kvrc_paged_norm_rope_cache.restype = I32
    L.kvrc_paged_blk_norm_rope_cache.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I64,
                                                 I64, I64, I32, F, P, P]
    L.kvrc_paged_blk_norm_rope_cache.restype = I32
    L.kvrc_norm_rope_cache.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, I32,
                                       F, P, P]
    L.kvrc_norm_rope_cache.restype = I32
    L.kvrc_mla_kv_head_workspace_bytes.argtypes = [I64]
    L.kvrc_mla_kv_head_workspace_bytes.restype = I64
    L.kvrc_mla_kv_head_paged.argtypes = [P, P, P, F, P, P, P, P, P, P, I64, I64, I64, I64, I32,
                                         F, P, I64, P, P]
    L.kvrc_mla_kv_head_paged.restype = I32
    L.kvrc_mla_kv_head_paged_blk.argtypes = [P, P, P, F, P, P, P, P, P, P, I64, I64, I64, I64,
                                             I64, I32, F, P, I64, P, P]
    L.kvrc_mla_kv_head_paged_blk.restype = I32
    L.qsa_select_topk.argtypes = [P, P, P, I64, F, I64, I64, I64, I64, I64, I64, I64, I64, P, P,
                                  P, P]
    L.qsa_select_topk.restype = I32
    L.qsa_prepare.argtypes = [P, P, P, I64, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, F,
                              P, P]
    L.qsa_prepare.restype = I32
    L.kvrc_selftest_arith.argtypes = [P, P, P, P, P, I64, P]
    L.kvrc_selftest_arith.restype = I32
    L.kvrc_selftest_recip.argtypes = [P, P, I64, P]
    L.kvrc_selftest_recip.restype = I32
    L.kvrc_selftest_e4m3.argtypes = [P, P, I64, P]
    L.kvrc_selftest_e4m3.restype = I32
    L.kvrc_selftest_empty.argtypes = [I64, I32, P]
    L.kvrc_selftest_empty.restype = I32
    L.kvrc_selftest_copy.argtypes = [P, P, I64, P]
    L.kvrc_selftest_copy.restype = I32
    L.kvrc_selftest_mla_kv_head_stalled.argtypes = [P, P, P, F, P, P, P, P, P, P, I64, I64, I64,
                                                    I64, I32, F, P, I64, P, I64, P, P]
    L.kvrc_selftest_mla_kv_head_stalled.restype = I32
    L.kvrc_mla_kv_head_paged_noalloc.argtypes = [P, P, P, F, P, P, P, P, P, P, I64, I64, I64,
                                                 I64, I32, F, P, P]
    L.kvrc_mla_kv_head_paged_noalloc.restype = I32
    _lib = L
    return L


def _status_string(status: int) -> str:
    try:
        return lib().kvrc_status_string(status).decode()
    except Exception:  # pragma: no cover - only when the library is missing
        return "?"


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _need(t, name, dtypes, ndim=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


_BF16 = (torch.bfloat16,)


def _kv_shapes(kv, gamma, cos, sin):
    _need(kv, "kv", _BF16, 4)
    _need(cos, "cos", _BF16, 4)
    _need(sin, "sin", _BF16, 4)
    _need(gamma, "gamma", _BF16, 1)
    B, n, S, D = kv.shape
    Dk = cos.shape[-1]
    Dv = D - Dk
    if n != 1 or tuple(cos.shape) != (B, 1, S, Dk) or tuple(sin.shape) != (B, 1, S, Dk):
        raise ValueError("kv must be [B,1,S,Dv+Dk] and cos/sin [B,1,S,Dk]")
    if tuple(gamma.shape) != (Dv,):
        raise ValueError("gamma must be [Dv]")
    return B, S, Dv, Dk


# ckv cache element types: bf16 rows, int8 codes, or FLOAT8 E4M3FN codes
# (torch.float8_e4m3fn, or their raw bytes as torch.uint8).
_CKV = (torch.bfloat16, torch.int8, torch.float8_e4m3fn, torch.uint8)


def _cache_dtype(ckv_cache, ckv_scale):
    if ckv_cache.dtype == torch.bfloat16:
        if ckv_scale is not None:
            raise ValueError("ckv_scale is only used with a quantised (int8 / fp8) ckv cache")
        return CACHE_BF16
    _need(ckv_scale, "ckv_scale", (torch.float32,))
    return CACHE_INT8 if ckv_cache.dtype == torch.int8 else CACHE_FP8_E4M3


def _err_ptr(err_count):
    if err_count is None:
        return None
    _need(err_count, "err_count", (torch.int32,))
    return err_count.data_ptr()


def _check(status, what):
    if status != 0:
        raise KvrcError(status, what)


def _paged_args(kv, gamma, cos, sin, slot_mapping, k_cache, ckv_cache, ckv_scale, eps,
                err_count, stream):
    """Checked C-ABI argument tuple of kvrc_paged_norm_rope_cache."""
    B, S, Dv, Dk = _kv_shapes(kv, gamma, cos, sin)
    _need(slot_mapping, "slot_mapping", (torch.int64,), 1)
    _need(k_cache, "k_cache", _BF16, 4)
    _need(ckv_cache, "ckv_cache", _CKV, 4)
    NB, BS = k_cache.shape[0], k_cache.shape[1]
    if slot_mapping.numel() != B * S:
        raise ValueError("slot_mapping must have B*S entries")
    if tuple(k_cache.shape) != (NB, BS, 1, Dk) or tuple(ckv_cache.shape) != (NB, BS, 1, Dv):
        raise ValueError("caches must be [num_blocks, block_size, 1, Dk] and [.., Dv]")
    dt = _cache_dtype(ckv_cache, ckv_scale)
    if ckv_scale is not None and tuple(ckv_scale.shape) != (NB, BS, 1):
        raise ValueError("ckv_scale must be [num_blocks, block_size, 1]")
    return (_ptr(kv), _ptr(gamma), _ptr(cos), _ptr(sin), _ptr(slot_mapping), _ptr(k_cache),
            _ptr(ckv_cache), _ptr(ckv_scale), B, S, Dv, Dk, NB, BS, dt, float(eps),
            _err_ptr(err_count), _stream(stream))


def kvrc_paged_norm_rope_cache(kv, gamma, cos, sin, slot_mapping, k_cache, ckv_cache,
                               ckv_scale=None, *, eps=1e-6, err_count=None, stream=None):
    """Paged (PA_BNSD) fused norm-rope-cache; updates the caches in place."""
    args = _paged_args(kv, gamma, cos, sin, slot_mapping, k_cache, ckv_cache, ckv_scale, eps,
                       err_count, stream)
    _check(lib().kvrc_paged_norm_rope_cache(*args), "kvrc_paged_norm_rope_cache")


def kvrc_paged_blk_norm_rope_cache(kv, gamma, cos, sin, block_index, k_cache, ckv_cache,
                                   ckv_scale=None, *, eps=1e-6, err_count=None, stream=None):
    """Block-indexed paged mode (PA_BLK_BNSD): block_index [B * ceil(S / block_size)]."""
    B, S, Dv, Dk = _kv_shapes(kv, gamma, cos, sin)
    _need(block_index, "block_index", (torch.int64,), 1)
    _need(k_cache, "k_cache", _BF16, 4)
    _need(ckv_cache, "ckv_cache", _CKV, 4)
    NB, BS = k_cache.shape[0], k_cache.shape[1]
    if BS < 1 or block_index.numel() != B * (-(-S // BS)):
        raise ValueError("block_index must have B * ceil(S / block_size) entries")
    if tuple(k_cache.shape) != (NB, BS, 1, Dk) or tuple(ckv_cache.shape) != (NB, BS, 1, Dv):
        raise ValueError("caches must be [num_blocks, block_size, 1, Dk] and [.., Dv]")
    dt = _cache_dtype(ckv_cache, ckv_scale)
    if ckv_scale is not None and tuple(ckv_scale.shape) != (NB, BS, 1):
        raise ValueError("ckv_scale must be [num_blocks, block_size, 1]")
    st = lib().kvrc_paged_blk_norm_rope_cache(
        _ptr(kv), _ptr(gamma), _ptr(cos), _ptr(sin), _ptr(block_index), _ptr(k_cache),
        _ptr(ckv_cache), _ptr(ckv_scale), B, S, Dv, Dk, NB, BS, dt, float(eps),
        _err_ptr(err_count), _stream(stream))
    _check(st, "kvrc_paged_blk_norm_rope_cache")


def kvrc_norm_rope_cache(kv, gamma, cos, sin, index, k_cache, ckv_cache, ckv_scale=None, *,
                         eps=1e-6, err_count=None, stream=None):
    """Norm (contiguous) cache mode; index [B, S]; caches [Bc, 1, Sc, d]."""
    B, S, Dv, Dk = _kv_shapes(kv, gamma, cos, sin)
    _need(index, "index", (torch.int64,), 2)
    _need(k_cache, "k_cache", _BF16, 4)
    _need(ckv_cache, "ckv_cache", _CKV, 4)
    Bc, Sc = k_cache.shape[0], k_cache.shape[2]
    if tuple(index.shape) != (B, S):
        raise ValueError("index must be [B, S]")
    if tuple(k_cache.shape) != (Bc, 1, Sc, Dk) or tuple(ckv_cache.shape) != (Bc, 1, Sc, Dv):
        raise ValueError("caches must be [Bc, 1, Sc, Dk] and [Bc, 1, Sc, Dv]")
    dt = _cache_dtype(ckv_cache, ckv_scale)
    if ckv_scale is not None and tuple(ckv_scale.shape) != (Bc, 1, Sc):
        raise ValueError("ckv_scale must be [Bc, 1, Sc]")
    st = lib().kvrc_norm_rope_cache(_ptr(kv), _ptr(gamma), _ptr(cos), _ptr(sin), _ptr(index),
                                    _ptr(k_cache), _ptr(ckv_cache), _ptr(ckv_scale), B, S, Dv, Dk,
                                    Bc, Sc, dt, float(eps), _err_ptr(err_count), _stream(stream))
    _check(st, "kvrc_norm_rope_cache")


def kvrc_mla_kv_head_workspace_bytes(T):
    """Bytes of device workspace kvrc_mla_kv_head_paged needs for T tokens."""
    n = lib().kvrc_mla_kv_head_workspace_bytes(int(T))
    if n < 0:
        raise ValueError("T out of range")
    return n


def _mla_caches(k_cache, ckv_cache, ckv_scale):
    """Checked (NB, BS, ckv dtype) of the MLA head's caches."""
    _need(k_cache, "k_cache", _BF16, 4)
    _need(ckv_cache, "ckv_cache", _CKV, 4)
    NB, BS = k_cache.shape[0], k_cache.shape[1]
    if tuple(k_cache.shape) != (NB, BS, 1, 64) or tuple(ckv_cache.shape) != (NB, BS, 1, 512):
        raise ValueError("caches must be [num_blocks, block_size, 1, 64] and [.., 512]")
    dt = _cache_dtype(ckv_cache, ckv_scale)
    if ckv_scale is not None and tuple(ckv_scale.shape) != (NB, BS, 1):
        raise ValueError("ckv_scale must be [num_blocks, block_size, 1]")
    return NB, BS, dt


def kvrc_mla_kv_head_paged(x, w_dkv_kr, gamma, cos, sin, slot_mapping, k_cache, ckv_cache,
                           ckv_scale=None, *, workspace, alpha_kv=1.0, eps=1e-6, err_count=None,
                           stream=None, _stall_us=None, _steals=None):
    """MLA kv-path head into paged caches: x [T, He], w_dkv_kr [576, He],
    gamma [512], cos / sin [T, 64], slot_mapping [T]; k_cache
    [NB, BS, 1, 64] (bf16) and ckv_cache [NB, BS, 1, 512] (bf16, or int8 /
    E4M3FN codes with ckv_scale [NB, BS, 1] float32) are updated in place.
    workspace: a contiguous device tensor of at least
    kvrc_mla_kv_head_workspace_bytes(T) bytes, all zero before its first use
    (each call leaves it zero); calls that may overlap need separate ones.
    _stall_us / _steals (tests only): call kvrc_selftest_mla_kv_head_stalled,
    which holds back the second workgroup of every pair (include/kvrc_selftest.h)."""
    _need(x, "x", _BF16, 2)
    _need(w_dkv_kr, "w_dkv_kr", _BF16, 2)
    _need(gamma, "gamma", _BF16, 1)
    _need(cos, "cos", _BF16, 2)
    _need(sin, "sin", _BF16, 2)
    _need(slot_mapping, "slot_mapping", (torch.int64,), 1)
    NB, BS, dt = _mla_caches(k_cache, ckv_cache, ckv_scale)
    T, He = x.shape
    if tuple(w_dkv_kr.shape) != (576, He):
        raise ValueError("w_dkv_kr must be [576, He]")
    if tuple(gamma.shape) != (512,):
        raise ValueError("gamma must be [512]")
    if tuple(cos.shape) != (T, 64) or tuple(sin.shape) != (T, 64):
        raise ValueError("cos / sin must be [T, 64]")
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must have T entries")
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or \
            not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    if _stall_us is not None:
        if _steals is not None:
            _need(_steals, "_steals", (torch.int32,), 1)
        st = lib().kvrc_selftest_mla_kv_head_stalled(
            _ptr(x), _ptr(w_dkv_kr), _ptr(gamma), float(alpha_kv), _ptr(cos), _ptr(sin),
            _ptr(slot_mapping), _ptr(k_cache), _ptr(ckv_cache), _ptr(ckv_scale), T, He, NB, BS,
            dt, float(eps), _ptr(workspace), ws_bytes, _err_ptr(err_count), int(_stall_us),
            _ptr(_steals), _stream(stream))
        _check(st, "kvrc_selftest_mla_kv_head_stalled")
        return
    st = lib().kvrc_mla_kv_head_paged(_ptr(x), _ptr(w_dkv_kr), _ptr(gamma), float(alpha_kv),
                                      _ptr(cos), _ptr(sin), _ptr(slot_mapping), _ptr(k_cache),
                                      _ptr(ckv_cache), _ptr(ckv_scale), T, He, NB, BS, dt,
                                      float(eps),
                                      _ptr(workspace), ws_bytes, _err_ptr(err_count),
                                      _stream(stream))
    _check(st, "kvrc_mla_kv_head_paged")


def kvrc_mla_kv_head_paged_noalloc(x, w_dkv_kr, gamma, cos, sin, slot_mapping, k_cache,
                                   ckv_cache, ckv_scale=None, *, alpha_kv=1.0, eps=1e-6,
                                   err_count=None, stream=None):
    """kvrc_mla_kv_head_paged without a workspace argument: the library's
    static device workspace serves (T <= MLA_NOALLOC_MAX_TOKENS); the call
    allocates nothing. Calls that overlap on one device race."""
    _need(x, "x", _BF16, 2)
    _need(w_dkv_kr, "w_dkv_kr", _BF16, 2)
    _need(gamma, "gamma", _BF16, 1)
    _need(cos, "cos", _BF16, 2)
    _need(sin, "sin", _BF16, 2)
    _need(slot_mapping, "slot_mapping", (torch.int64,), 1)
    NB, BS, dt = _mla_caches(k_cache, ckv_cache, ckv_scale)
    T, He = x.shape
    if tuple(w_dkv_kr.shape) != (576, He):
        raise ValueError("w_dkv_kr must be [576, He]")
    if tuple(gamma.shape) != (512,):
        raise ValueError("gamma must be [512]")
    if tuple(cos.shape) != (T, 64) or tuple(sin.shape) != (T, 64):
        raise ValueError("cos / sin must be [T, 64]")
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must have T entries")
    st = lib().kvrc_mla_kv_head_paged_noalloc(_ptr(x), _ptr(w_dkv_kr), _ptr(gamma),
                                              float(alpha_kv), _ptr(cos), _ptr(sin),
                                              _ptr(slot_mapping), _ptr(k_cache), _ptr(ckv_cache),
                                              _ptr(ckv_scale), T, He, NB, BS, dt, float(eps),
                                              _err_ptr(err_count), _stream(stream))
    _check(st, "kvrc_mla_kv_head_paged_noalloc")


def kvrc_mla_kv_head_paged_blk(x, w_dkv_kr, gamma, cos, sin, block_index, k_cache, ckv_cache,
                               ckv_scale=None, *, workspace, alpha_kv=1.0, eps=1e-6,
                               err_count=None, stream=None):
    """MLA kv-path head with the block-indexed placement: x [B, S, He],
    cos / sin [B, S, 64], block_index [B, ceil(S / block_size)] (or flat);
    caches and workspace as for kvrc_mla_kv_head_paged (workspace of
    kvrc_mla_kv_head_workspace_bytes(B * S) bytes)."""
    _need(x, "x", _BF16, 3)
    _need(w_dkv_kr, "w_dkv_kr", _BF16, 2)
    _need(gamma, "gamma", _BF16, 1)
    _need(cos, "cos", _BF16, 3)
    _need(sin, "sin", _BF16, 3)
    _need(block_index, "block_index", (torch.int64,), None)
    NB, BS, dt = _mla_caches(k_cache, ckv_cache, ckv_scale)
    B, S, He = x.shape
    if tuple(w_dkv_kr.shape) != (576, He):
        raise ValueError("w_dkv_kr must be [576, He]")
    if tuple(gamma.shape) != (512,):
        raise ValueError("gamma must be [512]")
    if tuple(cos.shape) != (B, S, 64) or tuple(sin.shape) != (B, S, 64):
        raise ValueError("cos / sin must be [B, S, 64]")
    if block_index.numel() != B * (-(-S // BS) if S else 0):
        raise ValueError("block_index must hold B * ceil(S / block_size) entries")
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or \
            not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().kvrc_mla_kv_head_paged_blk(_ptr(x), _ptr(w_dkv_kr), _ptr(gamma), float(alpha_kv),
                                          _ptr(cos), _ptr(sin), _ptr(block_index), _ptr(k_cache),
                                          _ptr(ckv_cache), _ptr(ckv_scale), B, S, He, NB, BS, dt,
                                          float(eps),
                                          _ptr(workspace), ws_bytes, _err_ptr(err_count),
                                          _stream(stream))
    _check(st, "kvrc_mla_kv_head_paged_blk")


def kvrc_selftest_arith(a, b, q_shared, q_ieee, root, *, stream=None):
    """Device arithmetic self-test (include/kvrc_selftest.h); float32 tensors."""
    for name, t in (("a", a), ("b", b), ("q_shared", q_shared), ("q_ieee", q_ieee),
                    ("root", root)):
        _need(t, name, (torch.float32,), 1)
        if t.numel() != a.numel():
            raise ValueError("all self-test arrays must have the same length")
    st = lib().kvrc_selftest_arith(_ptr(a), _ptr(b), _ptr(q_shared), _ptr(q_ieee), _ptr(root),
                                   a.numel(), _stream(stream))
    _check(st, "kvrc_selftest_arith")


def kvrc_selftest_recip(b, recip, *, stream=None):
    """Reciprocal self-test (include/kvrc_selftest.h): float32 b -> the
    kernels' reciprocal of each element."""
    _need(b, "b", (torch.float32,), 1)
    _need(recip, "recip", (torch.float32,), 1)
    if recip.numel() != b.numel():
        raise ValueError("b and recip must have the same length")
    _check(lib().kvrc_selftest_recip(_ptr(b), _ptr(recip), b.numel(), _stream(stream)),
           "kvrc_selftest_recip")


def kvrc_selftest_e4m3(x, code, *, stream=None):
    """E4M3FN conversion self-test (include/kvrc_selftest.h): float32 x -> uint8 codes."""
    _need(x, "x", (torch.float32,), 1)
    _need(code, "code", (torch.uint8,), 1)
    if code.numel() != x.numel():
        raise ValueError("x and code must have the same length")
    _check(lib().kvrc_selftest_e4m3(_ptr(x), _ptr(code), x.numel(), _stream(stream)),
           "kvrc_selftest_e4m3")


def kvrc_selftest_empty(workgroups, threads=256, *, stream=None):
    """Measurement probe: an empty kernel of `workgroups` x `threads`."""
    _check(lib().kvrc_selftest_empty(int(workgroups), int(threads), _stream(stream)),
           "kvrc_selftest_empty")


def kvrc_selftest_copy(src, dst, *, stream=None):
    """Measurement probe: a plain 16-byte-vector device copy of src into dst
    (contiguous GPU tensors of the same byte size, a multiple of 16)."""
    for name, t in (("src", src), ("dst", dst)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same byte size")
    _check(lib().kvrc_selftest_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)),
           "kvrc_selftest_copy")


def qsa_prepare(raw_index_keys, block_keys, key_length, rope_cos, rope_sin, k_norm_weight,
                past_incomplete_raw_keys, past_incomplete_rope, next_incomplete_raw_keys,
                next_incomplete_rope, *, key_block_size, eps=1e-6, err_count=None, stream=None):
    """QSAPrepare block keys; writes block_keys rows of the completed blocks and
    the next carry state. rope_cos/rope_sin/past/next rope None disables the
    rotation; k_norm_weight None disables the normalisation."""
    _need(raw_index_keys, "raw_index_keys", _BF16, 3)
    N, L, Di = raw_index_keys.shape
    _need(block_keys, "block_keys", _BF16, 3)
    _need(key_length, "key_length", (torch.int64,), 1)
    _need(past_incomplete_raw_keys, "past_incomplete_raw_keys", _BF16, 3)
    _need(next_incomplete_raw_keys, "next_incomplete_raw_keys", _BF16, 3)
    kbs = int(key_block_size)
    Bcap = block_keys.shape[1]
    if tuple(block_keys.shape) != (N, Bcap, Di):
        raise ValueError("block_keys must be [N, Bcap, Di]")
    for name, t in (("past_incomplete_raw_keys", past_incomplete_raw_keys),
                    ("next_incomplete_raw_keys", next_incomplete_raw_keys)):
        if tuple(t.shape) != (N, kbs - 1, Di):
            raise ValueError(f"{name} must be [N, key_block_size-1, Di]")
    Dr = 0
    if rope_cos is not None:
        _need(rope_cos, "rope_cos", (torch.float32,), 3)
        _need(rope_sin, "rope_sin", (torch.float32,), 3)
        Dr = rope_cos.shape[-1]
        if tuple(rope_cos.shape) != (N, L, Dr) or tuple(rope_sin.shape) != (N, L, Dr):
            raise ValueError("rope_cos/rope_sin must be [N, L, Dr]")
        for name, t in (("past_incomplete_rope", past_incomplete_rope),
                        ("next_incomplete_rope", next_incomplete_rope)):
            _need(t, name, (torch.float32,), 2)
            if tuple(t.shape) != (N, 2 * Dr):
                raise ValueError(f"{name} must be [N, 2*Dr]")
    if k_norm_weight is not None:
        _need(k_norm_weight, "k_norm_weight", _BF16, 1)
    st = lib().qsa_prepare(_ptr(raw_index_keys), _ptr(block_keys), _ptr(key_length),
                           key_length.numel(), _ptr(rope_cos), _ptr(rope_sin), _ptr(k_norm_weight),
                           _ptr(past_incomplete_raw_keys), _ptr(past_incomplete_rope),
                           _ptr(next_incomplete_raw_keys), _ptr(next_incomplete_rope), N, L, Di,
                           Dr, Bcap, kbs, float(eps), _err_ptr(err_count), _stream(stream))
    _check(st, "qsa_prepare")


def select_blocks_capacity(Bcap: int, sel_ratio: int, cmp_ratio: int) -> int:
    """Jcap: selection-score columns for a block-key capacity Bcap."""
    return (Bcap + sel_ratio + cmp_ratio - 3) // sel_ratio + 1 if Bcap > 0 else 0


def qsa_select_topk(query, block_keys, key_length, scores, indices, *, key_block_size,
                    sel_ratio=1, cmp_ratio=1, scale=None, err_count=None, stream=None):
    """Block selection: query [N, H, Di] and block_keys [N, Bcap, Di] (bf16),
    key_length [N] or [1]; writes scores [N, Jcap] (float32) and indices
    [N, topk] (int32). scale defaults to 1 / sqrt(Di)."""
    _need(query, "query", _BF16, 3)
    _need(block_keys, "block_keys", _BF16, 3)
    _need(key_length, "key_length", (torch.int64,), 1)
    _need(scores, "scores", (torch.float32,), 2)
    _need(indices, "indices", (torch.int32,), 2)
    N, H, Di = query.shape
    Bcap = block_keys.shape[1]
    if tuple(block_keys.shape) != (N, Bcap, Di):
        raise ValueError("block_keys must be [N, Bcap, Di]")
    jcap = select_blocks_capacity(Bcap, int(sel_ratio), int(cmp_ratio))
    if tuple(scores.shape) != (N, jcap):
        raise ValueError(f"scores must be [N, {jcap}]")
    if indices.shape[0] != N:
        raise ValueError("indices must be [N, topk]")
    if scale is None:
        scale = 1.0 / float(Di) ** 0.5
    st = lib().qsa_select_topk(_ptr(query), _ptr(block_keys), _ptr(key_length),
                               key_length.numel(), float(scale), N, H, Di, Bcap,
                               int(key_block_size), int(sel_ratio), int(cmp_ratio),
                               indices.shape[1], _ptr(scores), _ptr(indices),
                               _err_ptr(err_count), _stream(stream))
    _check(st, "qsa_select_topk")
