"""CPU oracle for one paged FP8 decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its
binding) never does.  The arithmetic lives in ``fp8kv_oracle.c`` (plain C,
binary64); this file only marshals numpy arrays into it.

Every function cites the passage it follows in the C source's comments.
Parity pins: see tests/test_oracle_*.py (closed forms, brute force, a library
routine for the e4m3 table, an independently written bit-level encoder).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
_lib = None

_p = ctypes.c_void_p
_i32 = ctypes.c_int32


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.oracle_e4m3_table.restype = None
        L.oracle_e4m3_table.argtypes = [_p]
        L.oracle_e4m3_encode_f32_array.restype = None
        L.oracle_e4m3_encode_f32_array.argtypes = [_p, _p, ctypes.c_long]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_bf16_rne.argtypes = [ctypes.c_double]
        L.oracle_verify.restype = None
        L.oracle_verify.argtypes = [_p, _p, _i32, _p, _i32, _p, _i32, _i32, _p]
        L.oracle_append.restype = ctypes.c_int
        L.oracle_append.argtypes = [_i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p,
                                    _i32, _p, _p, _p, _i32, _i32, _p]
        L.oracle_attention.restype = ctypes.c_int
        L.oracle_attention.argtypes = [_i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _i32,
                                       _p, _i32, _p, _i32, ctypes.c_float, _p, _p, _p, _p, _i32]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_set_num_threads.restype = None
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(int(code) & 0xFF)


def e4m3_encode(v: float) -> int:
    return int(lib().oracle_e4m3_encode(float(v)))


def e4m3_encode_f32(x) -> np.ndarray:
    """Vectorised encode of binary32 inputs."""
    a = _c(x, np.float32)
    out = np.zeros(a.shape, np.uint8)
    lib().oracle_e4m3_encode_f32_array(_ptr(a), _ptr(out), a.size)
    return out


def e4m3_table() -> np.ndarray:
    out = np.zeros(256, np.float64)
    lib().oracle_e4m3_table(_ptr(out))
    return out


def bf16_rne(v: float) -> int:
    return int(lib().oracle_bf16_rne(float(v)))


def verify(page_table, expected_tags, ctx_lens, pool_tags, page_size: int = 16) -> np.ndarray:
    pt = _c(page_table, np.int32)
    et = _c(expected_tags, np.uint32)
    cl = _c(ctx_lens, np.int32)
    tg = _c(pool_tags, np.uint32)
    B = cl.shape[0]
    out = np.zeros(B, np.uint8)
    lib().oracle_verify(_ptr(pt), _ptr(et), pt.shape[1] if pt.ndim == 2 else 0, _ptr(cl), B,
                        _ptr(tg), tg.shape[0], page_size, _ptr(out))
    return out


def new_cache(num_pages: int, Hkv: int, cache_dtype: int = 0, D: int = 128, S: int = 16):
    dt = np.uint8 if cache_dtype == 0 else np.uint16
    return (np.zeros((num_pages, Hkv, S, D), dt), np.zeros((num_pages, Hkv, S, D), dt))


def append(k_cache, v_cache, k_scale, v_scale, k_new, v_new, token_seq, token_pos,
           page_table, abort=None, cache_dtype: int = 0) -> int:
    """Quantize-on-append into logical caches [pages][Hkv][S][D] (in place)."""
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    N, Hkv, S, D = k_cache.shape
    ks = _c(k_scale, np.float32)
    vs = _c(v_scale, np.float32)
    kn = _c(k_new, np.uint16)
    vn = _c(v_new, np.uint16)
    ts = _c(token_seq, np.int32)
    tp = _c(token_pos, np.int32)
    pt = _c(page_table, np.int32)
    ab = None if abort is None else _c(abort, np.uint8)
    return lib().oracle_append(cache_dtype, N, S, Hkv, D, _ptr(k_cache), _ptr(v_cache),
                               _ptr(ks), _ptr(vs), _ptr(kn), _ptr(vn), ts.shape[0],
                               _ptr(ts), _ptr(tp), _ptr(pt), pt.shape[0], pt.shape[1], _ptr(ab))


def attention(k_cache, v_cache, k_scale, v_scale, q, page_table, ctx_lens, sm_scale,
              abort=None, cache_dtype: int = 0, rows=None):
    """Returns (out64 [B][Hq][D] float64, out_bf16 bits [B][Hq][D] uint16)."""
    N, Hkv, S, D = k_cache.shape
    qq = _c(q, np.uint16)
    B, Hq, _ = qq.shape
    pt = _c(page_table, np.int32)
    cl = _c(ctx_lens, np.int32)
    ks = _c(k_scale, np.float32)
    vs = _c(v_scale, np.float32)
    ab = None if abort is None else _c(abort, np.uint8)
    out = np.zeros((B, Hq, D), np.float64)
    ob = np.zeros((B, Hq, D), np.uint16)
    rr = None if rows is None else _c(rows, np.int32)
    st = lib().oracle_attention(cache_dtype, N, S, Hkv, D, _ptr(k_cache), _ptr(v_cache),
                                _ptr(ks), _ptr(vs), _ptr(qq), Hq, _ptr(pt), pt.shape[1],
                                _ptr(cl), B, float(sm_scale), _ptr(ab), _ptr(out), _ptr(ob),
                                _ptr(rr), 0 if rr is None else rr.shape[0])
    if st != 0:
        raise ValueError("oracle_attention: a request names an invalid page")
    return out, ob


def attention_multi(k_cache, v_cache, k_scale, v_scale, q, page_table, ctx_lens, sm_scale,
                    abort=None, cache_dtype: int = 0):
    """Several new tokens per request verified in one step (speculative decoding:
    a draft proposes tokens, the main model checks them together -- page "Kimi
    and GLM Reasoning Slimming: Hands-On Test", section "It Follows the Same
    Path as Cloudflare's Earlier Infire Optimizations").  q is [B][T][Hq][D];
    ctx_lens counts the tokens after all T new ones were appended.  Query i
    stands for the new token at position ctx-T+i and sees the tokens up to and
    including it: it is single-query attention over the first ctx-(T-1-i)
    tokens (a query with no token to see gives +0, as an empty context does).
    Returns (out64 [B][T][Hq][D] float64, out_bf16 bits [B][T][Hq][D])."""
    qq = _c(q, np.uint16)
    B, T, Hq, D = qq.shape
    cl = _c(ctx_lens, np.int32)
    out = np.zeros((B, T, Hq, D), np.float64)
    ob = np.zeros((B, T, Hq, D), np.uint16)
    for i in range(T):
        ci = np.maximum(cl - (T - 1 - i), 0).astype(np.int32)
        out[:, i], ob[:, i] = attention(k_cache, v_cache, k_scale, v_scale,
                                        np.ascontiguousarray(qq[:, i]), page_table, ci, sm_scale,
                                        abort=abort, cache_dtype=cache_dtype)
    return out, ob


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the attention rows (timing only; results do not depend on it)."""
    lib().oracle_set_num_threads(int(n))
