"""Python binding for libfp8kv (FP8 paged decode attention with page tags).

Argument marshalling only: every step of the decode path runs in the HIP
library (``libfp8kv.so``, built in-tree by ``build.py``).  PyTorch supplies
device memory and the current stream; nothing here computes.  If the library
is missing the import fails -- there is no fallback.

Names mirror the C ABI in ``include/fp8kv.h``:
  Pool, verify_tags, append, verify_append, verify_append_q, decode_attention,
  decode_attention_noalloc, decode_attention_q, decode_attention_shared, decode_workspace_size,
  decode_workspace_size_q, decode_workspace_size_shared,
  decode_num_workers, cache_offset, cache_bytes, debug_convert_e4m3;
  step() chains the step's calls in the order the pages give.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8kv.so")

E4M3, BF16 = 0, 1
OUT_BF16, OUT_F32 = 0, 1
PAGE_SIZE = 16
HEAD_DIM = 128

_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported shape or dtype",
           -3: "out of pages", -4: "workspace too small", -5: "HIP error"}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python decode_attention_paged_fp8kv_amd/build.py` "
        "(or __graft_entry__.build()); there is no non-HIP fallback")

_lib = ctypes.CDLL(LIB_PATH)
_p = ctypes.c_void_p
_i32 = ctypes.c_int32


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("cache_dtype", ctypes.c_int32)]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_status_string = _sig("fp8kv_status_string", ctypes.c_char_p, [_i32])
_last_hip_error = _sig("fp8kv_last_hip_error", _i32, [])
_cache_bytes = _sig("fp8kv_cache_bytes", ctypes.c_size_t, [ctypes.POINTER(CacheDesc)])
_cache_offset = _sig("fp8kv_cache_offset", ctypes.c_int64,
                     [ctypes.POINTER(CacheDesc), _i32, _i32, _i32, _i32, _i32])
_pool_create = _sig("fp8kv_pool_create", _i32, [_i32, ctypes.c_uint64, ctypes.POINTER(_p)])
_pool_destroy = _sig("fp8kv_pool_destroy", None, [_p])
_pool_alloc = _sig("fp8kv_pool_alloc", _i32, [_p, _i32, _p, _p])
_pool_free = _sig("fp8kv_pool_free", _i32, [_p, _i32, _p])
_pool_share = _sig("fp8kv_pool_share", _i32, [_p, _i32, _p])
_pool_refcount = _sig("fp8kv_pool_refcount", _i32, [_p, _i32])
_pool_tag = _sig("fp8kv_pool_tag", ctypes.c_uint32, [_p, _i32])
_pool_num_free = _sig("fp8kv_pool_num_free", _i32, [_p])
_pool_read_tags = _sig("fp8kv_pool_read_tags", _i32, [_p, _p])
_pool_sync = _sig("fp8kv_pool_sync", _i32, [_p, _p, _p])
_verify = _sig("fp8kv_verify_tags", _i32, [_p, _p, _i32, _p, _i32, _p, _i32, _i32, _p, _p])
_append = _sig("fp8kv_append", _i32, [ctypes.POINTER(CacheDesc), _p, _p, _p, _p, _p, _p, _i32,
                                      _p, _p, _i32, _p, _i32, _p, _p])
_num_workers = _sig("fp8kv_decode_num_workers", _i32, [_i32])
_ws_size = _sig("fp8kv_decode_workspace_size", ctypes.c_size_t,
                [ctypes.POINTER(CacheDesc), _i32, _i32, _i32])
_decode = _sig("fp8kv_decode_attention", _i32,
               [ctypes.POINTER(CacheDesc), _p, _p, _p, _p, _p, _i32, _p, _i32, _p, _i32,
                ctypes.c_float, _p, _p, _i32, _i32, _p, ctypes.c_size_t, _p])
_decode_noalloc = _sig("fp8kv_decode_attention_noalloc", _i32,
                       [ctypes.POINTER(CacheDesc), _p, _p, _p, _p, _p, _i32, _p, _i32, _p, _i32,
                        ctypes.c_float, _p, _p, _i32, _i32, _p])
NOALLOC_SCRATCH_BYTES = 32 << 20   # FP8KV_NOALLOC_SCRATCH_BYTES
_ws_size_q = _sig("fp8kv_decode_workspace_size_q", ctypes.c_size_t,
                  [ctypes.POINTER(CacheDesc), _i32, _i32, _i32, _i32])
_decode_q = _sig("fp8kv_decode_attention_q", _i32,
                 [ctypes.POINTER(CacheDesc), _p, _p, _p, _p, _p, _i32, _i32, _p, _i32, _p, _i32,
                  ctypes.c_float, _p, _p, _i32, _i32, _p, ctypes.c_size_t, _p])
_ws_size_shared = _sig("fp8kv_decode_workspace_size_shared", ctypes.c_size_t,
                       [ctypes.POINTER(CacheDesc), _i32, _i32, _i32, _i32, _p, _p, _i32])
_decode_shared = _sig("fp8kv_decode_attention_shared", _i32,
                      [ctypes.POINTER(CacheDesc), _p, _p, _p, _p, _p, _i32, _i32, _p, _p, _p,
                       _i32, _p, _i32, ctypes.c_float, _p, _p, _i32, _i32, _p, ctypes.c_size_t,
                       _p])
_verify_append = _sig("fp8kv_verify_append", _i32,
                      [ctypes.POINTER(CacheDesc), _p, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _p,
                       _i32, _p, _p, _p])
_verify_append_q = _sig("fp8kv_verify_append_q", _i32,
                        [ctypes.POINTER(CacheDesc), _p, _p, _p, _p, _p, _p, _p, _i32, _p, _p,
                         _i32, _p, _i32, _p, _p, _p])
_debug_convert = _sig("fp8kv_debug_convert_e4m3", _i32, [_p, _p, _i32, _i32, _p])
_read_sink_words = _sig("fp8kv_debug_read_sink_words", _i32, [])
_read_bandwidth = _sig("fp8kv_debug_read_bandwidth", _i32, [_p, ctypes.c_size_t, _p, _p])


class Fp8kvError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = f"{where}: {_status_string(status).decode()} ({status})"
        if status == -5:
            msg += f", hipError {_last_hip_error()}"
        super().__init__(msg)
        self.status = status


def _check(status: int, where: str):
    if status != 0:
        raise Fp8kvError(status, where)


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: Optional[torch.Tensor], dtypes, name: str, allow_none: bool = False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _shape(t, shape, name: str):
    """t has exactly this shape (None: any extent along that axis)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dim() != len(shape) or any(e is not None and t.shape[i] != e for i, e in enumerate(shape)):
        want = "[" + ", ".join("*" if e is None else str(e) for e in shape) + "]"
        raise ValueError(f"{name}: shape {list(t.shape)}, expected {want}")


def _min_numel(t, n: int, name: str):
    if t is not None and t.numel() < n:
        raise ValueError(f"{name}: {t.numel()} elements, at least {n} needed")


def _min_bytes(t, n: int, name: str):
    if t is not None and t.numel() * t.element_size() < n:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, at least {n} needed")


def _check_cache(d: "CacheDesc", k_cache, v_cache, k_scale, v_scale):
    """The pools hold cache_bytes(d) bytes each; an e4m3 cache has Hkv scales."""
    n = cache_bytes(d)
    if n == 0:
        raise ValueError("invalid cache descriptor")
    _min_bytes(k_cache, n, "k_cache")
    _min_bytes(v_cache, n, "v_cache")
    if d.cache_dtype == E4M3:
        _min_numel(k_scale, d.num_kv_heads, "k_scale")
        _min_numel(v_scale, d.num_kv_heads, "v_scale")


def _check_out(out, shape, out_dtype: int):
    _shape(out, shape, "out")
    ok = (torch.bfloat16, torch.int16, torch.uint16) if out_dtype == OUT_BF16 else (torch.float32,)
    if out_dtype not in (OUT_BF16, OUT_F32):
        raise ValueError(f"out_dtype {out_dtype}: OUT_BF16 or OUT_F32")
    if out.dtype not in ok:
        raise ValueError(f"out: dtype {out.dtype} does not hold out_dtype {out_dtype}")


_BITS16 = (torch.bfloat16, torch.int16, torch.uint16)
_I32 = (torch.int32,)
_U32 = (torch.int32, torch.uint32)
_U8 = (torch.uint8,)
_F32 = (torch.float32,)


def desc(num_pages: int, num_kv_heads: int, cache_dtype: int = E4M3) -> CacheDesc:
    return CacheDesc(num_pages, PAGE_SIZE, num_kv_heads, HEAD_DIM, cache_dtype)


def cache_bytes(d: CacheDesc) -> int:
    return int(_cache_bytes(ctypes.byref(d)))


def cache_offset(d: CacheDesc, is_v: int, page: int, kv_head: int, slot: int, dim: int) -> int:
    return int(_cache_offset(ctypes.byref(d), is_v, page, kv_head, slot, dim))


def new_cache(d: CacheDesc, device="cuda"):
    """Allocate the K and V pools (uint8 byte tensors) for a descriptor."""
    n = cache_bytes(d)
    if n == 0:
        raise ValueError("invalid cache descriptor")
    k = torch.zeros(n, dtype=torch.uint8, device=device)
    v = torch.zeros(n, dtype=torch.uint8, device=device)
    return k, v


# ---------------------------------------------------------------------------
# page pool
# ---------------------------------------------------------------------------
class Pool:
    """Free list + per-page generation tags (host object in the library)."""

    def __init__(self, num_pages: int, seed: int = 0):
        h = _p()
        _check(_pool_create(num_pages, seed, ctypes.byref(h)), "pool_create")
        self._h = h
        self.num_pages = num_pages

    def close(self):
        if self._h:
            _pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc(self, n: int):
        import numpy as np
        ids = np.zeros(n, np.int32)
        tags = np.zeros(n, np.uint32)
        _check(_pool_alloc(self._h, n, ids.ctypes.data, tags.ctypes.data), "pool_alloc")
        return ids, tags

    def free(self, ids):
        import numpy as np
        a = np.ascontiguousarray(ids, np.int32)
        _check(_pool_free(self._h, a.size, a.ctypes.data), "pool_free")

    def share(self, ids):
        """Add one holder to each page (a request mapping a shared prefix); returns
        the pages' current tags, which the new holder records."""
        import numpy as np
        a = np.ascontiguousarray(ids, np.int32)
        _check(_pool_share(self._h, a.size, a.ctypes.data), "pool_share")
        return np.array([_pool_tag(self._h, int(i)) for i in a], np.uint32)

    def refcount(self, page_id: int) -> int:
        return int(_pool_refcount(self._h, page_id))

    def tag(self, page_id: int) -> int:
        return int(_pool_tag(self._h, page_id))

    @property
    def num_free(self) -> int:
        return int(_pool_num_free(self._h))

    def tags(self):
        import numpy as np
        out = np.zeros(self.num_pages, np.uint32)
        _check(_pool_read_tags(self._h, out.ctypes.data), "pool_read_tags")
        return out

    def sync(self, d_tags: torch.Tensor, stream=None):
        _min_numel(d_tags, self.num_pages, "d_tags")
        _dev(d_tags, _U32, "d_tags")
        _check(_pool_sync(self._h, d_tags.data_ptr(), _stream(stream)), "pool_sync")


# ---------------------------------------------------------------------------
# hot path
# ---------------------------------------------------------------------------
class Launch:
    """One entry point with its arguments checked and marshalled once: calling
    it calls the C function again with the same pointers and sizes (nothing is
    checked or allocated).  It holds the tensors it points into, which must keep
    their storage; their contents may change between calls.  Made by the hot-path
    functions below with prepare=True, for loops whose per-call host time
    matters."""
    __slots__ = ("_fn", "_args", "_what", "_result", "_keep")

    def __init__(self, fn, args, what, result, keep):
        self._fn, self._args, self._what, self._result, self._keep = fn, args, what, result, keep

    def __call__(self):
        _check(self._fn(*self._args), self._what)
        return self._result


def _run(fn, args, what, result, keep, prepare):
    if prepare:
        return Launch(fn, tuple(args), what, result, keep)
    _check(fn(*args), what)
    return result


def verify_tags(page_table, expected_tags, ctx_lens, pool_tags, abort=None, stream=None,
                prepare: bool = False):
    """Batched page-tag check; returns the uint8 abort tensor [B] (or, with
    prepare=True, a Launch that runs the check and returns it)."""
    _shape(ctx_lens, (None,), "ctx_lens")
    B = ctx_lens.shape[0]
    _shape(page_table, (B, None), "page_table")
    P = page_table.shape[1]
    _shape(expected_tags, (B, P), "expected_tags")
    _shape(pool_tags, (None,), "pool_tags")
    _min_numel(abort, B, "abort")
    if abort is None:
        abort = torch.empty(B, dtype=torch.uint8, device=ctx_lens.device)
    args = (_dev(page_table, _I32, "page_table"), _dev(expected_tags, _U32, "expected_tags"),
            P, _dev(ctx_lens, _I32, "ctx_lens"), B, _dev(pool_tags, _U32, "pool_tags"),
            pool_tags.shape[0], PAGE_SIZE, _dev(abort, _U8, "abort"), _stream(stream))
    return _run(_verify, args, "verify_tags", abort,
                (page_table, expected_tags, ctx_lens, pool_tags, abort), prepare)


def append(d: CacheDesc, k_cache, v_cache, k_scale, v_scale, k_new, v_new, token_seq, token_pos,
           page_table, abort=None, stream=None, prepare: bool = False):
    """Quantize-on-append of num_tokens new K/V rows ([T][Hkv][128] BF16)."""
    _shape(token_seq, (None,), "token_seq")
    T = token_seq.shape[0]
    _shape(token_pos, (T,), "token_pos")
    _shape(k_new, (T, d.num_kv_heads, HEAD_DIM), "k_new")
    _shape(v_new, (T, d.num_kv_heads, HEAD_DIM), "v_new")
    _shape(page_table, (None, None), "page_table")
    _min_numel(abort, page_table.shape[0], "abort")
    _check_cache(d, k_cache, v_cache, k_scale, v_scale)
    fp8 = d.cache_dtype == E4M3
    args = (ctypes.byref(d), _dev(k_cache, _U8 + _BITS16, "k_cache"),
            _dev(v_cache, _U8 + _BITS16, "v_cache"),
            _dev(k_scale, _F32, "k_scale", allow_none=not fp8),
            _dev(v_scale, _F32, "v_scale", allow_none=not fp8),
            _dev(k_new, _BITS16, "k_new"), _dev(v_new, _BITS16, "v_new"), T,
            _dev(token_seq, _I32, "token_seq"), _dev(token_pos, _I32, "token_pos"),
            page_table.shape[0], _dev(page_table, _I32, "page_table"), page_table.shape[1],
            _dev(abort, _U8, "abort", allow_none=True), _stream(stream))
    return _run(_append, args, "append", None,
                (d, k_cache, v_cache, k_scale, v_scale, k_new, v_new, token_seq, token_pos,
                 page_table, abort), prepare)


def _check_verify_append(d, k_cache, v_cache, k_scale, v_scale, new_pos, page_table,
                         expected_tags, pool_tags, abort, B):
    _check_cache(d, k_cache, v_cache, k_scale, v_scale)
    _shape(new_pos, (B,), "new_pos")
    _shape(page_table, (B, None), "page_table")
    _shape(expected_tags, tuple(page_table.shape), "expected_tags")
    _shape(pool_tags, (None,), "pool_tags")
    # the kernel reads the current tag of any page id below num_pages
    _min_numel(pool_tags, d.num_pages, "pool_tags")
    _min_numel(abort, B, "abort")


def verify_append(d: CacheDesc, k_cache, v_cache, k_scale, v_scale, k_new, v_new, new_pos,
                  page_table, expected_tags, ctx_lens, pool_tags, abort=None, stream=None,
                  prepare: bool = False):
    """Tag check + the step's append in one launch (one new token per request);
    returns the uint8 abort tensor [B]."""
    _shape(ctx_lens, (None,), "ctx_lens")
    B = ctx_lens.shape[0]
    _check_verify_append(d, k_cache, v_cache, k_scale, v_scale, new_pos, page_table,
                         expected_tags, pool_tags, abort, B)
    _shape(k_new, (B, d.num_kv_heads, HEAD_DIM), "k_new")
    _shape(v_new, (B, d.num_kv_heads, HEAD_DIM), "v_new")
    if abort is None:
        abort = torch.empty(B, dtype=torch.uint8, device=ctx_lens.device)
    fp8 = d.cache_dtype == E4M3
    args = (ctypes.byref(d), _dev(k_cache, _U8 + _BITS16, "k_cache"),
            _dev(v_cache, _U8 + _BITS16, "v_cache"),
            _dev(k_scale, _F32, "k_scale", allow_none=not fp8),
            _dev(v_scale, _F32, "v_scale", allow_none=not fp8),
            _dev(k_new, _BITS16, "k_new"), _dev(v_new, _BITS16, "v_new"),
            _dev(new_pos, _I32, "new_pos"), _dev(page_table, _I32, "page_table"),
            _dev(expected_tags, _U32, "expected_tags"), page_table.shape[1],
            _dev(ctx_lens, _I32, "ctx_lens"), B, _dev(pool_tags, _U32, "pool_tags"),
            _dev(abort, _U8, "abort"), _stream(stream))
    return _run(_verify_append, args, "verify_append", abort,
                (d, k_cache, v_cache, k_scale, v_scale, k_new, v_new, new_pos, page_table,
                 expected_tags, ctx_lens, pool_tags, abort), prepare)


def verify_append_q(d: CacheDesc, k_cache, v_cache, k_scale, v_scale, k_new, v_new, new_pos,
                    page_table, expected_tags, ctx_lens, pool_tags, abort=None, stream=None,
                    prepare: bool = False):
    """Tag check + the append of q_len new tokens per request in one launch:
    k_new / v_new [B][q_len][Hkv][128], token i of request b at position
    new_pos[b] + i; returns the uint8 abort tensor [B]."""
    _shape(ctx_lens, (None,), "ctx_lens")
    B = ctx_lens.shape[0]
    _shape(k_new, (B, None, d.num_kv_heads, HEAD_DIM), "k_new")
    T = k_new.shape[1]
    _shape(v_new, (B, T, d.num_kv_heads, HEAD_DIM), "v_new")
    _check_verify_append(d, k_cache, v_cache, k_scale, v_scale, new_pos, page_table,
                         expected_tags, pool_tags, abort, B)
    if abort is None:
        abort = torch.empty(B, dtype=torch.uint8, device=ctx_lens.device)
    fp8 = d.cache_dtype == E4M3
    args = (ctypes.byref(d), _dev(k_cache, _U8 + _BITS16, "k_cache"),
            _dev(v_cache, _U8 + _BITS16, "v_cache"),
            _dev(k_scale, _F32, "k_scale", allow_none=not fp8),
            _dev(v_scale, _F32, "v_scale", allow_none=not fp8),
            _dev(k_new, _BITS16, "k_new"), _dev(v_new, _BITS16, "v_new"),
            _dev(new_pos, _I32, "new_pos"), T, _dev(page_table, _I32, "page_table"),
            _dev(expected_tags, _U32, "expected_tags"), page_table.shape[1],
            _dev(ctx_lens, _I32, "ctx_lens"), B, _dev(pool_tags, _U32, "pool_tags"),
            _dev(abort, _U8, "abort"), _stream(stream))
    return _run(_verify_append_q, args, "verify_append_q", abort,
                (d, k_cache, v_cache, k_scale, v_scale, k_new, v_new, new_pos, page_table,
                 expected_tags, ctx_lens, pool_tags, abort), prepare)


def decode_num_workers(requested: int = 0) -> int:
    return int(_num_workers(requested))


def decode_workspace_size(d: CacheDesc, batch: int, num_q_heads: int, num_workers: int = 0) -> int:
    return int(_ws_size(ctypes.byref(d), batch, num_q_heads, num_workers))


def _check_decode(d, k_cache, v_cache, k_scale, v_scale, page_table, ctx_lens, abort, B):
    _check_cache(d, k_cache, v_cache, k_scale, v_scale)
    _shape(page_table, (B, None), "page_table")
    _shape(ctx_lens, (B,), "ctx_lens")
    _min_numel(abort, B, "abort")


def decode_attention(d: CacheDesc, k_cache, v_cache, k_scale, v_scale, q, page_table, ctx_lens,
                     abort=None, out=None, out_dtype: int = OUT_BF16,
                     sm_scale: Optional[float] = None, num_workers: int = 0, workspace=None,
                     stream=None, prepare: bool = False):
    """Paged decode attention; returns out [B][Hq][128] (bf16 or f32)."""
    _shape(q, (None, None, HEAD_DIM), "q")
    B, Hq, D = q.shape
    _check_decode(d, k_cache, v_cache, k_scale, v_scale, page_table, ctx_lens, abort, B)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), device=q.device,
                          dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32)
    _check_out(out, (B, Hq, D), out_dtype)
    need = decode_workspace_size(d, B, Hq, num_workers)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    fp8 = d.cache_dtype == E4M3
    args = (ctypes.byref(d), _dev(k_cache, _U8 + _BITS16, "k_cache"),
            _dev(v_cache, _U8 + _BITS16, "v_cache"),
            _dev(k_scale, _F32, "k_scale", allow_none=not fp8),
            _dev(v_scale, _F32, "v_scale", allow_none=not fp8),
            _dev(q, _BITS16, "q"), Hq, _dev(page_table, _I32, "page_table"),
            page_table.shape[1], _dev(ctx_lens, _I32, "ctx_lens"), B,
            float(sm_scale), _dev(abort, _U8, "abort", allow_none=True),
            _dev(out, (torch.bfloat16, torch.int16, torch.float32), "out"), out_dtype,
            num_workers, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream(stream))
    return _run(_decode, args, "decode_attention", out,
                (d, k_cache, v_cache, k_scale, v_scale, q, page_table, ctx_lens, abort, out,
                 workspace), prepare)


def decode_attention_noalloc(d: CacheDesc, k_cache, v_cache, k_scale, v_scale, q, page_table,
                             ctx_lens, out, abort=None, out_dtype: int = OUT_BF16,
                             sm_scale: Optional[float] = None, num_workers: int = 0,
                             stream=None, prepare: bool = False):
    """decode_attention without a workspace: the library's fixed device scratch
    (NOALLOC_SCRATCH_BYTES per device) holds the partial states, so nothing is
    allocated (out must be given).  Calls on one device share the scratch:
    overlapping calls race."""
    _shape(q, (None, None, HEAD_DIM), "q")
    B, Hq, D = q.shape
    _check_decode(d, k_cache, v_cache, k_scale, v_scale, page_table, ctx_lens, abort, B)
    _check_out(out, (B, Hq, D), out_dtype)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    fp8 = d.cache_dtype == E4M3
    args = (ctypes.byref(d), _dev(k_cache, _U8 + _BITS16, "k_cache"),
            _dev(v_cache, _U8 + _BITS16, "v_cache"),
            _dev(k_scale, _F32, "k_scale", allow_none=not fp8),
            _dev(v_scale, _F32, "v_scale", allow_none=not fp8),
            _dev(q, _BITS16, "q"), Hq, _dev(page_table, _I32, "page_table"),
            page_table.shape[1], _dev(ctx_lens, _I32, "ctx_lens"), B,
            float(sm_scale), _dev(abort, _U8, "abort", allow_none=True),
            _dev(out, (torch.bfloat16, torch.int16, torch.float32), "out"), out_dtype,
            num_workers, _stream(stream))
    return _run(_decode_noalloc, args, "decode_attention_noalloc", out,
                (d, k_cache, v_cache, k_scale, v_scale, q, page_table, ctx_lens, abort, out),
                prepare)


def decode_workspace_size_q(d: CacheDesc, batch: int, num_q_heads: int, q_len: int,
                            num_workers: int = 0) -> int:
    return int(_ws_size_q(ctypes.byref(d), batch, num_q_heads, q_len, num_workers))


def decode_attention_q(d: CacheDesc, k_cache, v_cache, k_scale, v_scale, q, page_table, ctx_lens,
                       abort=None, out=None, out_dtype: int = OUT_BF16,
                       sm_scale: Optional[float] = None, num_workers: int = 0, workspace=None,
                       stream=None, prepare: bool = False):
    """Decode attention with q_len queries per request (several new tokens checked
    at once; query i attends the cache up to its own token).  q [B][q_len][Hq][128];
    ctx_lens counts tokens after all q_len new ones; returns out [B][q_len][Hq][128]."""
    _shape(q, (None, None, None, HEAD_DIM), "q")
    B, T, Hq, D = q.shape
    _check_decode(d, k_cache, v_cache, k_scale, v_scale, page_table, ctx_lens, abort, B)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, T, Hq, D), device=q.device,
                          dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32)
    _check_out(out, (B, T, Hq, D), out_dtype)
    need = decode_workspace_size_q(d, B, Hq, T, num_workers)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    fp8 = d.cache_dtype == E4M3
    args = (ctypes.byref(d), _dev(k_cache, _U8 + _BITS16, "k_cache"),
            _dev(v_cache, _U8 + _BITS16, "v_cache"),
            _dev(k_scale, _F32, "k_scale", allow_none=not fp8),
            _dev(v_scale, _F32, "v_scale", allow_none=not fp8),
            _dev(q, _BITS16, "q"), Hq, T, _dev(page_table, _I32, "page_table"),
            page_table.shape[1], _dev(ctx_lens, _I32, "ctx_lens"), B,
            float(sm_scale), _dev(abort, _U8, "abort", allow_none=True),
            _dev(out, (torch.bfloat16, torch.int16, torch.float32), "out"), out_dtype,
            num_workers, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream(stream))
    return _run(_decode_q, args, "decode_attention_q", out,
                (d, k_cache, v_cache, k_scale, v_scale, q, page_table, ctx_lens, abort, out,
                 workspace), prepare)


def _groups(group_start, prefix_len):
    """Host int32 arrays of a prompt-group description (kept alive by the caller)."""
    import numpy as np
    gs = np.ascontiguousarray(np.asarray(group_start, dtype=np.int32))
    pl = np.ascontiguousarray(np.asarray(prefix_len, dtype=np.int32))
    if gs.ndim != 1 or pl.ndim != 1 or gs.size != pl.size + 1:
        raise ValueError("group_start needs one entry more than prefix_len")
    return gs, pl


def decode_workspace_size_shared(d: CacheDesc, batch: int, num_q_heads: int, max_pages: int,
                                 group_start, prefix_len, num_workers: int = 0) -> int:
    gs, pl = _groups(group_start, prefix_len)
    return int(_ws_size_shared(ctypes.byref(d), batch, num_q_heads, max_pages, pl.size,
                               gs.ctypes.data, pl.ctypes.data, num_workers))


def decode_attention_shared(d: CacheDesc, k_cache, v_cache, k_scale, v_scale, q, page_table,
                            ctx_lens, group_start, prefix_len, abort=None, out=None,
                            out_dtype: int = OUT_BF16, sm_scale: Optional[float] = None,
                            num_workers: int = 0, workspace=None, stream=None,
                            prepare: bool = False):
    """decode_attention for a batch whose requests [group_start[k],
    group_start[k+1]) continue prompt k of prefix_len[k] tokens (a multiple of
    16), on the pages their tables list first: each prompt's pages are read
    once per kv-head for its whole group.  Returns out [B][Hq][128]."""
    _shape(q, (None, None, HEAD_DIM), "q")
    B, Hq, D = q.shape
    _check_decode(d, k_cache, v_cache, k_scale, v_scale, page_table, ctx_lens, abort, B)
    gs, pl = _groups(group_start, prefix_len)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), device=q.device,
                          dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32)
    _check_out(out, (B, Hq, D), out_dtype)
    P = page_table.shape[1]
    need = decode_workspace_size_shared(d, B, Hq, P, gs, pl, num_workers)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    fp8 = d.cache_dtype == E4M3
    args = (ctypes.byref(d), _dev(k_cache, _U8 + _BITS16, "k_cache"),
            _dev(v_cache, _U8 + _BITS16, "v_cache"),
            _dev(k_scale, _F32, "k_scale", allow_none=not fp8),
            _dev(v_scale, _F32, "v_scale", allow_none=not fp8),
            _dev(q, _BITS16, "q"), Hq, pl.size, gs.ctypes.data, pl.ctypes.data,
            _dev(page_table, _I32, "page_table"), P, _dev(ctx_lens, _I32, "ctx_lens"), B,
            float(sm_scale), _dev(abort, _U8, "abort", allow_none=True),
            _dev(out, (torch.bfloat16, torch.int16, torch.float32), "out"), out_dtype,
            num_workers, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream(stream))
    return _run(_decode_shared, args, "decode_attention_shared", out,
                (d, k_cache, v_cache, k_scale, v_scale, q, page_table, ctx_lens, abort, out,
                 workspace, gs, pl), prepare)


def step(d: CacheDesc, k_cache, v_cache, k_scale, v_scale, q, k_new, v_new, new_pos,
         page_table, ctx_lens, expected_tags=None, pool_tags=None, abort=None, out=None,
         out_dtype: int = OUT_BF16, sm_scale: Optional[float] = None, num_workers: int = 0,
         workspace=None, stream=None):
    """One decode step of one layer in the pages' order: the tag check of every
    page the step reads, the append of each request's new token (skipped for
    aborted requests), then attention (+0 rows for them).  With expected_tags
    and pool_tags the check and the append are one launch (verify_append);
    without them this is the no-op tracker: append and attention, no check.
    q [B][Hq][128], k_new / v_new [B][Hkv][128] BF16 bits, new_pos [B] = L_b,
    ctx_lens [B] = L_b + 1.  Returns (out, abort); abort is None without the
    tracker.  Page allocation and the tag upload (Pool.alloc / Pool.sync)
    come before, on the host."""
    if (expected_tags is None) != (pool_tags is None):
        raise ValueError("expected_tags and pool_tags go together (both or neither)")
    if expected_tags is not None:
        abort = verify_append(d, k_cache, v_cache, k_scale, v_scale, k_new, v_new, new_pos,
                              page_table, expected_tags, ctx_lens, pool_tags, abort=abort,
                              stream=stream)
    else:
        seq = torch.arange(ctx_lens.shape[0], dtype=torch.int32, device=ctx_lens.device)
        append(d, k_cache, v_cache, k_scale, v_scale, k_new, v_new, seq, new_pos, page_table,
               stream=stream)
        abort = None
    out = decode_attention(d, k_cache, v_cache, k_scale, v_scale, q, page_table, ctx_lens,
                           abort=abort, out=out, out_dtype=out_dtype, sm_scale=sm_scale,
                           num_workers=num_workers, workspace=workspace, stream=stream)
    return out, abort


def debug_read_bandwidth(buf: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None):
    """Streaming read of every byte of buf (a contiguous device tensor, size a
    multiple of 16 bytes): the measurement reference for the tile loads.
    Returns the sink words (an XOR of what was read)."""
    if sink is None:
        sink = torch.empty(int(_read_sink_words()), dtype=torch.int32, device=buf.device)
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    _check(_read_bandwidth(buf.data_ptr(), buf.numel() * buf.element_size(),
                           _dev(sink, _I32, "sink"), _stream(stream)), "debug_read_bandwidth")
    return sink


def debug_convert_e4m3(codes: torch.Tensor, which: int, stream=None) -> torch.Tensor:
    out = torch.empty(codes.numel(), dtype=torch.float32, device=codes.device)
    _check(_debug_convert(_dev(codes, _U8, "codes"), out.data_ptr(), codes.numel(), which,
                          _stream(stream)), "debug_convert_e4m3")
    return out


def status_string(status: int) -> str:
    return _status_string(status).decode()


def raw_library():
    """The ctypes handle (used by tests that call the C ABI directly)."""
    return _lib
