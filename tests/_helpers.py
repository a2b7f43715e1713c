"""Test-side helpers shared by the GPU parity tests (not collected).

* `tile_index` -- the cache-tile layout documented in include/fp8kv.h,
  written out again here with numpy, so a layout mistake in the library's
  append or attention shows up as a parity failure;
* oracle-side state for a workload, built only from the numpy generator and
  the oracle (never from anything the GPU produced).
"""
from __future__ import annotations

import math

import numpy as np

import oracle
import workloads

D, S = 128, 16
SM_SCALE = float(np.float32(1.0 / math.sqrt(D)))


def tile_index(is_v: bool, elem_bytes: int) -> np.ndarray:
    """[slot][dim] -> element index inside one (page, kv-head) tile."""
    C = 16 // elem_bytes
    slot = np.arange(S)[:, None]
    d = np.arange(D)[None, :]
    if is_v:
        f = 4 * (d % 8) + slot % 4
        lane = 16 * (slot // 4) + d // 8
    else:
        f = d % 32 + 0 * slot
        lane = 16 * (d // 32) + slot
    byte = (f // C) * 1024 + 16 * lane + elem_bytes * (f % C)
    return byte // elem_bytes


def unswizzle(pool_host: np.ndarray, Hkv: int, cache_dtype: int, pages, is_v: bool) -> np.ndarray:
    """Logical [len(pages)][Hkv][16][128] view of the given pages of a pool."""
    eb = 1 if cache_dtype == 0 else 2
    dt = np.uint8 if eb == 1 else np.uint16
    tile_elems = S * D
    arr = pool_host.view(dt).reshape(-1, Hkv, tile_elems)
    idx = tile_index(is_v, eb)
    sel = arr[np.asarray(pages, np.int64)]
    return sel[:, :, idx]


def oracle_state(w: workloads.Workload, ksh, vsh, cache_dtype=0, requests=None,
                 include_new=True, abort=None):
    """Logical K/V caches holding the requests' history (and, unless aborted,
    the appended token), encoded by the oracle from numpy-generated bits."""
    K, V = oracle.new_cache(w.num_pages, w.Hkv, cache_dtype)
    reqs = range(w.B) if requests is None else requests
    for b in reqs:
        L = int(w.ctx_before[b])
        if L > 0:
            kb = w.kv_tokens("k", b, 0, L)
            vb = w.kv_tokens("v", b, 0, L)
            oracle.append(K, V, ksh, vsh, kb, vb, np.full(L, b, np.int32),
                          np.arange(L, dtype=np.int32), w.page_table, cache_dtype=cache_dtype)
        if include_new:
            kn = w.kv_tokens("k", b, L, L + 1)
            vn = w.kv_tokens("v", b, L, L + 1)
            oracle.append(K, V, ksh, vsh, kn, vn, np.array([b], np.int32),
                          np.array([L], np.int32), w.page_table, abort=abort,
                          cache_dtype=cache_dtype)
    return K, V


def bf16_to_f32(bits) -> np.ndarray:
    return workloads.bf16_bits_to_f32(np.asarray(bits).view(np.uint16))


def bf16_neighbours_ok(bf16_bits: np.ndarray, ref64: np.ndarray) -> np.ndarray:
    """Whether each bf16 value is one of the two bf16 numbers that bracket the
    binary64 value (the value itself when it is a bf16 number).  Normal range
    only (|ref| >= 2^-126): bf16 keeps 8 significant bits there."""
    got = bf16_to_f32(bf16_bits).astype(np.float64)
    a = np.abs(ref64)
    _, e = np.frexp(a)                       # a = m * 2^e, m in [0.5, 1)
    sp = np.ldexp(1.0, e - 8)                # bf16 spacing at a
    lo = np.floor(a / sp) * sp
    hi = np.ceil(a / sp) * sp
    same_sign = (np.signbit(got) == np.signbit(ref64)) | (got == 0)
    return same_sign & ((np.abs(got) == lo) | (np.abs(got) == hi))


def check_outputs(got_f32: np.ndarray, got_bf16_bits: np.ndarray, ref64: np.ndarray,
                  tol: float = 2e-3):
    """Tolerance of the attention output (reading A9 of the 2e-3 bound).

    f32 mode: |o_gpu - o_oracle| <= tol everywhere.
    bf16 mode: the bf16 output is bitwise the round-to-nearest-even of the f32
    output; where |o_oracle| < 1 it is within tol of the oracle, where
    |o_oracle| >= 1 it is one of the two bf16 neighbours of the oracle's
    value (bf16 spacing alone exceeds tol there).
    Returns the max abs error of the f32 output."""
    err = np.abs(got_f32.astype(np.float64) - ref64)
    assert np.isfinite(got_f32).all()
    assert err.max() <= tol, f"max abs err {err.max():.3e}"
    if got_bf16_bits is not None:
        gb = np.asarray(got_bf16_bits).view(np.uint16)
        f = np.ascontiguousarray(got_f32, np.float32).view(np.uint32).astype(np.uint64)
        rne = ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)
        assert (gb == rne).all(), "bf16 output is not the RNE of the f32 output"
        small = np.abs(ref64) < 1.0
        eb = np.abs(bf16_to_f32(gb).astype(np.float64) - ref64)
        assert (eb[small] <= tol).all(), f"bf16 err {eb[small].max():.3e} where |o| < 1"
        assert bf16_neighbours_ok(gb[~small], ref64[~small]).all(), \
            "bf16 output not a neighbour of the oracle where |o| >= 1"
    return float(err.max())


def bf16_differences(got_bf16_bits: np.ndarray, ref_bf16_bits: np.ndarray) -> int:
    """bf16 output elements that differ from the oracle's own bf16 rounding of
    its binary64 result (reported, not bounded: a value within the f32 error
    of a rounding midpoint may go either way)."""
    return int((np.asarray(got_bf16_bits).view(np.uint16) !=
                np.asarray(ref_bf16_bits).view(np.uint16)).sum())
