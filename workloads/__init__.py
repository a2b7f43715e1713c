"""Seeded synthetic inputs for one paged decode step.

This module only *generates inputs*.  It holds none of the method's
arithmetic (no tag check, no FP8 encoding, no attention): those live in the
HIP library and, independently, in the CPU oracle.  Both sides receive the
bits produced here.

Element values come from a counter-based generator so that any slice of any
tensor can be regenerated on its own, bit-identically, by two backends:

* ``numpy`` (host, uint32 arithmetic) -- used by the oracle side;
* ``torch`` (any device, int64 arithmetic masked to 32 bits) -- used to build
  full-size inputs directly in device memory;
* ``host`` (the same generator in C with OpenMP, ``gen.c``) -- the numpy
  backend's values at full-size speed, for oracle-side inputs of the full
  workloads (checked against the numpy backend bit for bit).

Generator: the 32-bit integer finaliser "lowbias32" (x ^= x>>16; x *= 0x7feb352d;
x ^= x>>15; x *= 0x846ca68b; x ^= x>>16), applied to (element counter + stream
key) mod 2^32.  The high 16 bits index a 65,536-entry table of N(0,1)
quantiles at (i+0.5)/65536, each rounded to BF16, so every drawn value is a
BF16 number approximately N(0,1) distributed.  The low 16 bits decide
outliers where a workload asks for them.

Workloads follow the five synthetic decode configurations of the design
(tiny, uniform, ragged, long-context, capacity+integrity).  A workload's
context length L_b is the number of tokens cached *before* the step: the step appends token
L_b and attends over L_b + 1 tokens, i.e. n_b = ceil((L_b+1)/16) pages.
"""
from __future__ import annotations

import dataclasses
import statistics
from typing import Optional

import numpy as np

D_HEAD = 128
PAGE = 16

_M32 = 0xFFFFFFFF
_C1 = 0x7FEB352D
_C2 = 0x846CA68B

# tensor ids that key the streams
_T_Q, _T_K, _T_V = 1, 2, 3
_PREFIX_ROW = 1 << 24   # stream row of a common prompt (requests are rows 0..B-1)


def _build_normal_table() -> np.ndarray:
    nd = statistics.NormalDist()
    vals = np.array([nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)],
                    dtype=np.float32)
    bits = vals.view(np.uint32).astype(np.uint64)
    rnd = ((bits >> 16) & 1) + 0x7FFF
    return ((bits + rnd) >> 16).astype(np.uint16)


NORMAL_BF16 = _build_normal_table()          # uint16 BF16 bit patterns
BF16_20 = np.uint16(0x41A0)                   # +20.0
BF16_25 = np.uint16(0x41C8)                   # +25.0


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# counter-based generator, two backends
# --------------------------------------------------------------------------
_GEN_LIB = None


def _gen_lib():
    """ctypes handle of libgen.so (built with gcc on first use)."""
    global _GEN_LIB
    if _GEN_LIB is None:
        import ctypes
        import os
        here = os.path.dirname(os.path.abspath(__file__))
        path = os.path.join(here, "libgen.so")
        if not os.path.exists(path):
            import importlib.util
            spec = importlib.util.spec_from_file_location("workloads_build",
                                                          os.path.join(here, "build.py"))
            mod = importlib.util.module_from_spec(spec)
            spec.loader.exec_module(mod)
            mod.build()
        lib = ctypes.CDLL(path)
        lib.gen_draw_bits.restype = None
        lib.gen_draw_bits.argtypes = [ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64,
                                      ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint16,
                                      ctypes.c_void_p]
        _GEN_LIB = lib
    return _GEN_LIB


def _draw_host(key: int, start: int, count: int, outlier_per_65536: int,
               outlier_bits) -> np.ndarray:
    out = np.empty(count, np.uint16)
    _gen_lib().gen_draw_bits(int(key) & _M32, int(start), int(count),
                             NORMAL_BF16.ctypes.data, int(outlier_per_65536),
                             int(outlier_bits), out.ctypes.data)
    return out


def _hash_np(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.uint32, copy=True)
    x ^= x >> np.uint32(16)
    x *= np.uint32(_C1)
    x ^= x >> np.uint32(15)
    x *= np.uint32(_C2)
    x ^= x >> np.uint32(16)
    return x


def _hash_scalar(x: int) -> int:
    x = int(x) & _M32
    x ^= x >> 16
    x = (x * _C1) & _M32
    x ^= x >> 15
    x = (x * _C2) & _M32
    x ^= x >> 16
    return x


def _hash_torch(x):
    x = x ^ (x >> 16)
    x = (x * _C1) & _M32
    x = x ^ (x >> 15)
    x = (x * _C2) & _M32
    x = x ^ (x >> 16)
    return x


def stream_key(seed: int, tensor_id: int, row: int) -> int:
    seed, tensor_id, row = int(seed), int(tensor_id), int(row)   # never numpy ints
    k = _hash_scalar(seed * 0x9E3779B1 + 0x85EBCA77)
    k = _hash_scalar(k ^ (tensor_id * 0xC2B2AE3D))
    return _hash_scalar(k + row * 0x27D4EB2F)


def draw_bits(key: int, start: int, count: int, backend: str = "numpy",
              device=None, outlier_per_65536: int = 0, outlier_bits=BF16_20):
    """BF16 bit patterns for counters [start, start+count) of one stream.

    numpy and host backends return uint16; torch backend returns int16 (same
    bits).
    """
    if count == 0:
        if backend in ("numpy", "host"):
            return np.zeros(0, np.uint16)
        import torch
        return torch.zeros(0, dtype=torch.int16, device=device)
    key, start, count = int(key), int(start), int(count)
    if backend == "host":
        return _draw_host(key, start, count, outlier_per_65536, outlier_bits)
    if backend == "numpy":
        ctr = np.arange(start, start + count, dtype=np.uint64)
        x = ((ctr + np.uint64(key)) & np.uint64(_M32)).astype(np.uint32)
        h = _hash_np(x)
        out = NORMAL_BF16[(h >> np.uint32(16)).astype(np.int64)]
        if outlier_per_65536:
            lo = h & np.uint32(0xFFFF)
            sel = lo < np.uint32(outlier_per_65536)
            neg = (h >> np.uint32(15)) & np.uint32(1)
            ob = np.where(neg == 1, np.uint16(int(outlier_bits) | 0x8000),
                          np.uint16(outlier_bits))
            out = np.where(sel, ob, out).astype(np.uint16)
        return out
    import torch
    ctr = torch.arange(start, start + count, dtype=torch.int64, device=device)
    h = _hash_torch((ctr + key) & _M32)
    table = _torch_table(device)
    out = table[(h >> 16)]
    if outlier_per_65536:
        sel = (h & 0xFFFF) < outlier_per_65536
        neg = ((h >> 15) & 1) == 1
        pos_v = torch.tensor(np.int16(np.uint16(outlier_bits).view(np.int16)),
                             device=device)
        neg_v = torch.tensor(np.uint16(int(outlier_bits) | 0x8000).view(np.int16),
                             device=device)
        out = torch.where(sel, torch.where(neg, neg_v, pos_v), out)
    return out


def draw_bits_at(key: int, counters: np.ndarray, outlier_per_65536: int = 0,
                 outlier_bits=BF16_20) -> np.ndarray:
    """numpy backend of draw_bits for an explicit array of counters."""
    key = int(key)
    ctr = np.asarray(counters, dtype=np.uint64)
    x = ((ctr + np.uint64(key)) & np.uint64(_M32)).astype(np.uint32)
    h = _hash_np(x)
    out = NORMAL_BF16[(h >> np.uint32(16)).astype(np.int64)]
    if outlier_per_65536:
        sel = (h & np.uint32(0xFFFF)) < np.uint32(outlier_per_65536)
        neg = (h >> np.uint32(15)) & np.uint32(1)
        ob = np.where(neg == 1, np.uint16(int(outlier_bits) | 0x8000), np.uint16(outlier_bits))
        out = np.where(sel, ob, out).astype(np.uint16)
    return out


_TABLE_CACHE: dict = {}


def _torch_table(device):
    import torch
    key = str(device)
    if key not in _TABLE_CACHE:
        _TABLE_CACHE[key] = torch.from_numpy(NORMAL_BF16.view(np.int16).copy()).to(device)
    return _TABLE_CACHE[key]


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    ctx_before: np.ndarray        # int32 [B]: L_b, tokens cached before the step
    num_pages: int
    page_table: np.ndarray        # int32 [B][P]; -1 beyond n_b
    expected_tags: np.ndarray     # uint32 [B][P]
    pool_tags: np.ndarray         # uint32 [num_pages]: current tag per physical page
    stale: np.ndarray             # bool [B][P]: entries whose tag is stale
    outlier_per_65536: int = 0    # K/V outliers at +-20
    saturate_new: bool = False    # overwrite 4 values of the appended token with +-25
    D: int = D_HEAD
    S: int = PAGE
    # tokens [0, prefix_len) of every request are one common stream (a shared
    # prompt); prefix_shared: their pages are the same physical pages for all.
    # With prompt_of (one prompt id per request, -1 for none) and prompt_lens,
    # each request continues its own prompt instead.
    prefix_len: int = 0
    prefix_shared: bool = False
    prompt_of: Optional[np.ndarray] = None
    prompt_lens: tuple = ()

    def prompt(self, b: int):
        """(prompt id, prompt tokens) of request b; (-1, 0) without one."""
        if self.prompt_of is None:
            return (0, self.prefix_len) if self.prefix_len > 0 else (-1, 0)
        k = int(self.prompt_of[b])
        return (k, int(self.prompt_lens[k])) if k >= 0 else (-1, 0)

    def first_of_prompt(self, b: int) -> bool:
        """Whether b is the first request of its prompt (the one whose appends
        write the shared pages)."""
        k, _ = self.prompt(b)
        if k < 0:
            return True
        if self.prompt_of is None:
            return b == 0
        return int(np.flatnonzero(self.prompt_of == k)[0]) == b

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def ctx_lens(self) -> np.ndarray:
        """Tokens attention reads per request (L_b + 1)."""
        return (self.ctx_before + 1).astype(np.int32)

    @property
    def n_pages(self) -> np.ndarray:
        return ((self.ctx_lens + self.S - 1) // self.S).astype(np.int32)

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def expected_abort(self) -> np.ndarray:
        """Requests holding a stale entry among the pages they read."""
        out = np.zeros(self.B, np.uint8)
        for b in range(self.B):
            out[b] = 1 if self.stale[b, : self.n_pages[b]].any() else 0
        return out

    # ---- element streams -------------------------------------------------
    def _kv_key(self, which: str, b: int) -> int:
        return stream_key(self.seed, _T_K if which == "k" else _T_V, b)

    def _prefix_key(self, which: str, k: int = 0) -> int:
        return stream_key(self.seed, _T_K if which == "k" else _T_V, _PREFIX_ROW + k)

    def _split(self, b: int, t0: int, t1: int):
        """[t0, t1) as (prompt stream?, start, end) runs: the request's prompt
        stream, then its own stream (counters keep their token positions)."""
        _, p = self.prompt(b)
        runs = []
        if t0 < min(t1, p):
            runs.append((True, t0, min(t1, p)))
        if max(t0, p) < t1:
            runs.append((False, max(t0, p), t1))
        return runs

    def kv_tokens(self, which: str, b: int, t0: int, t1: int,
                  backend: str = "numpy", device=None, with_saturation=True):
        """BF16 bits of K or V for request b, tokens [t0, t1), shape [t][Hkv][D].

        Token L_b is the token appended by the step.  When the workload asks
        for saturation, 4 values of that token in kv-head 0 are replaced by
        +-25 after scale calibration (they are excluded from amax)."""
        per_tok = self.Hkv * self.D
        k, _ = self.prompt(b)
        parts = [draw_bits(self._prefix_key(which, k) if pre else self._kv_key(which, b),
                           a * per_tok, (c - a) * per_tok, backend, device, self.outlier_per_65536)
                 for pre, a, c in self._split(b, t0, t1)]
        host = backend in ("numpy", "host")
        if len(parts) == 1:
            bits = parts[0]
        elif host:
            bits = np.concatenate(parts)
        else:
            import torch
            bits = torch.cat(parts)
        if host:
            bits = bits.reshape(t1 - t0, self.Hkv, self.D)
        else:
            bits = bits.view(t1 - t0, self.Hkv, self.D)
        L = int(self.ctx_before[b])
        if with_saturation and self.saturate_new and t0 <= L < t1:
            for d, sgn in zip((5, 40, 77, 120), (0, 0x8000, 0, 0x8000)):
                v = np.uint16(int(BF16_25) | sgn)
                if host:
                    bits[L - t0, 0, d] = v
                else:
                    bits[L - t0, 0, d] = int(v.view(np.int16))
        return bits

    def kv_tokens_head(self, which: str, b: int, t0: int, t1: int, g: int,
                       with_saturation=True) -> np.ndarray:
        """The same bits as kv_tokens(...)[:, g, :] (numpy), generated for one
        kv-head only: shape [t][D]."""
        d = np.arange(self.D, dtype=np.uint64)[None, :]
        parts = []
        kp, _ = self.prompt(b)
        for pre, a, c in self._split(b, t0, t1):
            t = np.arange(a, c, dtype=np.uint64)[:, None]
            ctr = (t * np.uint64(self.Hkv) + np.uint64(g)) * np.uint64(self.D) + d
            key = self._prefix_key(which, kp) if pre else self._kv_key(which, b)
            parts.append(draw_bits_at(key, ctr.ravel(), self.outlier_per_65536))
        bits = (np.concatenate(parts) if parts else np.zeros(0, np.uint16)).reshape(t1 - t0, self.D)
        L = int(self.ctx_before[b])
        if with_saturation and self.saturate_new and g == 0 and t0 <= L < t1:
            for dd, sgn in zip((5, 40, 77, 120), (0, 0x8000, 0, 0x8000)):
                bits[L - t0, dd] = np.uint16(int(BF16_25) | sgn)
        return bits

    def q_bits(self, backend: str = "numpy", device=None):
        """BF16 bits of Q, shape [B][Hq][D]."""
        rows = []
        for b in range(self.B):
            rows.append(draw_bits(stream_key(self.seed, _T_Q, b), 0, self.Hq * self.D,
                                  backend, device))
        if backend == "numpy":
            return np.stack(rows).reshape(self.B, self.Hq, self.D)
        import torch
        return torch.stack(rows).view(self.B, self.Hq, self.D)

    def q_bits_multi(self, q_len: int, backend: str = "numpy", device=None):
        """BF16 bits of q_len queries per request (speculative verification),
        shape [B][q_len][Hq][D].  Query i belongs to the new token at position
        L_b + 1 - q_len + i and is token q_len-1-i of the request's Q stream, so
        the newest query (i = q_len-1) is the one q_bits gives."""
        n = self.Hq * self.D
        rows = [draw_bits(stream_key(self.seed, _T_Q, b), 0, q_len * n, backend, device)
                for b in range(self.B)]
        if backend == "numpy":
            return np.stack(rows).reshape(self.B, q_len, self.Hq, self.D)[:, ::-1].copy()
        import torch
        return torch.stack(rows).view(self.B, q_len, self.Hq, self.D).flip(1).contiguous()

    def new_kv_bits(self, which: str, backend: str = "numpy", device=None):
        """BF16 bits of the appended token (position L_b) per request, [B][Hkv][D]."""
        rows = [self.kv_tokens(which, b, int(self.ctx_before[b]), int(self.ctx_before[b]) + 1,
                               backend, device)[0] for b in range(self.B)]
        if backend == "numpy":
            return np.stack(rows)
        import torch
        return torch.stack(rows)

    def amax_numpy(self, which: str) -> np.ndarray:
        """Per-kv-head max |x| over every generated value (history + new token,
        saturation overrides excluded).  Host backend; small workloads only."""
        am = np.zeros(self.Hkv, np.float32)
        for b in range(self.B):
            x = self.kv_tokens(which, b, 0, int(self.ctx_before[b]) + 1,
                               with_saturation=False)
            a = np.abs(bf16_bits_to_f32(x)).max(axis=(0, 2))
            am = np.maximum(am, a)
        return am


def scales_from_amax(amax: np.ndarray) -> np.ndarray:
    """Calibration recipe of the workloads: scale = fl32(amax / 448); amax==0 -> 1."""
    a = np.asarray(amax, dtype=np.float32)
    s = a / np.float32(448.0)
    return np.where(a > 0, s, np.float32(1.0)).astype(np.float32)


def _assign_pages(rng: np.random.Generator, n_pages: np.ndarray, pool: int):
    B = len(n_pages)
    P = int(n_pages.max())
    total = int(n_pages.sum())
    assert total <= pool, (total, pool)
    perm = rng.permutation(pool).astype(np.int32)
    pt = np.full((B, P), -1, np.int32)
    off = 0
    for b in range(B):
        n = int(n_pages[b])
        pt[b, :n] = perm[off: off + n]
        off += n
    return pt


def make(config: int, seed: Optional[int] = None, *, stale_mode: str = "entries",
         batch: Optional[int] = None) -> Workload:
    """Build workload `config` (1..5).  `seed` defaults to the config number.

    config 5's `stale_mode`: "entries" marks 1% of all used page-table entries
    stale; "requests" gives 1% of requests one stale entry each.
    `batch` truncates the request list (sampled runs)."""
    if seed is None:
        seed = config
    rng = np.random.Generator(np.random.PCG64(seed))
    outl, sat = 0, False
    stale_frac = 0.0
    pool = None
    if config == 1:
        name, B, Hq, Hkv = "tiny", 4, 8, 2
        L = np.array([17, 64, 100, 256], np.int32)
        pool = 64
    elif config == 2:
        name, B, Hq, Hkv = "uniform_32x8192", 32, 64, 8
        L = np.full(B, 8192, np.int32)
    elif config == 3:
        name, B, Hq, Hkv = "ragged_64_u1k_32k", 64, 64, 8
        L = rng.integers(1024, 32768, size=B, endpoint=True).astype(np.int32)
    elif config == 4:
        name, B, Hq, Hkv = "long_4x131072", 4, 64, 8
        L = np.full(B, 131072, np.int32)
        outl, sat = 66, True          # 66/65536 ~= 0.1%
    elif config == 5:
        name, B, Hq, Hkv = "capacity_256_log512_16k", 256, 32, 4
        L = np.exp(rng.uniform(np.log(512), np.log(16384), size=B)).astype(np.int32)
        pool = 81250
        stale_frac = 0.01
    else:
        raise ValueError(config)
    if batch is not None:
        B = batch
        L = L[:B]
    n_pages = (L + 1 + PAGE - 1) // PAGE
    if pool is None:
        pool = int(n_pages.sum())
    pt = _assign_pages(rng, n_pages, pool)
    P = pt.shape[1]
    etag = np.zeros((B, P), np.uint32)
    tags = rng.integers(0, 2**32, size=pool, dtype=np.uint64).astype(np.uint32)
    stale = np.zeros((B, P), bool)
    used = pt >= 0
    etag[used] = tags[pt[used]]
    if stale_frac > 0:
        if stale_mode == "entries":
            idx = np.flatnonzero(used.ravel())
            k = int(round(stale_frac * idx.size))
            pick = rng.choice(idx, size=k, replace=False)
            stale.ravel()[pick] = True
        elif stale_mode == "requests":
            k = max(1, int(round(stale_frac * B)))
            reqs = rng.choice(B, size=k, replace=False)
            for b in reqs:
                i = int(rng.integers(0, n_pages[b]))
                stale[b, i] = True
        else:
            raise ValueError(stale_mode)
        # the physical page was freed and handed out again: its tag moved on
        for b, i in zip(*np.nonzero(stale)):
            tags[pt[b, i]] = np.uint32((int(etag[b, i]) + 1) & _M32)
    return Workload(name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, ctx_before=L.astype(np.int32),
                    num_pages=pool, page_table=pt, expected_tags=etag, pool_tags=tags,
                    stale=stale, outlier_per_65536=outl, saturate_new=sat)


def shared_prefix(B: int = 64, prefix_len: int = 16384, suffix_max: int = 2048, Hq: int = 64,
                  Hkv: int = 8, seed: int = 6, shared: bool = True) -> Workload:
    """B requests continuing one common prompt of prefix_len tokens (a multiple of
    16), each with its own U[16, suffix_max] tokens after it.  shared: the
    prefix's pages are one set of physical pages mapped by every request (one
    holder each, the same tags); otherwise every request holds its own copy of
    the same values (the baseline without cache reuse).  Suffix lengths and the
    values do not depend on `shared`."""
    assert prefix_len % PAGE == 0
    rng = np.random.Generator(np.random.PCG64(seed))
    L = (prefix_len + rng.integers(16, suffix_max, size=B, endpoint=True)).astype(np.int32)
    n_pages = (L + 1 + PAGE - 1) // PAGE
    P0 = prefix_len // PAGE
    own = n_pages - P0 if shared else n_pages
    pool = int(own.sum()) + (P0 if shared else 0)
    perm = rng.permutation(pool).astype(np.int32)
    pt = np.full((B, int(n_pages.max())), -1, np.int32)
    off = 0
    if shared:
        pt[:, :P0] = perm[:P0]
        off = P0
    for b in range(B):
        k = int(own[b])
        pt[b, int(n_pages[b]) - k: int(n_pages[b])] = perm[off: off + k]
        off += k
    tags = rng.integers(0, 2**32, size=pool, dtype=np.uint64).astype(np.uint32)
    etag = np.zeros(pt.shape, np.uint32)
    used = pt >= 0
    etag[used] = tags[pt[used]]
    name = f"{'shared' if shared else 'private'}_prefix_{B}x{prefix_len}"
    return Workload(name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, ctx_before=L, num_pages=pool,
                    page_table=pt, expected_tags=etag, pool_tags=tags,
                    stale=np.zeros(pt.shape, bool), prefix_len=prefix_len, prefix_shared=shared)


def shared_prompts(groups, plain: int = 0, suffix_max: int = 256, Hq: int = 8, Hkv: int = 2,
                   seed: int = 9) -> Workload:
    """Several prompts, each continued by a group of requests that map its pages
    (groups: list of (requests, prompt tokens), prompt tokens a multiple of
    16), then `plain` requests without a shared prompt.  Everyone has
    U[16, suffix_max] own tokens (plain requests: that many in total)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    prompt_of, L = [], []
    for k, (n, plen) in enumerate(groups):
        assert plen % PAGE == 0
        prompt_of += [k] * n
        L += list(plen + rng.integers(16, suffix_max, size=n, endpoint=True))
    prompt_of += [-1] * plain
    L += list(rng.integers(16, suffix_max, size=plain, endpoint=True))
    L = np.array(L, np.int32)
    prompt_of = np.array(prompt_of, np.int32)
    B = len(L)
    n_pages = (L + 1 + PAGE - 1) // PAGE
    P0 = np.array([groups[k][1] // PAGE if k >= 0 else 0 for k in prompt_of], np.int64)
    pool = int((n_pages - P0).sum()) + sum(p // PAGE for _, p in groups)
    perm = rng.permutation(pool).astype(np.int32)
    pt = np.full((B, int(n_pages.max())), -1, np.int32)
    off = 0
    shared = {}
    for k, (_, plen) in enumerate(groups):
        shared[k] = perm[off: off + plen // PAGE]
        off += plen // PAGE
    for b in range(B):
        k = int(prompt_of[b])
        p0 = int(P0[b])
        if k >= 0:
            pt[b, :p0] = shared[k]
        own = int(n_pages[b]) - p0
        pt[b, p0: p0 + own] = perm[off: off + own]
        off += own
    tags = rng.integers(0, 2**32, size=pool, dtype=np.uint64).astype(np.uint32)
    etag = np.zeros(pt.shape, np.uint32)
    used = pt >= 0
    etag[used] = tags[pt[used]]
    return Workload(name=f"shared_prompts_{len(groups)}", seed=seed, B=B, Hq=Hq, Hkv=Hkv,
                    ctx_before=L, num_pages=pool, page_table=pt, expected_tags=etag,
                    pool_tags=tags, stale=np.zeros(pt.shape, bool), prefix_shared=True,
                    prompt_of=prompt_of, prompt_lens=tuple(p for _, p in groups))


def custom(name: str, ctx_before, Hq: int, Hkv: int, seed: int = 7,
           pool_slack: int = 0, outlier_per_65536: int = 0) -> Workload:
    """A small workload with explicit lengths (edge-case tests)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    L = np.asarray(ctx_before, np.int32)
    n_pages = (L + 1 + PAGE - 1) // PAGE
    pool = int(n_pages.sum()) + pool_slack
    pt = _assign_pages(rng, n_pages, pool)
    tags = rng.integers(0, 2**32, size=pool, dtype=np.uint64).astype(np.uint32)
    etag = np.zeros(pt.shape, np.uint32)
    used = pt >= 0
    etag[used] = tags[pt[used]]
    return Workload(name=name, seed=seed, B=len(L), Hq=Hq, Hkv=Hkv, ctx_before=L,
                    num_pages=pool, page_table=pt, expected_tags=etag, pool_tags=tags,
                    stale=np.zeros(pt.shape, bool), outlier_per_65536=outlier_per_65536)
