"""Device-resident state for one decode step of a workload.

Inputs are drawn on the device by the torch backend of the seeded generator
(bit-identical to the numpy backend the oracle side uses).  The cache is then
filled by the library's own append entry point -- the way a prefill would
write it -- so every byte in HBM is produced by the product path.  Scales
follow the workloads' calibration recipe (amax over every generated value of
a kv-head, / 448), amax being taken with torch on the generated data.

Nothing here computes any part of the method.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

import decode_attention_paged_fp8kv_amd as fp8kv

from . import Workload, scales_from_amax


@dataclasses.dataclass
class DeviceStep:
    w: Workload
    desc: "fp8kv.CacheDesc"
    K: torch.Tensor
    V: torch.Tensor
    k_scale: torch.Tensor
    v_scale: torch.Tensor
    k_scale_host: np.ndarray
    v_scale_host: np.ndarray
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    page_table: torch.Tensor
    expected_tags: torch.Tensor
    pool_tags: torch.Tensor
    ctx_lens: torch.Tensor      # L_b + 1
    token_seq: torch.Tensor
    token_pos: torch.Tensor     # L_b
    abort: torch.Tensor
    num_workers: int
    workspace: Optional[torch.Tensor]
    out: torch.Tensor
    # the default step's launches, prepared once per stream (a serving loop's
    # way: no per-call argument checks on the host), with and without the tracker
    _prepared: Optional[dict] = dataclasses.field(default=None, repr=False)

    @property
    def cache_dtype(self) -> int:
        return self.desc.cache_dtype

    def verify(self, stream=None):
        fp8kv.verify_tags(self.page_table, self.expected_tags, self.ctx_lens, self.pool_tags,
                          abort=self.abort, stream=stream)

    def append(self, use_abort=True, stream=None):
        fp8kv.append(self.desc, self.K, self.V, self.k_scale, self.v_scale, self.k_new,
                     self.v_new, self.token_seq, self.token_pos, self.page_table,
                     abort=self.abort if use_abort else None, stream=stream)

    def verify_append(self, stream=None):
        fp8kv.verify_append(self.desc, self.K, self.V, self.k_scale, self.v_scale, self.k_new,
                            self.v_new, self.token_pos, self.page_table, self.expected_tags,
                            self.ctx_lens, self.pool_tags, abort=self.abort, stream=stream)

    def decode(self, use_abort=True, out_dtype=fp8kv.OUT_BF16, out=None, stream=None,
               num_workers=None):
        if out is None:
            out = self.out if out_dtype == fp8kv.OUT_BF16 else torch.empty(
                self.out.shape, dtype=torch.float32, device=self.out.device)
        nw = self.num_workers if num_workers is None else num_workers
        return fp8kv.decode_attention(
            self.desc, self.K, self.V, self.k_scale, self.v_scale, self.q, self.page_table,
            self.ctx_lens, abort=self.abort if use_abort else None, out=out,
            out_dtype=out_dtype, num_workers=nw,
            workspace=self.workspace if nw == self.num_workers else None, stream=stream)

    def _prepare(self, check_tags: bool):
        """The default step's launches (fused check + append and attention with
        the tracker; append and attention without it), checked and marshalled
        once per stream and set of tensors: both forms then run the same launch
        path, one C call per kernel launch."""
        h = (check_tags, torch.cuda.current_stream().cuda_stream, self.num_workers,
             *map(id, (self.K, self.V, self.k_scale, self.v_scale, self.k_new, self.v_new,
                       self.token_seq, self.token_pos, self.page_table, self.expected_tags,
                       self.ctx_lens, self.pool_tags, self.abort, self.q, self.out,
                       self.workspace)))
        cache = self._prepared if self._prepared is not None else {}
        self._prepared = cache
        if cache.get(check_tags, (None,))[0] != h:
            if check_tags:
                first = fp8kv.verify_append(self.desc, self.K, self.V, self.k_scale, self.v_scale,
                                            self.k_new, self.v_new, self.token_pos,
                                            self.page_table, self.expected_tags, self.ctx_lens,
                                            self.pool_tags, abort=self.abort, prepare=True)
            else:
                first = fp8kv.append(self.desc, self.K, self.V, self.k_scale, self.v_scale,
                                     self.k_new, self.v_new, self.token_seq, self.token_pos,
                                     self.page_table, prepare=True)
            dec = fp8kv.decode_attention(
                self.desc, self.K, self.V, self.k_scale, self.v_scale, self.q, self.page_table,
                self.ctx_lens, abort=self.abort if check_tags else None, out=self.out,
                out_dtype=fp8kv.OUT_BF16, num_workers=self.num_workers, workspace=self.workspace,
                prepare=True)
            cache[check_tags] = (h, first, dec)
        return cache[check_tags]

    def prepared(self, check_tags: bool = True):
        """The default step's two prepared launches for the current stream:
        (fused check + append, or the plain append without the tracker;
        attention into the bf16 rows)."""
        _, first, dec = self._prepare(check_tags)
        return first, dec

    def step(self, check_tags=True, out_dtype=fp8kv.OUT_BF16, stream=None, fused=True):
        """One decode step: tag check + append (one launch when fused), then
        attention.  check_tags=False is the no-op tracker path.  The default
        form (fused, bf16 rows, current stream) runs prepared launches, with
        the tracker and without it alike."""
        if fused and out_dtype == fp8kv.OUT_BF16 and stream is None:
            _, first, dec = self._prepare(check_tags)
            first()
            return dec()
        if check_tags and fused:
            self.verify_append(stream)
        else:
            if check_tags:
                self.verify(stream)
            self.append(use_abort=check_tags, stream=stream)
        return self.decode(use_abort=check_tags, out_dtype=out_dtype, stream=stream)


@dataclasses.dataclass
class SpecStep:
    """A step that checks q_len new tokens per request at once (speculative
    verification) over a DeviceStep's cache: the request's context after the
    step is still L_b + 1, its newest q_len tokens (positions L_b+1-q_len ..
    L_b, fewer when the context is shorter) are appended by the step, and
    query i attends to the tokens up to its own.  Tag check and append are
    one launch (fp8kv_verify_append_q) when every context holds q_len tokens,
    else two."""
    base: DeviceStep
    q_len: int
    q: torch.Tensor             # [B][q_len][Hq][128]
    k_new: torch.Tensor         # [rows][Hkv][128]
    v_new: torch.Tensor
    token_seq: torch.Tensor
    token_pos: torch.Tensor
    workspace: torch.Tensor
    out: torch.Tensor
    k_new_q: Optional[torch.Tensor] = None   # [B][q_len][Hkv][128] for the fused launch
    v_new_q: Optional[torch.Tensor] = None
    first_pos: Optional[torch.Tensor] = None  # [B]: position of each first new token
    _prepared: Optional[tuple] = dataclasses.field(default=None, repr=False)

    def verify(self, stream=None):
        self.base.verify(stream)

    def append(self, use_abort=True, stream=None):
        s = self.base
        fp8kv.append(s.desc, s.K, s.V, s.k_scale, s.v_scale, self.k_new, self.v_new,
                     self.token_seq, self.token_pos, s.page_table,
                     abort=s.abort if use_abort else None, stream=stream)

    def decode(self, use_abort=True, out_dtype=fp8kv.OUT_BF16, stream=None):
        s = self.base
        out = self.out if out_dtype == fp8kv.OUT_BF16 else torch.empty(
            self.out.shape, dtype=torch.float32, device=self.out.device)
        return fp8kv.decode_attention_q(
            s.desc, s.K, s.V, s.k_scale, s.v_scale, self.q, s.page_table, s.ctx_lens,
            abort=s.abort if use_abort else None, out=out, out_dtype=out_dtype,
            num_workers=s.num_workers, workspace=self.workspace, stream=stream)

    def verify_append(self, stream=None):
        s = self.base
        fp8kv.verify_append_q(s.desc, s.K, s.V, s.k_scale, s.v_scale, self.k_new_q, self.v_new_q,
                              self.first_pos, s.page_table, s.expected_tags, s.ctx_lens,
                              s.pool_tags, abort=s.abort, stream=stream)

    def _prepare(self):
        """The fused check + append of the q_len tokens and the multi-query
        attention into the bf16 rows, prepared for the current stream (again
        when the stream or any tensor they hold changes)."""
        s = self.base
        h = (torch.cuda.current_stream().cuda_stream, s.num_workers,
             *map(id, (s.K, s.V, s.k_scale, s.v_scale, self.k_new_q, self.v_new_q,
                       self.first_pos, s.page_table, s.expected_tags, s.ctx_lens, s.pool_tags,
                       s.abort, self.q, self.out, self.workspace)))
        if self._prepared is None or self._prepared[0] != h:
            va = fp8kv.verify_append_q(s.desc, s.K, s.V, s.k_scale, s.v_scale, self.k_new_q,
                                       self.v_new_q, self.first_pos, s.page_table,
                                       s.expected_tags, s.ctx_lens, s.pool_tags,
                                       abort=s.abort, prepare=True)
            dec = fp8kv.decode_attention_q(
                s.desc, s.K, s.V, s.k_scale, s.v_scale, self.q, s.page_table, s.ctx_lens,
                abort=s.abort, out=self.out, out_dtype=fp8kv.OUT_BF16,
                num_workers=s.num_workers, workspace=self.workspace, prepare=True)
            self._prepared = (h, va, dec)
        return self._prepared

    def prepared(self):
        """The step's two prepared launches for the current stream: the fused
        check + append of the q_len tokens, and the multi-query attention."""
        if self.k_new_q is None:
            raise ValueError("a context shorter than q_len: the check and append are two launches")
        _, first, dec = self._prepare()
        return first, dec

    def step(self, check_tags=True, out_dtype=fp8kv.OUT_BF16, stream=None, fused=True):
        if (check_tags and fused and self.k_new_q is not None and out_dtype == fp8kv.OUT_BF16
                and stream is None):
            _, first, dec = self._prepare()
            first()
            return dec()
        if check_tags and fused and self.k_new_q is not None:
            self.verify_append(stream)
        else:
            if check_tags:
                self.verify(stream)
            self.append(use_abort=check_tags, stream=stream)
        return self.decode(use_abort=check_tags, out_dtype=out_dtype, stream=stream)


def build_spec(s: DeviceStep, q_len: int) -> SpecStep:
    """The q_len-token step over an already built (history-filled) DeviceStep."""
    w, dev = s.w, s.K.device
    t0 = np.maximum(w.ctx_lens - q_len, 0)
    t1 = w.ctx_lens
    kn = torch.cat([w.kv_tokens("k", b, int(t0[b]), int(t1[b]), "torch", dev)
                    for b in range(w.B)]).contiguous()
    vn = torch.cat([w.kv_tokens("v", b, int(t0[b]), int(t1[b]), "torch", dev)
                    for b in range(w.B)]).contiguous()
    seq = np.repeat(np.arange(w.B, dtype=np.int32), t1 - t0)
    pos = np.concatenate([np.arange(a, c, dtype=np.int32) for a, c in zip(t0, t1)])
    need = fp8kv.decode_workspace_size_q(s.desc, w.B, w.Hq, q_len, s.num_workers)
    if need == 0:
        raise ValueError(f"{w.Hq // w.Hkv} q-heads per kv-head x q_len {q_len} exceeds the "
                         "decode kernel's 32 columns")
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    full = bool((t1 - t0 == q_len).all())   # every request has q_len new tokens
    torch.cuda.synchronize()
    return SpecStep(base=s, q_len=q_len, q=w.q_bits_multi(q_len, "torch", dev), k_new=kn,
                    v_new=vn, token_seq=torch.from_numpy(seq).to(dev),
                    token_pos=torch.from_numpy(pos).to(dev), workspace=ws,
                    out=torch.empty((w.B, q_len, w.Hq, 128), dtype=torch.bfloat16, device=dev),
                    k_new_q=kn.view(w.B, q_len, w.Hkv, 128) if full else None,
                    v_new_q=vn.view(w.B, q_len, w.Hkv, 128) if full else None,
                    first_pos=torch.from_numpy(t0.astype(np.int32)).to(dev) if full else None)


def _bf16(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.bfloat16)


def kv_amax(w: Workload, which: str, device) -> np.ndarray:
    am = torch.zeros(w.Hkv, dtype=torch.float32, device=device)
    for b in range(w.B):
        n = int(w.ctx_before[b]) + 1
        first = 0 if w.first_of_prompt(b) else w.prompt(b)[1]   # a prompt counts once
        x = _bf16(w.kv_tokens(which, b, first, n, "torch", device, with_saturation=False))
        am = torch.maximum(am, x.float().abs().amax(dim=(0, 2)))
    return am.cpu().numpy()


def build(w: Workload, cache_dtype: int = fp8kv.E4M3, device="cuda", num_workers: int = 0,
          fill: bool = True, fill_chunk_tokens: int = 1 << 20) -> DeviceStep:
    d = fp8kv.desc(w.num_pages, w.Hkv, cache_dtype)
    K, V = fp8kv.new_cache(d, device)
    ksh = scales_from_amax(kv_amax(w, "k", device))
    vsh = scales_from_amax(kv_amax(w, "v", device))
    ks = torch.from_numpy(ksh).to(device)
    vs = torch.from_numpy(vsh).to(device)
    pt = torch.from_numpy(np.ascontiguousarray(w.page_table)).to(device)
    if fill:
        # history tokens 0..L_b-1 of every request, in chunks
        seqs, poss, ks_rows, vs_rows, tot = [], [], [], [], 0

        def flush():
            nonlocal seqs, poss, ks_rows, vs_rows, tot
            if not seqs:
                return
            fp8kv.append(d, K, V, ks, vs, torch.cat(ks_rows), torch.cat(vs_rows),
                         torch.cat(seqs), torch.cat(poss), pt)
            seqs, poss, ks_rows, vs_rows, tot = [], [], [], [], 0

        for b in range(w.B):
            L = int(w.ctx_before[b])
            # pages of a shared prompt are written once, through the first request
            first = 0 if (not w.prefix_shared or w.first_of_prompt(b)) else w.prompt(b)[1]
            for t0 in range(first, L, fill_chunk_tokens):
                t1 = min(L, t0 + fill_chunk_tokens)
                ks_rows.append(w.kv_tokens("k", b, t0, t1, "torch", device).contiguous())
                vs_rows.append(w.kv_tokens("v", b, t0, t1, "torch", device).contiguous())
                seqs.append(torch.full((t1 - t0,), b, dtype=torch.int32, device=device))
                poss.append(torch.arange(t0, t1, dtype=torch.int32, device=device))
                tot += t1 - t0
                if tot >= fill_chunk_tokens:
                    flush()
        flush()
    q = w.q_bits("torch", device).contiguous()
    k_new = w.new_kv_bits("k", "torch", device).contiguous()
    v_new = w.new_kv_bits("v", "torch", device).contiguous()
    # 0: the library's default grid (all workgroups resident, at most 24 per
    # (request, kv-head), 2/3 as many for two column tiles)
    nw = num_workers
    need = fp8kv.decode_workspace_size(d, w.B, w.Hq, nw)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=device)
    torch.cuda.synchronize()
    return DeviceStep(
        w=w, desc=d, K=K, V=V, k_scale=ks, v_scale=vs, k_scale_host=ksh, v_scale_host=vsh,
        q=q, k_new=k_new, v_new=v_new, page_table=pt,
        expected_tags=torch.from_numpy(w.expected_tags.view(np.int32).copy()).to(device),
        pool_tags=torch.from_numpy(w.pool_tags.view(np.int32).copy()).to(device),
        ctx_lens=torch.from_numpy(w.ctx_lens).to(device),
        token_seq=torch.arange(w.B, dtype=torch.int32, device=device),
        token_pos=torch.from_numpy(w.ctx_before.astype(np.int32)).to(device),
        abort=torch.zeros(w.B, dtype=torch.uint8, device=device),
        num_workers=nw, workspace=ws,
        out=torch.empty((w.B, w.Hq, 128), dtype=torch.bfloat16, device=device))
