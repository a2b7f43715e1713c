"""A multi-step decode loop over the library: requests start from a prompt
already in the cache and generate one token per step for one layer.

Every step appends each live request's new token and attends over everything
cached so far.  A request takes a new page from the pool whenever its next
token starts one (every 16 steps), as a paged cache manager would.  This is
the setting of the integrity section's overhead study (prompts of 8,192
tokens, 1,000 generated tokens, a handful of concurrent requests) with the
model replaced by synthetic Q/K/V.

A model step runs `layers` layers; every layer has its own K/V pool addressed
by the same page table (page ids and their tags are per page, for all layers),
so the tag check runs once per step while append and attention run per layer.

tracker=True : after a page allocation the new pages' tags go to the device
               with the page table, in one copy (the loop mirrors the pool's
               tags from what the pool's alloc returns); the batched tag check
               runs before the first layer's append (fused check + append),
               later layers' appends and every attention honour the abort
               flags, and aborted requests are retired (their pages freed).
tracker=False: the no-op tracker: the same page allocation and page-table
               upload, plain appends and attention without abort flags.

Both modes copy B bytes back to the host after each step (the abort flags,
which stay zero without the tracker), standing in for the per-step read-back
of sampled tokens that any decode loop has; the flags ride along with it.

Inputs come from the counter-based generator of this package (streams keyed
by request), so a short loop can be replayed exactly by the oracle side.
Only the library's entry points do work on the device besides two small
torch operations per step (advancing the positions, reading the flags back)
and the page-table uploads; the entry points are called through launches
prepared once (fp8kv prepare=True), as a serving loop would.
"""
from __future__ import annotations

import time
from typing import List, Optional

import numpy as np
import torch

import decode_attention_paged_fp8kv_amd as fp8kv

from . import PAGE, D_HEAD, _T_K, _T_Q, _T_V, draw_bits, scales_from_amax, stream_key


def token_bits(seed: int, which: str, b: int, t0: int, t1: int, heads: int, backend="numpy",
               device=None):
    """BF16 bits of tokens [t0, t1) of request b: [t1-t0][heads][128].  Q of step s
    is token s of the Q stream; K/V token t is the t-th cached token."""
    tid = {"q": _T_Q, "k": _T_K, "v": _T_V}[which]
    key = stream_key(seed, tid, b)
    x = draw_bits(key, t0 * heads * D_HEAD, (t1 - t0) * heads * D_HEAD, backend, device)
    return x.reshape(t1 - t0, heads, D_HEAD)


class DecodeLoop:
    """State of B requests decoding together on one stream."""

    def __init__(self, batch: int, prompt_len: int, gen_len: int, num_q_heads: int = 64,
                 num_kv_heads: int = 8, tracker: bool = True, seed: int = 0,
                 cache_dtype: int = fp8kv.E4M3, step_sets: Optional[int] = None,
                 out_dtype: int = fp8kv.OUT_BF16, slack_pages: int = 16, layers: int = 1,
                 graph: bool = False, device="cuda"):
        """step_sets: how many distinct per-step Q/K/V sets to generate (None: one
        per step, exact inputs; a small number cycles them, enough for timing).
        graph: the launches of each step set (every layer's append and attention,
        and the check) are captured once in a HIP graph and each step replays
        one graph; host work (page allocation, table upload, read-back of the
        abort flags) stays outside."""
        assert num_q_heads % num_kv_heads == 0
        self.B, self.P, self.T = batch, prompt_len, gen_len
        self.Hq, self.Hkv = num_q_heads, num_kv_heads
        self.tracker, self.seed, self.dev = tracker, seed, device
        self.layers = layers
        self.out_dtype = out_dtype
        self.max_pages = -(-(prompt_len + gen_len) // PAGE)
        self.num_pages = batch * self.max_pages + slack_pages
        self.desc = fp8kv.desc(self.num_pages, num_kv_heads, cache_dtype)

        # pool with a seeded first-in-first-out order of free pages
        self.pool = fp8kv.Pool(self.num_pages, seed=seed)
        ids, _ = self.pool.alloc(self.num_pages)
        self.pool.free(np.random.default_rng(seed).permutation(ids))

        # per-step inputs, generated on the device before any step runs
        S = gen_len if step_sets is None else min(step_sets, gen_len)
        self.step_sets = S

        def per_step(which, heads, first_token):
            rows = [token_bits(seed, which, b, first_token, first_token + S, heads, "torch", device)
                    for b in range(batch)]
            return torch.stack(rows, 1).contiguous()      # [S][B][heads][128] int16

        self.q_steps = per_step("q", num_q_heads, 0)
        self.k_steps = per_step("k", num_kv_heads, prompt_len)
        self.v_steps = per_step("v", num_kv_heads, prompt_len)

        # scales: amax over every value the run will store (prompt and generated)
        def amax(which, steps):
            m = torch.zeros(num_kv_heads, dtype=torch.float32, device=device)
            for b in range(batch):
                x = token_bits(seed, which, b, 0, prompt_len, num_kv_heads, "torch", device)
                m = torch.maximum(m, x.view(torch.bfloat16).float().abs().amax(dim=(0, 2)))
            return torch.maximum(m, steps.view(torch.bfloat16).float().abs().amax(dim=(0, 1, 3)))
        self.k_scale = torch.from_numpy(scales_from_amax(amax("k", self.k_steps).cpu().numpy())).to(device)
        self.v_scale = torch.from_numpy(scales_from_amax(amax("v", self.v_steps).cpu().numpy())).to(device)

        eb = 1 if cache_dtype == fp8kv.E4M3 else 2
        tile = PAGE * D_HEAD * eb

        def pool_bytes():
            x = torch.zeros(self.num_pages * num_kv_heads * tile, dtype=torch.uint8, device=device)
            return x.view(torch.int16) if cache_dtype == fp8kv.BF16 else x
        # one K and one V pool per layer (the layers' inputs are the same streams)
        self.Ks = [pool_bytes() for _ in range(layers)]
        self.Vs = [pool_bytes() for _ in range(layers)]
        self.K, self.V = self.Ks[0], self.Vs[0]

        # page table, expected tags and the pool's tags in one buffer, so that
        # one upload carries all three after an allocation (a second copy for
        # the tags, as fp8kv_pool_sync makes, would put one more transfer
        # ahead of that step's kernels): a pinned host mirror and its device
        # copy, each region starting on a 256-byte boundary
        def up(n):
            return -(-n // 64) * 64
        n_tab = batch * self.max_pages
        o_et, o_tags = up(n_tab), 2 * up(n_tab)
        self.meta_host = torch.zeros(o_tags + up(self.num_pages), dtype=torch.int32).pin_memory()
        self.meta = torch.empty_like(self.meta_host, device=device)

        def regions(t):
            return (t[:n_tab].view(batch, self.max_pages),
                    t[o_et:o_et + n_tab].view(batch, self.max_pages),
                    t[o_tags:o_tags + self.num_pages])
        self.pt_host, self.et_host, self.tags_host = regions(self.meta_host)
        self.page_table, self.expected, self.tags = regions(self.meta)
        self.pt_host.fill_(-1)
        # numpy views of the host regions for the per-step writes (a torch
        # index assignment costs microseconds of host time)
        self._pt_np, self._et_np, self._tags_np = (x.numpy() for x in regions(self.meta_host))
        self._meta_bytes = {True: self.meta, False: self.meta[:n_tab]}
        self._meta_src = {True: self.meta_host, False: self.meta_host[:n_tab]}
        self.lens = torch.empty((2, batch), dtype=torch.int32, device=device)  # new_pos; ctx_lens
        self.abort = torch.zeros(batch, dtype=torch.uint8, device=device)
        self.abort_host = torch.zeros(batch, dtype=torch.uint8).pin_memory()
        # the flags as bytes, compared with the flags of the requests already
        # retired (a byte compare; numpy's any() costs microseconds per step)
        self._flag_bytes = memoryview(self.abort_host.numpy())
        self.out = torch.empty((batch, num_q_heads, D_HEAD), device=device,
                               dtype=torch.bfloat16 if out_dtype == fp8kv.OUT_BF16 else torch.float32)
        self.token_seq = torch.arange(batch, dtype=torch.int32, device=device)
        self.workspace = torch.empty(max(1, fp8kv.decode_workspace_size(
            self.desc, batch, num_q_heads, 0)), dtype=torch.uint8, device=device)
        self.pages: List[List[int]] = [[] for _ in range(batch)]
        self._fill_prompt()
        self.reset()
        self._launches = [self._prepare(i) for i in range(S)]
        self.graph = graph
        self._graphs = [self._capture(i) for i in range(S)] if graph else None

    # ------------------------------------------------------------------ setup
    def _take_pages(self, b: int, n: int):
        ids, tags = self.pool.alloc(n)
        k = len(self.pages[b])
        self._pt_np[b, k:k + n] = ids
        if self.tracker:       # the request remembers the tags; the pool's go up too
            self._et_np[b, k:k + n] = tags.view(np.int32)
            self._tags_np[ids] = tags.view(np.int32)
        self.pages[b].extend(ids.tolist())

    def _grow(self):
        """One new page for each live request, in one pool call and a few
        vectorized writes (the host work of an allocation step)."""
        rows = self._live_rows
        if rows.size == 0:
            return
        ids, tags = self.pool.alloc(rows.size)
        cols = np.array([len(self.pages[b]) for b in rows.tolist()])
        self._pt_np[rows, cols] = ids
        if self.tracker:
            t = tags.view(np.int32)
            self._et_np[rows, cols] = t
            self._tags_np[ids] = t
        for b, i in zip(rows.tolist(), ids.tolist()):
            self.pages[b].append(i)

    def _fill_prompt(self):
        n = -(-self.P // PAGE)
        for b in range(self.B):
            self._take_pages(b, n)
        self.prompt_pages = [list(p) for p in self.pages]
        self.page_table.copy_(self.pt_host)
        kb = torch.cat([token_bits(self.seed, "k", b, 0, self.P, self.Hkv, "torch", self.dev)
                        for b in range(self.B)])
        vb = torch.cat([token_bits(self.seed, "v", b, 0, self.P, self.Hkv, "torch", self.dev)
                        for b in range(self.B)])
        seq = torch.arange(self.B, dtype=torch.int32, device=self.dev).repeat_interleave(self.P)
        pos = torch.arange(self.P, dtype=torch.int32, device=self.dev).repeat(self.B)
        for K, V in zip(self.Ks, self.Vs):
            fp8kv.append(self.desc, K, V, self.k_scale, self.v_scale, kb, vb, seq, pos,
                         self.page_table)
        torch.cuda.synchronize()

    def reset(self):
        """Back to the state right after the prompt: generated pages returned.
        Not after an abort (a retired request's prompt pages are gone)."""
        if not all(getattr(self, "live", [True])) or getattr(self, "reclaimed", None):
            raise RuntimeError("reset after an abort or a reclaimed page: build a new loop")
        for b in range(self.B):
            extra = self.pages[b][len(self.prompt_pages[b]):]
            if extra:
                self.pool.free(extra)
            self.pages[b] = list(self.prompt_pages[b])
            self.pt_host[b, len(self.pages[b]):] = -1
        self.tags_host.copy_(torch.from_numpy(self.pool.tags().view(np.int32)))
        self.meta.copy_(self.meta_host)
        self.lens[0].fill_(self.P)
        self.lens[1].fill_(self.P + 1)
        self.abort.zero_()
        self.live = [True] * self.B
        self._live_rows = np.arange(self.B)
        self._retired_flags = bytes(self.B)
        self.reclaimed = set()
        self.step_index = 0
        torch.cuda.synchronize()

    def _prepare(self, i: int):
        """The step's launches for input set i, checked and marshalled once."""
        q, kn, vn = self.q_steps[i], self.k_steps[i], self.v_steps[i]
        ab = self.abort if self.tracker else None
        calls = []
        for layer, (K, V) in enumerate(zip(self.Ks, self.Vs)):
            if self.tracker and layer == 0:
                calls.append(fp8kv.verify_append(
                    self.desc, K, V, self.k_scale, self.v_scale, kn, vn, self.lens[0],
                    self.page_table, self.expected, self.lens[1], self.tags, abort=self.abort,
                    prepare=True))
            else:
                calls.append(fp8kv.append(
                    self.desc, K, V, self.k_scale, self.v_scale, kn, vn, self.token_seq,
                    self.lens[0], self.page_table, abort=ab, prepare=True))
            calls.append(fp8kv.decode_attention(
                self.desc, K, V, self.k_scale, self.v_scale, q, self.page_table, self.lens[1],
                abort=ab, out=self.out, out_dtype=self.out_dtype, workspace=self.workspace,
                prepare=True))
        return calls

    def _capture(self, i: int):
        """Step set i's launches recorded in a HIP graph.  The launches are
        marshalled inside the capture, so they name the capturing stream; the
        graph holds their pointers, whose contents (page table, lengths, flags)
        each replay reads afresh."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for launch in self._prepare(i):
                launch()
        torch.cuda.synchronize()
        return g

    # ------------------------------------------------------------------ step
    def step(self) -> float:
        """One decode step for all live requests; returns its wall time in seconds
        (host work, launches and the device work, synchronized at the end)."""
        t0 = time.perf_counter()
        s = self.step_index
        pos = self.P + s
        if pos % PAGE == 0:                       # the new token opens a page
            self._grow()
            # one copy: the page table, with the tracker also the expected
            # tags and the new pages' tags
            self._meta_bytes[self.tracker].copy_(self._meta_src[self.tracker], non_blocking=True)
        if self._graphs is not None:
            self._graphs[s % self.step_sets].replay()
        else:
            for launch in self._launches[s % self.step_sets]:
                launch()
        self.abort_host.copy_(self.abort, non_blocking=True)
        self.lens.add_(1)
        torch.cuda.synchronize()
        if self.tracker and self._flag_bytes.tobytes() != self._retired_flags:
            self._retire(np.flatnonzero(self.abort_host.numpy()))
        self.step_index += 1
        return time.perf_counter() - t0

    def _retire(self, rows):
        """Fail closed: an aborted request stops; its pages go back to the pool
        and from the next step on it neither appends nor reads anything."""
        rows = [int(b) for b in rows if self.live[int(b)]]
        if not rows:
            return          # already retired: their flags stay set, nothing to do
        for b in rows:
            self.live[b] = False
            self._retired_flags = bytes(0 if lv else 1 for lv in self.live)
            self._live_rows = np.flatnonzero(self.live)
            self.pool.free([p for p in self.pages[b] if p not in self.reclaimed])
            self.pages[b] = []
            self.pt_host[b, :] = -1
        self.page_table.copy_(self.pt_host)
        dead = torch.tensor([b for b in range(self.B) if not self.live[b]], device=self.dev)
        self.lens[0, dead] = -(1 << 30)       # no position: nothing is appended
        self.lens[1, dead] = -(1 << 30) + 1   # stays negative: no pages are read

    def reclaim(self, b: int, page_index: int):
        """Give one of request b's pages to another holder behind its back: the
        pool frees it and hands it out again, which changes its tag; request b
        still maps it with the tag it remembers.  The new tag goes up with the
        tables, as after any allocation.  Request b no longer holds the page:
        retiring it leaves the page with its new holder."""
        pid = self.pages[b][page_index]
        self.pool.free([pid])
        ids, tags = self.pool.alloc(self.pool.num_free)   # first in, first out: pid last
        assert int(ids[-1]) == pid
        self._tags_np[ids] = tags.view(np.int32)
        self.pool.free(ids[:-1])
        self.reclaimed.add(pid)
        self.meta.copy_(self.meta_host)

    def corrupt_expected(self, b: int, page_index: int):
        """Make request b remember a wrong tag for one of its pages (the view a
        request has after its page was reclaimed behind its back)."""
        self.et_host[b, page_index] = self.et_host[b, page_index] ^ 1
        self.expected.copy_(self.et_host)

    def run(self, steps: Optional[int] = None) -> np.ndarray:
        steps = self.T if steps is None else steps
        return np.array([self.step() for _ in range(steps)])

    def close(self):
        self.pool.close()
