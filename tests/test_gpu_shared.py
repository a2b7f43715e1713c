"""GPU: two requests over a shared prefix (pages held by both, same tags).

Request A holds a 2-page prefix and its own last page; request B maps the
same prefix pages (pool share) and holds its own last page.  A decode step
(fused check + append, attention) must match the oracle over the same page
tables; after A is cancelled B still passes the check; once the prefix pages
are handed out again, B's old view aborts and the new owner passes.
"""
import numpy as np
import pytest
import torch

import oracle
from _helpers import SM_SCALE, check_outputs, unswizzle
from workloads import bf16_bits_to_f32, scales_from_amax
from workloads.decode_loop import token_bits

pytestmark = pytest.mark.gpu

SEED, HQ, HKV, NPAGES = 21, 8, 2, 16
PREFIX = 32                       # two full pages
LA, LB = 42, 37                   # tokens cached before the step (A, B)


def _tokens(which, b, n, heads=HKV):
    """Request b's tokens 0..n-1: the shared prefix stream, then its own."""
    pre = token_bits(SEED, which, 100, 0, PREFIX, heads)
    own = token_bits(SEED, which, b, PREFIX, n, heads)
    return np.concatenate([pre, own])


def test_shared_prefix_decode_and_isolation():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_paged_fp8kv_amd as fp8kv
    dev = "cuda"
    pool = fp8kv.Pool(NPAGES, seed=SEED)
    pre_ids, pre_tags = pool.alloc(2)
    a_tail, a_ttag = pool.alloc(1)
    b_tags = pool.share(pre_ids)
    b_tail, b_ttag = pool.alloc(1)
    pt = np.stack([np.r_[pre_ids, a_tail], np.r_[pre_ids, b_tail]]).astype(np.int32)
    et = np.stack([np.r_[pre_tags, a_ttag], np.r_[b_tags, b_ttag]]).astype(np.uint32)
    L = np.array([LA, LB], np.int32)

    toks = {w: [_tokens(w, b, int(L[b]) + 1) for b in range(2)] for w in ("k", "v")}
    scale = {w: scales_from_amax(np.maximum(*[np.abs(bf16_bits_to_f32(t)).max(axis=(0, 2))
                                              for t in toks[w]])) for w in ("k", "v")}

    d = fp8kv.desc(NPAGES, HKV)
    K, V = fp8kv.new_cache(d, dev)
    ks = torch.from_numpy(scale["k"]).to(dev)
    vs = torch.from_numpy(scale["v"]).to(dev)
    pt_d = torch.from_numpy(pt).to(dev)
    et_d = torch.from_numpy(et.view(np.int32)).to(dev)
    tags_d = torch.zeros(NPAGES, dtype=torch.int32, device=dev)
    pool.sync(tags_d)

    def dev_bits(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev)

    # history: the prefix once (through A's table), then each request's own tokens
    rows = [(0, 0, LA), (1, PREFIX, LB)]
    kb = np.concatenate([toks["k"][b][t0:t1] for b, t0, t1 in rows])
    vb = np.concatenate([toks["v"][b][t0:t1] for b, t0, t1 in rows])
    seq = np.concatenate([np.full(t1 - t0, b, np.int32) for b, t0, t1 in rows])
    pos = np.concatenate([np.arange(t0, t1, dtype=np.int32) for b, t0, t1 in rows])
    fp8kv.append(d, K, V, ks, vs, dev_bits(kb), dev_bits(vb), torch.from_numpy(seq).to(dev),
                 torch.from_numpy(pos).to(dev), pt_d)

    q = np.stack([token_bits(SEED, "q", b, 0, 1, HQ)[0] for b in range(2)])
    kn = np.stack([toks["k"][b][L[b]] for b in range(2)])
    vn = np.stack([toks["v"][b][L[b]] for b in range(2)])
    lens = torch.from_numpy(L).to(dev)
    ctx = torch.from_numpy(L + 1).to(dev)
    abort = torch.zeros(2, dtype=torch.uint8, device=dev)
    fp8kv.verify_append(d, K, V, ks, vs, dev_bits(kn), dev_bits(vn), lens, pt_d, et_d, ctx,
                        tags_d, abort=abort)
    out = fp8kv.decode_attention(d, K, V, ks, vs, dev_bits(q), pt_d, ctx, abort=abort,
                                 out_dtype=fp8kv.OUT_F32)
    torch.cuda.synchronize()
    assert abort.cpu().numpy().tolist() == [0, 0]

    # oracle: each request's full token list through its own table
    Ko, Vo = oracle.new_cache(NPAGES, HKV)
    for b in range(2):
        n = int(L[b]) + 1
        oracle.append(Ko, Vo, scale["k"], scale["v"], toks["k"][b], toks["v"][b],
                      np.full(n, b, np.int32), np.arange(n, dtype=np.int32), pt)
    used = np.unique(pt)
    assert (unswizzle(K.cpu().numpy(), HKV, 0, used, False) == Ko[used]).all()
    assert (unswizzle(V.cpu().numpy(), HKV, 0, used, True) == Vo[used]).all()
    ref, _ = oracle.attention(Ko, Vo, scale["k"], scale["v"], q, pt, L + 1, SM_SCALE)
    check_outputs(out.cpu().numpy(), None, ref)

    # A is cancelled: the prefix stays with B, whose check still passes
    pool.free(pt[0])
    pool.sync(tags_d)
    ab = fp8kv.verify_tags(pt_d[1:], et_d[1:], ctx[1:], tags_d)
    assert ab.cpu().numpy().tolist() == [0]
    # B releases everything; the prefix pages are reissued with new tags
    pool.free(pt[1])
    pool.alloc(pool.num_free - 4)
    c_ids, c_tags = pool.alloc(4)
    assert set(pre_ids.tolist()) <= set(c_ids.tolist())
    pool.sync(tags_d)
    pt2 = torch.from_numpy(np.stack([pt[1], c_ids[:3]]).astype(np.int32)).to(dev)
    et2 = torch.from_numpy(np.stack([et[1], c_tags[:3]]).view(np.int32)).to(dev)
    ab = fp8kv.verify_tags(pt2, et2, torch.tensor([LB + 1, 48], dtype=torch.int32, device=dev),
                           tags_d)
    assert ab.cpu().numpy().tolist() == [1, 0]
    pool.close()


def test_shared_prompt_workload_full_size():
    """64 requests continuing one 16,384-token prompt whose pages all of them map:
    abort flags clear, sampled (request, kv-head) pairs against the oracle (the
    prompt regenerated once per pair), and outputs bit-identical to the same
    requests holding private copies of the prompt (same values, lengths and
    work partition)."""
    import decode_attention_paged_fp8kv_amd as fp8kv
    import workloads
    from workloads import device
    outs = {}
    for shared in (True, False):
        w = workloads.shared_prefix(shared=shared)
        st = device.build(w)
        st.step(check_tags=True)
        outs[shared] = st.decode(True, out_dtype=fp8kv.OUT_F32)
        torch.cuda.synchronize()
        assert (st.abort.cpu().numpy() == 0).all()
        if shared:
            assert len(np.unique(w.page_table[:, :1024])) == 1024
            ws, sts = w, st
        else:
            del st
    assert torch.equal(outs[True], outs[False])
    w, st = ws, sts
    o32 = outs[True].cpu().numpy()
    q = w.q_bits()
    G = w.G
    for b, g in [(0, 0), (37, 5), (63, 7)]:
        n = int(w.ctx_lens[b])
        K, V = oracle.new_cache(w.num_pages, 1)
        sk, sv = st.k_scale_host[g:g + 1], st.v_scale_host[g:g + 1]
        oracle.append(K, V, sk, sv, w.kv_tokens_head("k", b, 0, n, g)[:, None, :],
                      w.kv_tokens_head("v", b, 0, n, g)[:, None, :], np.zeros(n, np.int32),
                      np.arange(n, dtype=np.int32), w.page_table[b:b + 1])
        ref, _ = oracle.attention(K, V, sk, sv, q[b:b + 1, g * G:(g + 1) * G], w.page_table[b:b + 1],
                                  w.ctx_lens[b:b + 1], SM_SCALE)
        err = check_outputs(o32[b, g * G:(g + 1) * G], None, ref[0])
        print(f"shared prompt b={b} g={g} ctx={n}: max abs err {err:.3e}")


# ---------------------------------------------------------------------------
# the shared-prompt call: the prompt's pages read once for the whole batch
# ---------------------------------------------------------------------------
def _shared_state(Hq, Hkv, cache_dtype=0, B=5, prefix=48, suffix=40, seed=6):
    import workloads
    from workloads import device
    w = workloads.shared_prefix(B=B, prefix_len=prefix, suffix_max=suffix, Hq=Hq, Hkv=Hkv,
                                seed=seed)
    st = device.build(w, cache_dtype=cache_dtype)
    st.step(check_tags=True)
    torch.cuda.synchronize()
    return w, st


def _shared_call(fp8kv, w, st, out_dtype, workers=0, ctx=None, abort=None, prefix=None,
                 groups=None, sm_scale=None):
    """The shared-prompt call: by default one group (the whole batch) on the
    workload's prompt; `groups` = (group_start, prefix_len) overrides it."""
    prefix = w.prefix_len if prefix is None else prefix
    gs, pl = groups if groups is not None else ([0, w.B], [prefix])
    out = fp8kv.decode_attention_shared(
        st.desc, st.K, st.V, st.k_scale, st.v_scale, st.q, st.page_table,
        st.ctx_lens if ctx is None else ctx, gs, pl, abort=abort, out_dtype=out_dtype,
        num_workers=workers, sm_scale=sm_scale)
    torch.cuda.synchronize()
    return (out.view(torch.int16) if out.dtype == torch.bfloat16 else out).cpu().numpy()


@pytest.mark.parametrize("Hq,Hkv,cd", [(8, 2, 0), (64, 8, 0), (4, 4, 0), (64, 2, 0), (8, 2, 1),
                                       (64, 8, 1)])
def test_shared_call_matches_oracle(Hq, Hkv, cd):
    import decode_attention_paged_fp8kv_amd as fp8kv
    from _helpers import oracle_state
    w, st = _shared_state(Hq, Hkv, cd)
    Ko, Vo = oracle_state(w, st.k_scale_host, st.v_scale_host, cd)
    ref, _ = oracle.attention(Ko, Vo, st.k_scale_host, st.v_scale_host, w.q_bits(), w.page_table,
                              w.ctx_lens, SM_SCALE, cache_dtype=cd)
    plain = st.decode(True, out_dtype=fp8kv.OUT_F32).cpu().numpy()
    for nw in (0, 8, 64):
        o32 = _shared_call(fp8kv, w, st, fp8kv.OUT_F32, nw)
        o16 = _shared_call(fp8kv, w, st, fp8kv.OUT_BF16, nw).view(np.uint16)
        err = check_outputs(o32, o16, ref)
        assert np.abs(o32 - plain).max() <= 1e-5
        print(f"shared call Hq={Hq} Hkv={Hkv} cache={cd} workers={nw}: max abs err {err:.3e}")


@pytest.mark.parametrize("sm_scale", [0.0, -0.3, 4.0])
@pytest.mark.parametrize("Hq,Hkv,cd", [(64, 8, 0), (64, 8, 1), (8, 1, 0)])
def test_shared_call_score_scales(Hq, Hkv, cd, sm_scale):
    """A zero, a negative and a large score scale through the prompt pass and
    the own-token decode (fused grid, bf16 cache's separate launches, 8
    columns) against the oracle."""
    import decode_attention_paged_fp8kv_amd as fp8kv
    from _helpers import oracle_state
    w, st = _shared_state(Hq, Hkv, cd)
    Ko, Vo = oracle_state(w, st.k_scale_host, st.v_scale_host, cd)
    ref, _ = oracle.attention(Ko, Vo, st.k_scale_host, st.v_scale_host, w.q_bits(), w.page_table,
                              w.ctx_lens, sm_scale, cache_dtype=cd)
    for nw in (0, 64):
        o32 = _shared_call(fp8kv, w, st, fp8kv.OUT_F32, nw, sm_scale=sm_scale)
        o16 = _shared_call(fp8kv, w, st, fp8kv.OUT_BF16, nw, sm_scale=sm_scale).view(np.uint16)
        err = check_outputs(o32, o16, ref)
        print(f"shared call sm_scale={sm_scale} Hq={Hq} cache={cd} workers={nw}: "
              f"max abs err {err:.3e}")


@pytest.mark.parametrize("cd", [0, 1])
def test_shared_call_edges(cd):
    """No prompt is the plain call (bitwise); aborted requests, contexts that
    stop inside the prompt and contexts longer than the table holds give +0
    rows, the others stay exact; bad prompt lengths are rejected before
    anything runs.  The e4m3 cache takes the one-grid path (prompt pass and
    own-token decode together), the bf16 cache the separate launches."""
    import decode_attention_paged_fp8kv_amd as fp8kv
    from _helpers import oracle_state
    w, st = _shared_state(8, 2, cd, B=6)
    plain = st.decode(True, out_dtype=fp8kv.OUT_F32).cpu().numpy()
    assert np.array_equal(_shared_call(fp8kv, w, st, fp8kv.OUT_F32, prefix=0), plain)
    ab = torch.tensor([0, 1, 0, 0, 0, 0], dtype=torch.uint8, device="cuda")
    ctx = w.ctx_lens.copy()
    ctx[2] = 16 * w.max_pages + 1    # longer than the table holds (fail closed)
    ctx[3] = w.prefix_len            # ends exactly at the end of the prompt
    ctx[4] = 20                      # ends inside the prompt
    o = _shared_call(fp8kv, w, st, fp8kv.OUT_F32, ctx=torch.from_numpy(ctx).cuda(), abort=ab)
    assert (o[[1, 2, 3, 4]] == 0).all()
    Ko, Vo = oracle_state(w, st.k_scale_host, st.v_scale_host, cd)
    ref, _ = oracle.attention(Ko, Vo, st.k_scale_host, st.v_scale_host, w.q_bits(), w.page_table,
                              w.ctx_lens, SM_SCALE, cache_dtype=cd)
    check_outputs(o[[0, 5]], None, ref[[0, 5]])
    assert fp8kv.decode_workspace_size_shared(st.desc, w.B, w.Hq, w.max_pages, [0, w.B], [8]) == 0
    for bad in (8, -16, 16 * (w.max_pages + 1)):
        with pytest.raises(fp8kv.Fp8kvError) as e:
            _shared_call(fp8kv, w, st, fp8kv.OUT_F32, prefix=bad)
        assert e.value.status == -1


def test_shared_call_full_size():
    """The 64-request, 16,384-token-prompt workload: sampled pairs against the
    oracle and every row against the plain call."""
    import decode_attention_paged_fp8kv_amd as fp8kv
    import workloads
    from workloads import device
    w = workloads.shared_prefix()
    st = device.build(w)
    st.step(check_tags=True)
    plain = st.decode(True, out_dtype=fp8kv.OUT_F32).cpu().numpy()
    o32 = _shared_call(fp8kv, w, st, fp8kv.OUT_F32)
    assert np.abs(o32 - plain).max() <= 1e-5
    q = w.q_bits()
    G = w.G
    for b, g in [(5, 1), (63, 6)]:
        n = int(w.ctx_lens[b])
        K, V = oracle.new_cache(w.num_pages, 1)
        sk, sv = st.k_scale_host[g:g + 1], st.v_scale_host[g:g + 1]
        oracle.append(K, V, sk, sv, w.kv_tokens_head("k", b, 0, n, g)[:, None, :],
                      w.kv_tokens_head("v", b, 0, n, g)[:, None, :], np.zeros(n, np.int32),
                      np.arange(n, dtype=np.int32), w.page_table[b:b + 1])
        ref, _ = oracle.attention(K, V, sk, sv, q[b:b + 1, g * G:(g + 1) * G], w.page_table[b:b + 1],
                                  w.ctx_lens[b:b + 1], SM_SCALE)
        err = check_outputs(o32[b, g * G:(g + 1) * G], None, ref[0])
        print(f"shared call full size b={b} g={g}: max abs err {err:.3e}")


@pytest.mark.parametrize("cd", [0, 1])
def test_shared_call_prompt_groups(cd):
    """Three prompts continued by groups of 5, 2 and 9 requests, then 4 requests
    without one, in a single call: every row against the oracle and the plain
    call; an empty group description is the plain call (bitwise); groups may
    skip requests and list prompts of 0 tokens; bad descriptions are rejected."""
    import decode_attention_paged_fp8kv_amd as fp8kv
    import workloads
    from workloads import device
    from _helpers import oracle_state
    w = workloads.shared_prompts([(5, 64), (2, 32), (9, 160)], plain=4, suffix_max=70, Hq=16, Hkv=4)
    st = device.build(w, cache_dtype=cd)
    st.step(check_tags=True)
    torch.cuda.synchronize()
    assert (st.abort.cpu().numpy() == 0).all()
    Ko, Vo = oracle_state(w, st.k_scale_host, st.v_scale_host, cd)
    ref, _ = oracle.attention(Ko, Vo, st.k_scale_host, st.v_scale_host, w.q_bits(), w.page_table,
                              w.ctx_lens, SM_SCALE, cache_dtype=cd)
    plain = st.decode(True, out_dtype=fp8kv.OUT_F32).cpu().numpy()
    groups = ([0, 5, 7, 16], [64, 32, 160])
    for nw in (0, 12):
        o32 = _shared_call(fp8kv, w, st, fp8kv.OUT_F32, nw, groups=groups)
        o16 = _shared_call(fp8kv, w, st, fp8kv.OUT_BF16, nw, groups=groups).view(np.uint16)
        err = check_outputs(o32, o16, ref)
        assert np.abs(o32 - plain).max() <= 1e-5
        print(f"3 prompt groups cache={cd} workers={nw}: max abs err {err:.3e}")
    assert np.array_equal(_shared_call(fp8kv, w, st, fp8kv.OUT_F32, groups=([0], [])), plain)
    # the middle group attended as usual (prompt of 0 tokens), the last one in part
    o = _shared_call(fp8kv, w, st, fp8kv.OUT_F32, groups=([0, 5, 7, 12], [64, 0, 160]))
    assert np.abs(o - plain).max() <= 1e-5
    check_outputs(o, None, ref)
    for gs, pl in (([0, 5, 3], [64, 32]), ([0, 5, 30], [64, 32]), ([0, 5], [24])):
        with pytest.raises(fp8kv.Fp8kvError) as e:
            _shared_call(fp8kv, w, st, fp8kv.OUT_F32, groups=(gs, pl))
        assert e.value.status == -1


@pytest.mark.parametrize("cd", [0, 1])
def test_shared_call_fails_closed(cd):
    """The prompt's pages are read through the group's first table, and each
    member's tag check covers its own table only: a member whose table lists
    other pages in the prompt range (valid ones, its check passes) gets +0
    rows; an aborted first member does not stop the others; a stale tag on a
    shared prompt page aborts exactly the members whose recorded tag it is."""
    import decode_attention_paged_fp8kv_amd as fp8kv
    from _helpers import oracle_state
    w, st = _shared_state(8, 2, cd, B=6)
    Ko, Vo = oracle_state(w, st.k_scale_host, st.v_scale_host, cd)
    ref, _ = oracle.attention(Ko, Vo, st.k_scale_host, st.v_scale_host, w.q_bits(), w.page_table,
                              w.ctx_lens, SM_SCALE, cache_dtype=cd)
    P0 = w.prefix_len // 16
    pt, et, tags = w.page_table.copy(), w.expected_tags.copy(), w.pool_tags.copy()
    # member 3 lists its own first page in place of the prompt's second one
    pt[3, 1], et[3, 1] = pt[3, P0], et[3, P0]
    pt_d = torch.from_numpy(pt).cuda()
    et_d = torch.from_numpy(et.view(np.int32)).cuda()
    ab = fp8kv.verify_tags(pt_d, et_d, st.ctx_lens, st.pool_tags)
    assert (ab.cpu().numpy() == 0).all()
    for nw in (0, 8):
        out = fp8kv.decode_attention_shared(st.desc, st.K, st.V, st.k_scale, st.v_scale, st.q,
                                            pt_d, st.ctx_lens, [0, w.B], [w.prefix_len],
                                            abort=ab, out_dtype=fp8kv.OUT_F32, num_workers=nw)
        o = out.cpu().numpy()
        assert (o[3].view(np.uint32) == 0).all()
        keep = [0, 1, 2, 4, 5]
        check_outputs(o[keep], None, ref[keep])
    # the group's first request aborted: the others are exact
    ab0 = torch.tensor([1, 0, 0, 0, 0, 0], dtype=torch.uint8, device="cuda")
    o = _shared_call(fp8kv, w, st, fp8kv.OUT_F32, abort=ab0)
    assert (o[0].view(np.uint32) == 0).all()
    check_outputs(o[1:], None, ref[1:])
    # a member recorded a stale tag for a shared prompt page: it alone aborts
    et2 = w.expected_tags.copy()
    et2[2, 0] ^= 0x10
    ab2 = fp8kv.verify_tags(st.page_table, torch.from_numpy(et2.view(np.int32)).cuda(),
                            st.ctx_lens, st.pool_tags)
    assert ab2.cpu().numpy().tolist() == [0, 0, 1, 0, 0, 0]
    o = _shared_call(fp8kv, w, st, fp8kv.OUT_F32, abort=ab2)
    assert (o[2].view(np.uint32) == 0).all()
    check_outputs(o[[0, 1, 3, 4, 5]], None, ref[[0, 1, 3, 4, 5]])
    # the shared page itself was handed out again: every member aborts
    tags[pt[0, 1]] += np.uint32(1)
    ab3 = fp8kv.verify_tags(st.page_table, st.expected_tags, st.ctx_lens,
                            torch.from_numpy(tags.view(np.int32)).cuda())
    assert (ab3.cpu().numpy() == 1).all()
    o = _shared_call(fp8kv, w, st, fp8kv.OUT_F32, abort=ab3)
    assert (o.view(np.uint32) == 0).all()
