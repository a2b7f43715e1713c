"""GPU: several new tokens per request checked in one step (speculative
verification) -- fp8kv_append of the q_len new tokens, then
fp8kv_decode_attention_q -- against the oracle's multi-query attention.

Query i of a request sees the cache up to its own new token.  Covered: the
(query, head) layouts G*q_len = 16, 12 and 5 columns (one 16-column MFMA
tile) and 24 and 32 columns and G = 32 (two tiles), both cache types,
histories whose new tokens cross page boundaries, several work partitions, an
aborted request, q_len = 1 against the single-query entry point (bitwise),
each row against a one-token decode over its own prefix, and the
G*q_len > 32 rejection.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from _helpers import SM_SCALE, check_outputs, unswizzle
from workloads import bf16_bits_to_f32, scales_from_amax
from workloads.decode_loop import token_bits

pytestmark = pytest.mark.gpu

SEED = 31


def _setup(fp8kv, hist, T, Hq, Hkv, seed=SEED, cache_dtype=0):
    """History of hist[b] tokens in the cache, the T new tokens appended by one
    fp8kv_append call; returns everything both sides need."""
    dev = "cuda"
    B = len(hist)
    ctx = np.array(hist, np.int32) + T
    n = [-(-int(c) // 16) for c in ctx]
    N = sum(n) + 5
    perm = np.random.default_rng(seed).permutation(N).astype(np.int32)
    pt = np.full((B, max(n)), -1, np.int32)
    k = 0
    for b in range(B):
        pt[b, :n[b]] = perm[k:k + n[b]]
        k += n[b]
    toks = {w: [token_bits(seed, w, b, 0, int(ctx[b]), Hkv) for b in range(B)] for w in "kv"}
    scale = {w: scales_from_amax(np.max([np.abs(bf16_bits_to_f32(t)).max(axis=(0, 2))
                                         for t in toks[w]], axis=0)) for w in "kv"}
    q = np.stack([token_bits(seed, "q", b, 0, T, Hq) for b in range(B)])   # [B][T][Hq][128]
    d = fp8kv.desc(N, Hkv, cache_dtype)
    K, V = fp8kv.new_cache(d, dev)
    st = dict(fp8kv=fp8kv, d=d, K=K, V=V, pt=pt, ctx=ctx, q=q, toks=toks, scale=scale, B=B, T=T,
              Hq=Hq, Hkv=Hkv, N=N, cd=cache_dtype,
              ks=torch.from_numpy(scale["k"]).to(dev), vs=torch.from_numpy(scale["v"]).to(dev),
              pt_d=torch.from_numpy(pt).to(dev), ctx_d=torch.from_numpy(ctx).to(dev),
              q_d=torch.from_numpy(q.view(np.int16)).to(dev))

    def append(rows):   # rows: (b, t0, t1)
        rows = [r for r in rows if r[2] > r[1]]
        if not rows:
            return
        kb = np.concatenate([toks["k"][b][t0:t1] for b, t0, t1 in rows])
        vb = np.concatenate([toks["v"][b][t0:t1] for b, t0, t1 in rows])
        seq = np.concatenate([np.full(t1 - t0, b, np.int32) for b, t0, t1 in rows])
        pos = np.concatenate([np.arange(t0, t1, dtype=np.int32) for b, t0, t1 in rows])
        fp8kv.append(d, K, V, st["ks"], st["vs"],
                     torch.from_numpy(np.ascontiguousarray(kb).view(np.int16)).to(dev),
                     torch.from_numpy(np.ascontiguousarray(vb).view(np.int16)).to(dev),
                     torch.from_numpy(seq).to(dev), torch.from_numpy(pos).to(dev), st["pt_d"])
    append([(b, 0, hist[b]) for b in range(B)])                 # the cached history
    append([(b, hist[b], hist[b] + T) for b in range(B)])       # the step's q_len new tokens
    return st


def _oracle(st, abort=None, sm_scale=SM_SCALE):
    Ko, Vo = oracle.new_cache(st["N"], st["Hkv"], st["cd"])
    for b in range(st["B"]):
        c = int(st["ctx"][b])
        if abort is not None and abort[b]:
            c -= st["T"]                         # the aborted request's new tokens: not written
        if c > 0:
            oracle.append(Ko, Vo, st["scale"]["k"], st["scale"]["v"], st["toks"]["k"][b][:c],
                          st["toks"]["v"][b][:c], np.full(c, b, np.int32),
                          np.arange(c, dtype=np.int32), st["pt"], cache_dtype=st["cd"])
    ref, _ = oracle.attention_multi(Ko, Vo, st["scale"]["k"], st["scale"]["v"], st["q"], st["pt"],
                                    st["ctx"], sm_scale, abort=abort, cache_dtype=st["cd"])
    return Ko, Vo, ref


def _run(st, out_dtype, num_workers=0, abort=None, sm_scale=None):
    f = st["fp8kv"]
    ab = None if abort is None else torch.from_numpy(abort).cuda()
    out = f.decode_attention_q(st["d"], st["K"], st["V"], st["ks"], st["vs"], st["q_d"],
                               st["pt_d"], st["ctx_d"], abort=ab, out_dtype=out_dtype,
                               num_workers=num_workers, sm_scale=sm_scale)
    torch.cuda.synchronize()
    return (out.view(torch.int16) if out.dtype == torch.bfloat16 else out).cpu().numpy()


@pytest.mark.parametrize("sm_scale", [0.0, -0.3, 4.0])
@pytest.mark.parametrize("Hq,Hkv,T", [(64, 8, 1), (64, 8, 4)])
@pytest.mark.parametrize("cd", [0, 1])
def test_score_scale_zero_negative_and_large(Hq, Hkv, T, cd, sm_scale):
    """The kernels fold the score scale's sign into Q and keep a zero scale
    just above 0: sm_scale 0 weighs every visible token alike, a negative
    one favours the lowest scores, a large one is nearly one-hot.  One tile
    (8 columns) and two tiles (32 columns), both cache types."""
    import decode_attention_paged_fp8kv_amd as fp8kv
    st = _setup(fp8kv, [1, 14, 47, 100, 300], T, Hq, Hkv, cache_dtype=cd)
    _, _, ref = _oracle(st, sm_scale=sm_scale)
    for nw in (0, 64):
        o32 = _run(st, fp8kv.OUT_F32, nw, sm_scale=sm_scale)
        o16 = _run(st, fp8kv.OUT_BF16, nw, sm_scale=sm_scale).view(np.uint16)
        err = check_outputs(o32, o16, ref)
        print(f"sm_scale={sm_scale} T={T} cache={cd} workers={nw}: max abs err {err:.3e}")


@pytest.mark.parametrize("Hq,Hkv,T", [(64, 8, 2), (8, 2, 3), (4, 4, 5),
                                      (64, 8, 3), (64, 8, 4), (64, 2, 1), (32, 2, 2), (16, 4, 5)])
@pytest.mark.parametrize("hist", [[1, 14, 15, 30, 47, 100], [0, 13, 16, 31]])
def test_multi_query_matches_oracle(Hq, Hkv, T, hist):
    import decode_attention_paged_fp8kv_amd as fp8kv
    st = _setup(fp8kv, hist, T, Hq, Hkv)
    Ko, Vo, ref = _oracle(st)
    used = np.unique(st["pt"][st["pt"] >= 0])
    assert (unswizzle(st["K"].cpu().numpy(), Hkv, 0, used, False) == Ko[used]).all()
    assert (unswizzle(st["V"].cpu().numpy(), Hkv, 0, used, True) == Vo[used]).all()
    for nw in (0, 8, 64):
        o32 = _run(st, fp8kv.OUT_F32, nw)
        o16 = _run(st, fp8kv.OUT_BF16, nw).view(np.uint16)
        err = check_outputs(o32, o16, ref)
        print(f"Hq={Hq} Hkv={Hkv} T={T} hist={hist} workers={nw}: max abs err {err:.3e}")


def test_one_query_equals_the_single_query_entry_point():
    import decode_attention_paged_fp8kv_amd as fp8kv
    st = _setup(fp8kv, [5, 40, 77], 1, 64, 8)
    a = _run(st, fp8kv.OUT_F32)
    b = fp8kv.decode_attention(st["d"], st["K"], st["V"], st["ks"], st["vs"], st["q_d"][:, 0],
                               st["pt_d"], st["ctx_d"], out_dtype=fp8kv.OUT_F32)
    torch.cuda.synchronize()
    assert np.array_equal(a[:, 0], b.cpu().numpy())


def test_rows_equal_one_token_decodes_over_their_prefix():
    import decode_attention_paged_fp8kv_amd as fp8kv
    T = 2
    st = _setup(fp8kv, [9, 31, 64, 200], T, 64, 8)
    multi = _run(st, fp8kv.OUT_F32)
    for i in range(T):
        ctx_i = torch.from_numpy(st["ctx"] - (T - 1 - i)).cuda()
        one = fp8kv.decode_attention(st["d"], st["K"], st["V"], st["ks"], st["vs"],
                                     st["q_d"][:, i].contiguous(), st["pt_d"], ctx_i,
                                     out_dtype=fp8kv.OUT_F32)
        torch.cuda.synchronize()
        assert np.abs(one.cpu().numpy() - multi[:, i]).max() <= 1e-5, i


def test_aborted_request_gives_zero_rows():
    import decode_attention_paged_fp8kv_amd as fp8kv
    st = _setup(fp8kv, [20, 33, 50], 2, 8, 2)
    ab = np.array([0, 1, 0], np.uint8)
    o = _run(st, fp8kv.OUT_F32, abort=ab)
    _, _, ref = _oracle(st)
    assert (o[1] == 0).all()
    check_outputs(o[[0, 2]], None, ref[[0, 2]])


@pytest.mark.parametrize("Hq,Hkv,T", [(64, 8, 4), (64, 8, 2)])
def test_bf16_cache(Hq, Hkv, T):
    import decode_attention_paged_fp8kv_amd as fp8kv
    st = _setup(fp8kv, [5, 16, 33, 70], T, Hq, Hkv, cache_dtype=fp8kv.BF16)
    _, _, ref = _oracle(st)
    for nw in (0, 16):
        err = check_outputs(_run(st, fp8kv.OUT_F32, nw), _run(st, fp8kv.OUT_BF16, nw).view(np.uint16),
                            ref)
        print(f"bf16 cache Hq={Hq} Hkv={Hkv} T={T} workers={nw}: max abs err {err:.3e}")


def test_too_many_columns_is_rejected():
    import decode_attention_paged_fp8kv_amd as fp8kv
    st = _setup(fp8kv, [3], 5, 64, 8)              # G = 8, q_len = 5: 40 columns
    assert fp8kv.decode_workspace_size_q(st["d"], 1, 64, 5) == 0
    with pytest.raises(fp8kv.Fp8kvError) as e:
        _run(st, fp8kv.OUT_F32)
    assert e.value.status == -2


@pytest.mark.parametrize("T", [2, 4])
def test_ragged_64_full_size(T):
    """The 64-request ragged workload with q_len 2 and 4 (G*q_len = 16 and 32
    columns), in the launch configuration the speculative-verification study
    times: sampled (request, kv-head) pairs against the oracle, and the newest
    query's rows against the one-token decode over the same cache."""
    import decode_attention_paged_fp8kv_amd as fp8kv
    import workloads
    from workloads import device
    w = workloads.make(3)
    st = device.build(w)
    sp = device.build_spec(st, T)
    o16 = sp.step(True).view(torch.int16)
    torch.cuda.synchronize()
    o16 = o16.cpu().numpy().view(np.uint16)
    o32 = sp.decode(out_dtype=fp8kv.OUT_F32)
    one = st.decode(out_dtype=fp8kv.OUT_F32)
    torch.cuda.synchronize()
    o32, one = o32.cpu().numpy(), one.cpu().numpy()
    assert (st.abort.cpu().numpy() == 0).all()
    assert np.abs(o32[:, -1] - one).max() <= 1e-6
    q = w.q_bits_multi(T)
    assert np.array_equal(q[:, -1], w.q_bits())
    G, L = w.G, w.ctx_lens
    for b, g in [(int(L.argmax()), 0), (int(L.argmin()), 7), (11, 4)]:
        n = int(L[b])
        K, V = oracle.new_cache(w.num_pages, 1)
        sk, sv = st.k_scale_host[g:g + 1], st.v_scale_host[g:g + 1]
        oracle.append(K, V, sk, sv, w.kv_tokens_head("k", b, 0, n, g)[:, None, :],
                      w.kv_tokens_head("v", b, 0, n, g)[:, None, :], np.zeros(n, np.int32),
                      np.arange(n, dtype=np.int32), w.page_table[b:b + 1])
        ref, _ = oracle.attention_multi(K, V, sk, sv, q[b:b + 1, :, g * G:(g + 1) * G],
                                        w.page_table[b:b + 1], L[b:b + 1], SM_SCALE)
        cols = slice(g * G, (g + 1) * G)
        err = check_outputs(o32[b, :, cols], o16[b, :, cols], ref[0])
        print(f"ragged q_len={T} b={b} g={g} ctx={n} max abs err {err:.3e}")


@pytest.mark.parametrize("Hq,Hkv,T", [(64, 8, 1), (64, 8, 2), (64, 8, 4), (8, 2, 5), (16, 16, 2)])
def test_fused_check_and_multi_token_append(Hq, Hkv, T):
    """fp8kv_verify_append_q (one launch) writes the same cache bytes and abort
    flags as the tag check followed by the gated append of the T tokens, with
    stale entries in some requests (their tokens are not written)."""
    import decode_attention_paged_fp8kv_amd as fp8kv
    hist = [20, 33, 50, 7, 100, 64]
    outs = []
    for fused in (True, False):
        st = _setup(fp8kv, hist, T, Hq, Hkv)
        B = st["B"]
        tags = np.random.default_rng(5).integers(0, 2 ** 32, st["N"], dtype=np.uint64).astype(np.uint32)
        et = np.where(st["pt"] >= 0, tags[np.clip(st["pt"], 0, None)], 0).astype(np.uint32)
        tags[st["pt"][1, 0]] += np.uint32(1)            # request 1 holds a stale entry
        tags[st["pt"][4, -1 if st["pt"][4, -1] >= 0 else 0]] += np.uint32(1)
        pos = (st["ctx"] - T).astype(np.int32)
        kb = np.stack([st["toks"]["k"][b][pos[b]:pos[b] + T] for b in range(B)])
        vb = np.stack([st["toks"]["v"][b][pos[b]:pos[b] + T] for b in range(B)])
        K, V = fp8kv.new_cache(st["d"], "cuda")       # fresh pools: only this step's writes
        dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
        args = (st["d"], K, V, st["ks"], st["vs"])
        et_d, tags_d = dev(et.view(np.int32)), dev(tags.view(np.int32))
        if fused:
            ab = fp8kv.verify_append_q(*args, dev(kb.view(np.int16)), dev(vb.view(np.int16)),
                                       dev(pos), st["pt_d"], et_d, st["ctx_d"], tags_d)
        else:
            ab = fp8kv.verify_tags(st["pt_d"], et_d, st["ctx_d"], tags_d)
            seq = np.repeat(np.arange(B, dtype=np.int32), T)
            p = (pos[:, None] + np.arange(T, dtype=np.int32)[None]).ravel().astype(np.int32)
            fp8kv.append(*args, dev(kb.reshape(B * T, Hkv, 128).view(np.int16)),
                         dev(vb.reshape(B * T, Hkv, 128).view(np.int16)), dev(seq), dev(p),
                         st["pt_d"], abort=ab)
        torch.cuda.synchronize()
        outs.append((ab.cpu().numpy(), K.cpu().numpy(), V.cpu().numpy()))
    (a0, k0, v0), (a1, k1, v1) = outs
    assert list(a0) == [0, 1, 0, 0, 1, 0] and np.array_equal(a0, a1)
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    assert k0.any()


def test_queries_with_nothing_to_see_give_zero_rows():
    """A context shorter than q_len (the caller's lengths): the first queries see
    no token and give +0 rows, the rest attend to their prefix, as the oracle."""
    import decode_attention_paged_fp8kv_amd as fp8kv
    T = 4                                               # G 8 x q_len 4: all 32 columns
    st = _setup(fp8kv, [0, 4, 40], T, 64, 8)
    ctx = np.array([2, 8, 3], np.int32)                 # shorter than written: allowed
    st["ctx_d"] = torch.from_numpy(ctx).cuda()
    st["ctx"] = ctx
    Ko, Vo = oracle.new_cache(st["N"], st["Hkv"])
    for b in range(st["B"]):
        c = int(ctx[b])
        oracle.append(Ko, Vo, st["scale"]["k"], st["scale"]["v"], st["toks"]["k"][b][:c],
                      st["toks"]["v"][b][:c], np.full(c, b, np.int32), np.arange(c, dtype=np.int32),
                      st["pt"])
    ref, _ = oracle.attention_multi(Ko, Vo, st["scale"]["k"], st["scale"]["v"], st["q"], st["pt"], ctx,
                                    SM_SCALE)
    for nw in (0, 8):
        o = _run(st, fp8kv.OUT_F32, nw)
        assert (o[0, :2] == 0).all() and (o[2, :1] == 0).all()
        assert np.abs(o[0, 2:]).max() > 0 and np.abs(o[2, 1:]).max() > 0
        check_outputs(o, None, ref)
