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
