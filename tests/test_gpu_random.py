"""GPU: seeded random cases against the oracle.  Each case draws its own
shape (kv-heads, q-heads per kv-head), lengths (empty, one token, page edges,
a few hundred tokens), worker count, cache type, stale entries, number of
queries per request, and, for the shared-prompt call, its prompt groups.
Cache bytes of the plain step are compared bit for bit; attention outputs to
the oracle's tolerance (f32 rows, and bf16 rows as their round-to-nearest-even).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import SM_SCALE, check_outputs, oracle_state, unswizzle

pytestmark = pytest.mark.gpu

PLAIN_CASES = 96
SHARED_CASES = 48


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _lengths(rng, B):
    edge = [0, 1, 15, 16, 17, 31, 32, 33, 255, 256]
    L = rng.integers(0, 700, B)
    for i in rng.choice(B, min(B, 3), replace=False):
        L[i] = rng.choice(edge)
    return L.astype(np.int32)


def _stale(rng, w, n):
    """Hand n requests' pages out again (their tag moves on): the check must
    abort them; a request sharing none of those pages is untouched."""
    live = [b for b in range(w.B) if w.n_pages[b] > 0]
    for b in rng.choice(live, min(n, len(live)), replace=False):
        i = int(rng.integers(0, w.n_pages[b]))
        w.pool_tags[w.page_table[b, i]] += np.uint32(1)
    for b in range(w.B):
        k = w.n_pages[b]
        w.stale[b, :k] = w.expected_tags[b, :k] != w.pool_tags[w.page_table[b, :k]]


@pytest.mark.parametrize("case", range(PLAIN_CASES))
def test_random_plain_and_multi_query(case):
    import decode_attention_paged_fp8kv_amd as fp8kv
    from workloads import device
    rng = np.random.default_rng(5000 + case)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    B = int(rng.integers(1, 13))
    cd = int(rng.integers(0, 2))
    workers = int(rng.choice([0, 4, 16, 64, 512]))
    w = workloads.custom(f"random{case}", _lengths(rng, B), Hq=G * Hkv, Hkv=Hkv,
                         seed=6000 + case, pool_slack=int(rng.integers(0, 4)))
    if B >= 3 and rng.random() < 0.5:     # some requests abort, the others run on
        _stale(rng, w, int(rng.integers(1, 3)))
    st = device.build(w, cache_dtype=cd, num_workers=workers)
    out16 = st.step(check_tags=True)
    out32 = st.decode(out_dtype=fp8kv.OUT_F32)
    ab = _host(st.abort)
    exp_ab = oracle.verify(w.page_table, w.expected_tags, w.ctx_lens, w.pool_tags)
    assert (ab == exp_ab).all()
    Ko, Vo = oracle_state(w, st.k_scale_host, st.v_scale_host, cd, abort=exp_ab)
    pages = np.arange(w.num_pages)
    assert (unswizzle(_host(st.K), w.Hkv, cd, pages, False) == Ko).all()
    assert (unswizzle(_host(st.V), w.Hkv, cd, pages, True) == Vo).all()
    ref, _ = oracle.attention(Ko, Vo, st.k_scale_host, st.v_scale_host, w.q_bits(), w.page_table,
                              w.ctx_lens, SM_SCALE, abort=exp_ab, cache_dtype=cd)
    err = check_outputs(_host(out32), _host(out16.view(torch.int16)), ref)
    # several queries per request over the same cache (the newest T tokens are
    # appended again by the step: the same bytes)
    T = int(rng.integers(2, 5))
    if G * T <= 32:
        sp = device.build_spec(st, T)
        o32 = _host(sp.decode(out_dtype=fp8kv.OUT_F32))
        refq, _ = oracle.attention_multi(Ko, Vo, st.k_scale_host, st.v_scale_host,
                                         w.q_bits_multi(T), w.page_table, w.ctx_lens, SM_SCALE,
                                         abort=exp_ab, cache_dtype=cd)
        err = max(err, check_outputs(o32, None, refq))
    print(f"case {case}: B={B} Hkv={Hkv} G={G} cache={cd} workers={workers} "
          f"aborted={int(exp_ab.sum())} q_len={T if G * T <= 32 else 1}: max abs err {err:.3e}")


@pytest.mark.parametrize("case", range(SHARED_CASES))
def test_random_shared_prompt_call(case):
    import decode_attention_paged_fp8kv_amd as fp8kv
    from workloads import device
    rng = np.random.default_rng(7000 + case)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    cd = int(rng.integers(0, 2))
    workers = int(rng.choice([0, 8, 64, 512]))
    groups = [(int(rng.integers(1, 7)), 16 * int(rng.integers(1, 11)))
              for _ in range(int(rng.integers(1, 4)))]
    plain = int(rng.integers(0, 4))
    w = workloads.shared_prompts(groups, plain=plain, suffix_max=int(rng.integers(17, 200)),
                                 Hq=G * Hkv, Hkv=Hkv, seed=8000 + case)
    st = device.build(w, cache_dtype=cd)
    st.step(check_tags=True)
    torch.cuda.synchronize()
    assert (_host(st.abort) == 0).all()
    Ko, Vo = oracle_state(w, st.k_scale_host, st.v_scale_host, cd)
    ref, _ = oracle.attention(Ko, Vo, st.k_scale_host, st.v_scale_host, w.q_bits(), w.page_table,
                              w.ctx_lens, SM_SCALE, cache_dtype=cd)
    gs = np.concatenate([[0], np.cumsum([n for n, _ in groups])]).tolist()
    pl = [p for _, p in groups]
    o32 = fp8kv.decode_attention_shared(st.desc, st.K, st.V, st.k_scale, st.v_scale, st.q,
                                        st.page_table, st.ctx_lens, gs, pl, abort=st.abort,
                                        out_dtype=fp8kv.OUT_F32, num_workers=workers)
    o16 = fp8kv.decode_attention_shared(st.desc, st.K, st.V, st.k_scale, st.v_scale, st.q,
                                        st.page_table, st.ctx_lens, gs, pl, abort=st.abort,
                                        num_workers=workers)
    err = check_outputs(_host(o32), _host(o16.view(torch.int16)), ref)
    print(f"shared case {case}: groups={groups} plain={plain} Hkv={Hkv} G={G} cache={cd} "
          f"workers={workers}: max abs err {err:.3e}")
