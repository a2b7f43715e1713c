"""Pins for the oracle's paged attention (CPU only).

Closed forms and invariants that a plausible mistake (a dropped scale, a
wrong GQA index, a page/slot mix-up, a missing normalisation, an off-by-one
in the token range) would break:
  * a context of one token returns that token's V exactly;
  * q = 0, or identical keys, returns the mean of V;
  * an fp64 brute force with math.fsum, no max subtraction and torch's
    float8 decode agrees to 1e-12 relative;
  * permuting physical pages is bitwise neutral; reordering requests
    permutes the output bitwise;
  * GQA equals G=1 with the kv-heads duplicated;
  * a BF16 cache holding the same values gives the same result bitwise;
  * aborted requests and empty contexts give +0.
"""
import math

import numpy as np
import torch

import oracle
import workloads

D, S = 128, 16


def _rand_cache(rng, N, Hkv, nan_free=True):
    K = rng.integers(0, 256, size=(N, Hkv, S, D), dtype=np.uint8)
    V = rng.integers(0, 256, size=(N, Hkv, S, D), dtype=np.uint8)
    if nan_free:
        for X in (K, V):
            X[(X & 0x7F) == 0x7F] = 0x3A
            # keep magnitudes modest so the brute force needs no max shift
            X[((X >> 3) & 0xF) > 9] &= 0xC7
    return K, V


def _case(seed=0, lens=(1, 5, 16, 17, 40), Hq=4, Hkv=2):
    rng = np.random.default_rng(seed)
    B = len(lens)
    n = [(L + S - 1) // S for L in lens]
    N = sum(n) + 3
    perm = rng.permutation(N).astype(np.int32)
    pt = np.full((B, max(n)), -1, np.int32)
    k = 0
    for b in range(B):
        pt[b, :n[b]] = perm[k:k + n[b]]
        k += n[b]
    K, V = _rand_cache(rng, N, Hkv)
    q = workloads.draw_bits(seed + 99, 0, B * Hq * D).reshape(B, Hq, D)
    ks = np.array([0.031, 0.017][:Hkv], np.float32)
    vs = np.array([0.5, 0.0625][:Hkv], np.float32)
    return K, V, ks, vs, q, pt, np.array(lens, np.int32)


def _f8(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def brute_force(K, V, ks, vs, q, pt, lens, sm):
    B, Hq, _ = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    qf = workloads.bf16_bits_to_f32(q).astype(np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            ws, rows = [], []
            for j in range(int(lens[b])):
                p, s = pt[b, j // S], j % S
                k = _f8(K[p, g, s]) * float(ks[g])
                v = _f8(V[p, g, s]) * float(vs[g])
                sc = float(np.float32(sm)) * math.fsum(qf[b, h] * k)
                assert abs(sc) < 50
                ws.append(math.exp(sc))
                rows.append(v)
            den = math.fsum(ws)
            for d in range(D):
                out[b, h, d] = math.fsum(w * r[d] for w, r in zip(ws, rows)) / den
    return out


SM = np.float32(1.0 / math.sqrt(D))


def test_brute_force_agrees():
    K, V, ks, vs, q, pt, L = _case()
    got, _ = oracle.attention(K, V, ks, vs, q, pt, L, SM)
    ref = brute_force(K, V, ks, vs, q, pt, L, SM)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-15)


def test_single_token_returns_v_exactly():
    K, V, ks, vs, q, pt, L = _case(lens=(1, 1, 1))
    got, _ = oracle.attention(K, V, ks, vs, q, pt, L, SM)
    for b in range(3):
        for h in range(4):
            g = h // 2
            v = _f8(V[pt[b, 0], g, 0]) * float(vs[g])
            assert (got[b, h] == v).all()


def test_zero_query_and_equal_keys_give_mean():
    K, V, ks, vs, q, pt, L = _case(lens=(3, 16, 33))
    q0 = np.zeros_like(q)
    got, _ = oracle.attention(K, V, ks, vs, q0, pt, L, SM)
    K2 = K.copy()
    K2[:] = K[0, :, 0:1, :]          # every token gets the same key bytes
    got2, _ = oracle.attention(K2, V, ks, vs, q, pt, L, SM)
    for b in range(3):
        for h in range(4):
            g = h // 2
            vals = [_f8(V[pt[b, j // S], g, j % S]) * float(vs[g]) for j in range(L[b])]
            mean = np.array([math.fsum(v[d] for v in vals) for d in range(D)]) / L[b]
            assert np.allclose(got[b, h], mean, rtol=1e-13, atol=1e-16)
            assert np.allclose(got2[b, h], mean, rtol=1e-13, atol=1e-16)


def test_page_permutation_is_bitwise_neutral():
    K, V, ks, vs, q, pt, L = _case(seed=4)
    ref, rb = oracle.attention(K, V, ks, vs, q, pt, L, SM)
    rng = np.random.default_rng(9)
    N = K.shape[0]
    perm = rng.permutation(N)            # new id of old page i is perm[i]
    K2 = np.empty_like(K)
    V2 = np.empty_like(V)
    K2[perm] = K
    V2[perm] = V
    pt2 = np.where(pt >= 0, perm[np.clip(pt, 0, None)], -1).astype(np.int32)
    got, gb = oracle.attention(K2, V2, ks, vs, q, pt2, L, SM)
    assert (got == ref).all() and (gb == rb).all()


def test_batch_reorder_permutes_output():
    K, V, ks, vs, q, pt, L = _case(seed=5)
    ref, _ = oracle.attention(K, V, ks, vs, q, pt, L, SM)
    order = np.array([3, 0, 4, 2, 1])
    got, _ = oracle.attention(K, V, ks, vs, q[order], pt[order], L[order], SM)
    assert (got == ref[order]).all()


def test_gqa_equals_duplicated_kv_heads():
    K, V, ks, vs, q, pt, L = _case(seed=6, Hq=4, Hkv=2)
    ref, _ = oracle.attention(K, V, ks, vs, q, pt, L, SM)
    K4 = np.repeat(K, 2, axis=1).copy()
    V4 = np.repeat(V, 2, axis=1).copy()
    got, _ = oracle.attention(K4, V4, np.repeat(ks, 2), np.repeat(vs, 2), q, pt, L, SM)
    assert (got == ref).all()


def test_bf16_cache_with_same_values_matches():
    K, V, ks, vs, q, pt, L = _case(seed=7)
    ks = np.array([0.125, 2.0], np.float32)     # powers of two: DEC*scale exact in bf16
    vs = np.array([0.5, 0.25], np.float32)
    ref, _ = oracle.attention(K, V, ks, vs, q, pt, L, SM)
    Kb = np.zeros(K.shape, np.uint16)
    Vb = np.zeros(V.shape, np.uint16)
    for g in range(2):
        kv = (_f8(K[:, g]) * float(ks[g])).astype(np.float32)
        vv = (_f8(V[:, g]) * float(vs[g])).astype(np.float32)
        Kb[:, g] = (kv.view(np.uint32) >> 16).astype(np.uint16)
        Vb[:, g] = (vv.view(np.uint32) >> 16).astype(np.uint16)
        assert (workloads.bf16_bits_to_f32(Kb[:, g]) == kv).all()
    one = np.ones(2, np.float32)
    got, _ = oracle.attention(Kb, Vb, one, one, q, pt, L, SM, cache_dtype=1)
    assert (got == ref).all()


def test_abort_and_empty_context_are_zero():
    K, V, ks, vs, q, pt, L = _case(seed=8)
    L2 = L.copy()
    L2[1] = 0
    ab = np.array([0, 0, 1, 0, 0], np.uint8)
    got, gb = oracle.attention(K, V, ks, vs, q, pt, L2, SM, abort=ab)
    assert (got[1] == 0).all() and (got[2] == 0).all()
    assert not np.signbit(got[1]).any() and not np.signbit(got[2]).any()
    assert (gb[1] == 0).all() and (gb[2] == 0).all()
    ref, _ = oracle.attention(K, V, ks, vs, q, pt, L, SM)
    for b in (0, 3, 4):
        assert (got[b] == ref[b]).all()


def test_bf16_output_is_rne_of_f64():
    K, V, ks, vs, q, pt, L = _case(seed=10)
    got, gb = oracle.attention(K, V, ks, vs, q, pt, L, SM)
    ref = torch.from_numpy(got.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    # float64 -> float32 -> bf16 may double-round; it agrees except exactly at
    # a bf16 midpoint, which random data does not hit.
    assert (gb.view(np.int16) == ref).all()


def test_workload_step_end_to_end():
    """Tiny workload: bulk fill by append, then append the step's token,
    then attend; outputs are convex combinations of the cached V rows."""
    w = workloads.make(1)
    ks = workloads.scales_from_amax(w.amax_numpy("k"))
    vs = workloads.scales_from_amax(w.amax_numpy("v"))
    K, V = oracle.new_cache(w.num_pages, w.Hkv)
    for b in range(w.B):
        n = int(w.ctx_before[b]) + 1
        kb = w.kv_tokens("k", b, 0, n)
        vb = w.kv_tokens("v", b, 0, n)
        oracle.append(K, V, ks, vs, kb, vb, np.full(n, b, np.int32),
                      np.arange(n, dtype=np.int32), w.page_table)
    out, _ = oracle.attention(K, V, ks, vs, w.q_bits(), w.page_table, w.ctx_lens, SM)
    assert np.isfinite(out).all()
    for b in range(w.B):
        for h in range(w.Hq):
            g = h // w.G
            vals = np.stack([_f8(V[w.page_table[b, j // S], g, j % S]) * float(vs[g])
                             for j in range(int(w.ctx_lens[b]))])
            assert (out[b, h] <= vals.max(0) + 1e-12).all()
            assert (out[b, h] >= vals.min(0) - 1e-12).all()


# ---------------------------------------------------------------------------
# several new tokens per request (speculative verification): query i sees the
# cached tokens and the new tokens up to its own
# ---------------------------------------------------------------------------
def _multi_case(T, seed=5, lens=(3, 16, 17, 33), Hq=4, Hkv=2):
    K, V, ks, vs, _, pt, L = _case(seed=seed, lens=lens, Hq=Hq, Hkv=Hkv)
    q = workloads.draw_bits(seed + 7, 0, len(lens) * T * Hq * D).reshape(len(lens), T, Hq, D)
    return K, V, ks, vs, q, pt, L


def test_multi_one_query_is_single_query_attention():
    K, V, ks, vs, q, pt, L = _multi_case(1)
    got, gb = oracle.attention_multi(K, V, ks, vs, q, pt, L, SM)
    ref, rb = oracle.attention(K, V, ks, vs, np.ascontiguousarray(q[:, 0]), pt, L, SM)
    assert (got[:, 0] == ref).all() and (gb[:, 0] == rb).all()


def test_multi_rows_agree_with_brute_force_over_their_prefix():
    T = 3
    K, V, ks, vs, q, pt, L = _multi_case(T)
    got, _ = oracle.attention_multi(K, V, ks, vs, q, pt, L, SM)
    for i in range(T):
        seen = L - (T - 1 - i)                     # query i: tokens 0 .. L-T+i
        ref = brute_force(K, V, ks, vs, np.ascontiguousarray(q[:, i]), pt, seen, SM)
        assert np.allclose(got[:, i], ref, rtol=1e-12, atol=1e-15), i


def test_multi_is_causal_among_the_new_tokens():
    """Changing the last new token's K and V changes only the last query."""
    T = 4
    K, V, ks, vs, q, pt, L = _multi_case(T, lens=(20, 35))
    a, _ = oracle.attention_multi(K, V, ks, vs, q, pt, L, SM)
    K2, V2 = K.copy(), V.copy()
    for b in range(len(L)):
        j = int(L[b]) - 1                          # position of the last new token
        p, s = pt[b, j // S], j % S
        K2[p, :, s] ^= 0x11
        V2[p, :, s] ^= 0x22
    b_, _ = oracle.attention_multi(K2, V2, ks, vs, q, pt, L, SM)
    assert (a[:, :T - 1] == b_[:, :T - 1]).all()
    assert not (a[:, T - 1] == b_[:, T - 1]).all()


def test_multi_queries_beyond_the_context_are_zero():
    T = 3
    K, V, ks, vs, q, pt, L = _multi_case(T, lens=(1, 2, 5))
    got, gb = oracle.attention_multi(K, V, ks, vs, q, pt, L, SM)
    assert (got[0, :2] == 0).all() and (got[1, :1] == 0).all() and (gb[0, :2] == 0).all()
    assert (got[0, 2] != 0).any() and (got[1, 1] != 0).any()


def test_thread_count_does_not_change_results():
    """Attention rows are computed by one thread each in a fixed order, so the
    thread count (timing only) leaves every bit unchanged."""
    rng = np.random.default_rng(12)
    B, Hq, Hkv, P = 5, 8, 2, 6
    n = [3, 1, 6, 2, 5]
    K, V = oracle.new_cache(40, Hkv)
    K[:] = rng.integers(0, 0x7F, K.shape, dtype=np.uint8)
    V[:] = rng.integers(0, 0x7F, V.shape, dtype=np.uint8)
    pt = np.full((B, P), -1, np.int32)
    perm = rng.permutation(40).astype(np.int32)
    k = 0
    for b in range(B):
        pt[b, :n[b]] = perm[k:k + n[b]]
        k += n[b]
    ctx = np.array([16 * x - 3 for x in n], np.int32)
    q = rng.integers(0, 0x4000, (B, Hq, 128), dtype=np.uint16)
    ks = np.full(Hkv, 0.05, np.float32)
    outs = []
    base = oracle.num_threads()
    for t in (1, max(2, base)):
        oracle.set_num_threads(t)
        outs.append(oracle.attention(K, V, ks, ks, q, pt, ctx, np.float32(0.088))[0])
    oracle.set_num_threads(base)
    assert np.array_equal(outs[0], outs[1])
