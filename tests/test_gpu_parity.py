"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Quantized cache bytes and abort flags must match bit for bit; attention
outputs within 2e-3 (f32 output mode), and the BF16 output must be the
round-to-nearest-even of the f32 one (see _helpers.check_outputs).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import SM_SCALE, check_outputs, oracle_state, unswizzle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_paged_fp8kv_amd as m
    return m


@pytest.fixture(scope="module")
def dev():
    from workloads import device
    return device


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# ---------------------------------------------------------------------------
# conversions and quantization
# ---------------------------------------------------------------------------
def test_on_read_conversion_all_codes(lib):
    codes = torch.arange(256, dtype=torch.uint8, device="cuda")
    tab = oracle.e4m3_table()
    for which in (0, 1):
        got = _host(lib.debug_convert_e4m3(codes, which)).astype(np.float64)
        nan = np.isnan(tab)
        assert (np.isnan(got) == nan).all(), which
        assert (got[~nan] == tab[~nan]).all(), which
        assert (np.signbit(got[~nan]) == np.signbit(tab[~nan])).all(), which


@pytest.mark.parametrize("cache_dtype", [0, 1])
def test_append_every_bf16_pattern(lib, cache_dtype):
    T, Hkv = 512, 1
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    kn = pats.reshape(T, Hkv, 128)
    vn = pats[::-1].copy().reshape(T, Hkv, 128)
    pt = np.arange(32, dtype=np.int32).reshape(1, 32)
    seq = np.zeros(T, np.int32)
    pos = np.arange(T, dtype=np.int32)
    scales = [1.0, 0.0123, float(np.float32(20) / np.float32(448)), 1e-3, 3.3e4, 2.0 ** -10, 7.0]
    d = lib.desc(32, Hkv, cache_dtype)
    for s in scales:
        sc = np.array([s], np.float32)
        K, V = lib.new_cache(d)
        lib.append(d, K, V, torch.from_numpy(sc).cuda(), torch.from_numpy(sc).cuda(),
                   torch.from_numpy(kn.view(np.int16)).cuda(),
                   torch.from_numpy(vn.view(np.int16)).cuda(),
                   torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                   torch.from_numpy(pt).cuda())
        Ko, Vo = oracle.new_cache(32, Hkv, cache_dtype)
        oracle.append(Ko, Vo, sc, sc, kn, vn, seq, pos, pt, cache_dtype=cache_dtype)
        gk = unswizzle(_host(K), Hkv, cache_dtype, range(32), False)
        gv = unswizzle(_host(V), Hkv, cache_dtype, range(32), True)
        bad_k = np.flatnonzero(gk.ravel() != Ko.ravel())
        bad_v = np.flatnonzero(gv.ravel() != Vo.ravel())
        assert bad_k.size == 0 and bad_v.size == 0, (s, bad_k[:8], bad_v[:8])


@pytest.mark.parametrize("cache_dtype", [0, 1])
def test_append_skips_what_is_out_of_range(lib, cache_dtype):
    """Tokens naming a request outside the table, a negative position, a
    position past the table, or a page id outside the pool are skipped: the
    pools hold exactly what the oracle writes for the valid tokens."""
    N, Hkv, P = 12, 2, 4
    rng = np.random.default_rng(17)
    pt = rng.permutation(N)[:3 * P].astype(np.int32).reshape(3, P)
    pt[1, 2] = -1
    pt[2, 3] = N + 3
    seq = np.array([0, 0, -1, 3, 1, 1, 1, 2, 2, 2, 0, 1], np.int32)
    pos = np.array([0, 17, 5, 5, -1, 33, 40, 63, 1, P * 16, 63, 2], np.int32)
    T = seq.size
    kn = rng.integers(0, 2 ** 16, (T, Hkv, 128)).astype(np.uint16)
    vn = rng.integers(0, 2 ** 16, (T, Hkv, 128)).astype(np.uint16)
    # no NaN inputs (their codes are checked elsewhere): clear the top exponent bit
    kn &= np.uint16(0xBFFF)
    vn &= np.uint16(0xBFFF)
    sc = np.array([0.05, 0.2], np.float32)
    d = lib.desc(N, Hkv, cache_dtype)
    K, V = lib.new_cache(d)
    lib.append(d, K, V, torch.from_numpy(sc).cuda(), torch.from_numpy(sc).cuda(),
               torch.from_numpy(kn.view(np.int16)).cuda(), torch.from_numpy(vn.view(np.int16)).cuda(),
               torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), torch.from_numpy(pt).cuda())
    Ko, Vo = oracle.new_cache(N, Hkv, cache_dtype)
    skipped = oracle.append(Ko, Vo, sc, sc, kn, vn, seq, pos, pt, cache_dtype=cache_dtype)
    assert (unswizzle(_host(K), Hkv, cache_dtype, range(N), False) == Ko).all()
    assert (unswizzle(_host(V), Hkv, cache_dtype, range(N), True) == Vo).all()
    print(f"append: {T} tokens, oracle skipped {skipped}")


# ---------------------------------------------------------------------------
# tag check
# ---------------------------------------------------------------------------
def test_verify_hand_cases_and_random(lib):
    from test_oracle_verify import _load_cases
    pool, cases = _load_cases()
    tags = np.array([pool[i] for i in range(len(pool))], np.uint32)
    P = max(len(c[2]) for c in cases)
    pt = np.full((len(cases), P), -1, np.int32)
    et = np.zeros((len(cases), P), np.uint32)
    cl = np.zeros(len(cases), np.int32)
    for b, (_, ctx, ids, tg, _) in enumerate(cases):
        pt[b, :len(ids)] = ids
        et[b, :len(tg)] = tg
        cl[b] = ctx
    exp = np.array([c[4] for c in cases], np.uint8)
    ab = lib.verify_tags(torch.from_numpy(pt).cuda(), torch.from_numpy(et.view(np.int32)).cuda(),
                         torch.from_numpy(cl).cuda(), torch.from_numpy(tags.view(np.int32)).cuda())
    assert (_host(ab) == exp).all()
    rng = np.random.default_rng(21)
    for trial in range(10):
        N = int(rng.integers(1, 5000))
        tags = rng.integers(0, 2 ** 32, N, dtype=np.uint64).astype(np.uint32)
        B = int(rng.integers(1, 300))
        P = int(rng.integers(1, 3000))
        ptr = rng.integers(0, N, size=(B, P)).astype(np.int32)
        bad = rng.random((B, P)) < 0.0005
        ptr[bad] = rng.choice(np.array([-1, -7, N, N + 5], np.int32), size=int(bad.sum()))
        ok = (ptr >= 0) & (ptr < N)
        etr = np.where(ok, tags[np.clip(ptr, 0, N - 1)], 0).astype(np.uint32)
        etr[rng.random((B, P)) < 0.001] += np.uint32(1)
        clr = rng.integers(-1, P * 16 + 40, B).astype(np.int32)
        exp = oracle.verify(ptr, etr, clr, tags)
        got = lib.verify_tags(torch.from_numpy(ptr).cuda(), torch.from_numpy(etr.view(np.int32)).cuda(),
                              torch.from_numpy(clr).cuda(), torch.from_numpy(tags.view(np.int32)).cuda())
        assert (_host(got) == exp).all(), trial


# ---------------------------------------------------------------------------
# full step on the tiny workload
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cache_dtype", [0, 1])
def test_tiny_step_parity(lib, dev, cache_dtype):
    w = workloads.make(1)
    st = dev.build(w, cache_dtype=cache_dtype)
    out16 = st.step(check_tags=True)
    out32 = st.decode(out_dtype=lib.OUT_F32)
    ab = _host(st.abort)
    exp_ab = oracle.verify(w.page_table, w.expected_tags, w.ctx_lens, w.pool_tags)
    assert (ab == exp_ab).all() and (ab == 0).all()
    Ko, Vo = oracle_state(w, st.k_scale_host, st.v_scale_host, cache_dtype, abort=exp_ab)
    pages = np.arange(w.num_pages)
    gk = unswizzle(_host(st.K), w.Hkv, cache_dtype, pages, False)
    gv = unswizzle(_host(st.V), w.Hkv, cache_dtype, pages, True)
    assert (gk == Ko).all() and (gv == Vo).all()
    ref, _ = oracle.attention(Ko, Vo, st.k_scale_host, st.v_scale_host, w.q_bits(), w.page_table,
                              w.ctx_lens, SM_SCALE, abort=exp_ab, cache_dtype=cache_dtype)
    err = check_outputs(_host(out32), _host(out16.view(torch.int16)), ref)
    print(f"tiny cache_dtype={cache_dtype} max abs err {err:.3e}")


# ---------------------------------------------------------------------------
# shapes, lengths, work partitions
# ---------------------------------------------------------------------------
EDGE_LENS = [0, 1, 14, 15, 16, 17, 30, 31, 32, 47, 63, 64, 65, 127, 255, 256, 300, 1023, 2100]


@pytest.mark.parametrize("G,Hkv", [(1, 4), (2, 2), (4, 2), (8, 1), (16, 1), (8, 3), (32, 1),
                                   (24, 2)])
@pytest.mark.parametrize("workers", [0, 4, 12, 64, 1024])
def test_lengths_groups_workers(lib, dev, G, Hkv, workers):
    """Few workers: slices cross many (request, kv-head) boundaries.  Many
    workers: most segments are split and merged."""
    w = workloads.custom("edge", EDGE_LENS, Hq=G * Hkv, Hkv=Hkv, seed=G * 10 + Hkv, pool_slack=5)
    st = dev.build(w, num_workers=workers)
    out16 = st.step(check_tags=True)
    out32 = st.decode(out_dtype=lib.OUT_F32)
    Ko, Vo = oracle_state(w, st.k_scale_host, st.v_scale_host)
    ref, _ = oracle.attention(Ko, Vo, st.k_scale_host, st.v_scale_host, w.q_bits(), w.page_table,
                              w.ctx_lens, SM_SCALE)
    err = check_outputs(_host(out32), _host(out16.view(torch.int16)), ref)
    assert err < 1e-4


@pytest.mark.parametrize("cache_dtype", [0, 1])
def test_fused_equals_separate_check_and_append(lib, dev, cache_dtype):
    w = workloads.make(5, batch=40)
    a = dev.build(w, cache_dtype=cache_dtype, num_workers=64)
    b = dev.build(w, cache_dtype=cache_dtype, num_workers=64)
    oa = _host(a.step(check_tags=True, fused=True).view(torch.int16)).copy()
    ob = _host(b.step(check_tags=True, fused=False).view(torch.int16)).copy()
    assert (_host(a.abort) == w.expected_abort).all()
    assert (_host(a.abort) == _host(b.abort)).all()
    assert (_host(a.K) == _host(b.K)).all() and (_host(a.V) == _host(b.V)).all()
    assert (oa == ob).all()


@pytest.mark.parametrize("tracker", [True, False])
def test_step_helper_equals_its_calls(lib, dev, tracker):
    """fp8kv.step runs check + append (one launch) and attention, or without the
    tags the no-op tracker's append and attention: the same bits as the calls."""
    import decode_attention_paged_fp8kv_amd as fp8kv
    w = workloads.make(5, batch=24)
    a = dev.build(w, num_workers=64)
    b = dev.build(w, num_workers=64)
    tags = dict(expected_tags=a.expected_tags, pool_tags=a.pool_tags) if tracker else {}
    out, ab = fp8kv.step(a.desc, a.K, a.V, a.k_scale, a.v_scale, a.q, a.k_new, a.v_new,
                         a.token_pos, a.page_table, a.ctx_lens, num_workers=64, **tags)
    ref = b.step(check_tags=tracker)
    assert torch.equal(out, ref)
    assert torch.equal(a.K, b.K) and torch.equal(a.V, b.V)
    if tracker:
        assert (_host(ab) == w.expected_abort).all() and torch.equal(ab, b.abort)
    else:
        assert ab is None


@pytest.mark.parametrize("workers", [0, 256, 3072, 6144])
def test_short_segments_among_long_ones(lib, dev, workers):
    """Many 1..40-token requests around a few long ones, 64/8 heads: slices
    hold many short (request, kv-head) segments, and with many workers some
    slices end inside a segment's leading work items and hold no page."""
    rng = np.random.default_rng(77)
    L = rng.integers(0, 41, 96)
    L[[5, 40, 77]] = [2047, 3000, 1500]
    w = workloads.custom("short_long", L, Hq=64, Hkv=8, seed=77, pool_slack=2)
    st = dev.build(w, num_workers=workers)
    out16 = st.step(check_tags=True)
    out32 = st.decode(out_dtype=lib.OUT_F32)
    Ko, Vo = oracle_state(w, st.k_scale_host, st.v_scale_host)
    ref, _ = oracle.attention(Ko, Vo, st.k_scale_host, st.v_scale_host, w.q_bits(), w.page_table,
                              w.ctx_lens, SM_SCALE)
    err = check_outputs(_host(out32), _host(out16.view(torch.int16)), ref)
    assert err < 1e-4
    print(f"short among long, workers={workers}: max abs err {err:.3e}")


def test_largest_batch(lib, dev):
    """4096 requests (the largest batch) with short contexts, 1% of them holding
    one stale entry: every abort flag, every cache byte and every output row
    against the oracle, also through the two-tile kernel with 8 queries per
    request; one request more is rejected."""
    rng = np.random.default_rng(4096)
    L = rng.integers(0, 41, 4096)
    w = workloads.custom("max_batch", L, Hq=8, Hkv=2, seed=4096, pool_slack=3)
    for b in rng.choice(4096, 41, replace=False):
        i = int(rng.integers(0, w.n_pages[b]))
        w.pool_tags[w.page_table[b, i]] += np.uint32(1)      # the page was handed out again
        w.stale[b, i] = True
    for b in range(4096):                                    # sharers of a bumped page see it too
        n = w.n_pages[b]
        w.stale[b, :n] = w.expected_tags[b, :n] != w.pool_tags[w.page_table[b, :n]]
    st = dev.build(w)
    out16 = st.step(check_tags=True)
    out32 = st.decode(out_dtype=lib.OUT_F32)
    ab = _host(st.abort)
    exp_ab = oracle.verify(w.page_table, w.expected_tags, w.ctx_lens, w.pool_tags)
    assert (exp_ab == w.expected_abort).all() and 30 <= exp_ab.sum() <= 41
    assert (ab == exp_ab).all()
    Ko, Vo = oracle_state(w, st.k_scale_host, st.v_scale_host, abort=exp_ab)
    pages = np.arange(w.num_pages)
    assert (unswizzle(_host(st.K), w.Hkv, 0, pages, False) == Ko).all()
    assert (unswizzle(_host(st.V), w.Hkv, 0, pages, True) == Vo).all()
    ref, _ = oracle.attention(Ko, Vo, st.k_scale_host, st.v_scale_host, w.q_bits(), w.page_table,
                              w.ctx_lens, SM_SCALE, abort=exp_ab)
    o32 = _host(out32)
    assert (o32[exp_ab == 1] == 0).all()
    err = check_outputs(o32, _host(out16.view(torch.int16)), ref)
    print(f"4096 requests, {int(exp_ab.sum())} aborted: max abs err {err:.3e}")
    # the same batch through the two-tile kernel: 8 queries per request (32 columns)
    q8 = workloads.draw_bits(77, 0, 4096 * 8 * 8 * 128).reshape(4096, 8, 8, 128)
    o8 = lib.decode_attention_q(st.desc, st.K, st.V, st.k_scale, st.v_scale,
                                torch.from_numpy(q8.view(np.int16)).cuda(), st.page_table,
                                st.ctx_lens, abort=st.abort, out_dtype=lib.OUT_F32)
    ref8, _ = oracle.attention_multi(Ko, Vo, st.k_scale_host, st.v_scale_host, q8, w.page_table,
                                     w.ctx_lens, SM_SCALE, abort=exp_ab)
    err8 = check_outputs(_host(o8), None, ref8)
    print(f"4096 requests x 8 queries (two tiles): max abs err {err8:.3e}")
    big = torch.zeros(4097, dtype=torch.int32, device="cuda")
    with pytest.raises(lib.Fp8kvError) as e:
        lib.decode_attention(st.desc, st.K, st.V, st.k_scale, st.v_scale,
                             torch.zeros((4097, 8, 128), dtype=torch.int16, device="cuda"),
                             torch.zeros((4097, 4), dtype=torch.int32, device="cuda"), big)
    assert e.value.status == -2


def test_read_reference_reads_every_byte_once(lib):
    """The streaming-read reference: the XOR of its sink words is the XOR of all
    words of the buffer (a chunk read twice or skipped would change it), for a
    size that is not a multiple of the grid's stride."""
    rng = np.random.default_rng(16)
    n = (1 << 26) + 16 * 12345
    host = rng.integers(0, 256, n, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    sink = _host(lib.debug_read_bandwidth(buf))
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert np.bitwise_xor.reduce(sink.view(np.uint32)) == want
    with pytest.raises(lib.Fp8kvError):
        lib.debug_read_bandwidth(buf[:100])


def test_empty_context_and_abort_rows_are_zero(lib, dev):
    w = workloads.custom("edge", [40, 100, 7, 300], Hq=8, Hkv=2, seed=3)
    st = dev.build(w, num_workers=8)
    st.step(check_tags=True)
    ref = _host(st.decode(out_dtype=lib.OUT_F32)).copy()
    cl = st.ctx_lens.clone()
    st.ctx_lens[1] = 0                       # empty context
    st.abort.copy_(torch.tensor([0, 0, 1, 0], dtype=torch.uint8))
    out = _host(st.decode(out_dtype=lib.OUT_F32))
    assert (out[1] == 0).all() and (out[2] == 0).all() and not np.signbit(out[1:3]).any()
    assert np.abs(out[0] - ref[0]).max() < 1e-5 and np.abs(out[3] - ref[3]).max() < 1e-5
    st.ctx_lens.copy_(cl)


def test_bad_page_ids_without_the_check(lib, dev):
    """The no-op tracker (no abort array) on a table with ids outside the pool
    in one request: nothing outside the pool is read (the loads of such a page
    are empty), the other requests' rows keep their bits, and the plain,
    multi-query and shared-prompt calls all return."""
    w = workloads.custom("bad_ids", [40, 100, 300, 77], Hq=16, Hkv=2, seed=9, pool_slack=3)
    st = dev.build(w, num_workers=16)
    st.step(check_tags=True)
    good = _host(st.decode(use_abort=False, out_dtype=lib.OUT_F32)).copy()
    pt = st.page_table.clone()
    N = w.num_pages
    bad = torch.tensor([-1, -7, N, N + 5, 2 ** 31 - 1, -(2 ** 31)], dtype=torch.int32, device="cuda")
    st.page_table[2, 1:1 + bad.numel()] = bad
    out = _host(st.decode(use_abort=False, out_dtype=lib.OUT_F32))
    keep = [0, 1, 3]
    assert (out[keep] == good[keep]).all()
    assert np.isfinite(out[2]).all()
    q4 = st.q.unsqueeze(1).expand(-1, 2, -1, -1).contiguous()        # two queries per request
    o4 = lib.decode_attention_q(st.desc, st.K, st.V, st.k_scale, st.v_scale, q4, st.page_table,
                                st.ctx_lens, out_dtype=lib.OUT_F32, num_workers=16)
    assert np.isfinite(_host(o4)).all()
    osh = lib.decode_attention_shared(st.desc, st.K, st.V, st.k_scale, st.v_scale, st.q,
                                      st.page_table, st.ctx_lens, [0, 4], [32],
                                      out_dtype=lib.OUT_F32, num_workers=16)
    assert np.isfinite(_host(osh)).all()
    st.page_table.copy_(pt)


def test_calls_on_another_stream(lib, dev):
    """The entry points enqueue on the stream they are given, or torch's
    current one: the step on a side stream (prepared launches made for it),
    then the check + append and the attention with an explicit stream
    argument, give the default stream's bits; the stale requests abort alike."""
    w = workloads.make(5, batch=24)
    a = dev.build(w, num_workers=64)
    b = dev.build(w, num_workers=64)
    c = dev.build(w, num_workers=64)
    ref = a.step(check_tags=True).clone()
    torch.cuda.synchronize()
    s1 = torch.cuda.Stream()
    with torch.cuda.stream(s1):
        out1 = b.step(check_tags=True)
    s1.synchronize()
    s2 = torch.cuda.Stream()
    lib.verify_append(c.desc, c.K, c.V, c.k_scale, c.v_scale, c.k_new, c.v_new, c.token_pos,
                      c.page_table, c.expected_tags, c.ctx_lens, c.pool_tags, abort=c.abort,
                      stream=s2)
    out2 = lib.decode_attention(c.desc, c.K, c.V, c.k_scale, c.v_scale, c.q, c.page_table,
                                c.ctx_lens, abort=c.abort, num_workers=64, stream=s2)
    s2.synchronize()
    assert (_host(a.abort) == w.expected_abort).all()
    for st, out in ((b, out1), (c, out2)):
        assert torch.equal(out, ref)
        assert torch.equal(st.abort, a.abort)
        assert torch.equal(st.K, a.K) and torch.equal(st.V, a.V)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def test_invariants(lib, dev):
    w = workloads.custom("inv", [100, 33, 700, 1500, 16, 2047], Hq=16, Hkv=2, seed=5, pool_slack=7)
    st = dev.build(w, num_workers=16)
    out = _host(st.step(check_tags=True).view(torch.int16)).copy()
    # run-to-run determinism
    for _ in range(3):
        assert (_host(st.decode().view(torch.int16)) == out).all()
    # permute physical pages (move the tiles, rewrite the page table): identical bits
    N = w.num_pages
    perm = torch.from_numpy(np.random.default_rng(1).permutation(N)).cuda()
    tile = st.K.numel() // N
    K2 = torch.empty_like(st.K).view(N, tile)
    V2 = torch.empty_like(st.V).view(N, tile)
    K2[perm] = st.K.view(N, tile)
    V2[perm] = st.V.view(N, tile)
    pt2 = torch.where(st.page_table >= 0, perm[st.page_table.clamp(min=0).long()].int(),
                      st.page_table)
    out2 = lib.decode_attention(st.desc, K2.view(-1), V2.view(-1), st.k_scale, st.v_scale, st.q,
                                pt2.contiguous(), st.ctx_lens, num_workers=16)
    assert (_host(out2.view(torch.int16)) == out).all()
    # reorder the batch: rows move with it (the work partition changes, so
    # agreement is to rounding, not bits)
    f_ref = _host(st.decode(out_dtype=lib.OUT_F32)).copy()
    order = torch.tensor([3, 0, 5, 1, 4, 2], device="cuda")
    out3 = lib.decode_attention(st.desc, st.K, st.V, st.k_scale, st.v_scale,
                                st.q[order].contiguous(), st.page_table[order].contiguous(),
                                st.ctx_lens[order].contiguous(), out_dtype=lib.OUT_F32,
                                num_workers=16)
    assert np.abs(_host(out3) - f_ref[order.cpu().numpy()]).max() < 1e-5
    # other partitions agree to rounding
    for nw in (4, 64, 4096):
        f2 = _host(st.decode(out_dtype=lib.OUT_F32, num_workers=nw))
        assert np.abs(f2 - f_ref).max() < 1e-5, nw


def test_abort_isolation(lib, dev):
    """Stale tags: aborted requests get +0 rows and write nothing; nothing the
    other requests produce depends on the aborted requests' pages."""
    w = workloads.make(5, batch=24)
    st = dev.build(w, num_workers=64)
    K0 = _host(st.K).copy()
    out = _host(st.step(check_tags=True).view(torch.int16)).copy()
    ab = _host(st.abort)
    assert (ab == w.expected_abort).all() and 0 < ab.sum() < w.B
    assert (out[ab == 1] == 0).all()
    # the aborted requests' new-token slots are untouched
    Kh = _host(st.K)
    d = st.desc
    for b in np.flatnonzero(ab):
        L = int(w.ctx_before[b])
        page = int(w.page_table[b, L // 16])
        for h in range(w.Hkv):
            for dim in (0, 77, 127):
                off = lib.cache_offset(d, 0, page, h, L % 16, dim)
                assert Kh[off] == K0[off]
    # scramble every page of the aborted requests: the other outputs keep their bits
    tile = st.K.numel() // w.num_pages
    gen = torch.Generator(device="cuda").manual_seed(3)
    for b in np.flatnonzero(ab):
        pages = torch.from_numpy(w.page_table[b, : w.n_pages[b]].astype(np.int64)).cuda()
        for X in (st.K, st.V):
            Xv = X.view(w.num_pages, tile)
            Xv[pages] = torch.randint(0, 256, (pages.numel(), tile), dtype=torch.uint8,
                                      device="cuda", generator=gen)
    out2 = _host(st.decode().view(torch.int16))
    assert (out2 == out).all()
    # survivors agree (to rounding) with a batch made of survivors only
    keep = np.flatnonzero(ab == 0)
    kt = torch.from_numpy(keep).cuda()
    f_all = _host(st.decode(out_dtype=lib.OUT_F32)).copy()
    out_k = lib.decode_attention(st.desc, st.K, st.V, st.k_scale, st.v_scale,
                                 st.q[kt].contiguous(), st.page_table[kt].contiguous(),
                                 st.ctx_lens[kt].contiguous(), out_dtype=lib.OUT_F32,
                                 num_workers=64)
    assert np.abs(_host(out_k) - f_all[keep]).max() < 1e-5


def test_pool_sync_and_device_check(lib):
    """Tags change on the host pool; pool_sync uploads them on the stream; the
    device check sees the new lifetime of a reclaimed page."""
    N = 300
    pool = lib.Pool(N, seed=9)
    d_tags = torch.zeros(N, dtype=torch.int32, device="cuda")
    pool.sync(d_tags)
    assert (_host(d_tags).view(np.uint32) == pool.tags()).all()
    reqs = [pool.alloc(k) for k in (5, 9, 2, 7)]
    P = 9
    pt = np.full((4, P), -1, np.int32)
    et = np.zeros((4, P), np.uint32)
    for b, (ids, tg) in enumerate(reqs):
        pt[b, :ids.size] = ids
        et[b, :tg.size] = tg
    cl = np.array([80, 144, 20, 100], np.int32)
    pool.sync(d_tags)
    dpt = torch.from_numpy(pt).cuda()
    det = torch.from_numpy(et.view(np.int32)).cuda()
    dcl = torch.from_numpy(cl).cuda()
    ab = lib.verify_tags(dpt, det, dcl, d_tags)
    assert (_host(ab) == 0).all()
    # request 1 is cancelled; its pages are reissued to a new request
    pool.free(reqs[1][0])
    _ = pool.alloc(pool.num_free - 9)
    new_ids, _ = pool.alloc(9)
    assert set(new_ids) == set(reqs[1][0])
    pool.sync(d_tags)
    ab = lib.verify_tags(dpt, det, dcl, d_tags)
    exp = oracle.verify(pt, et, cl, pool.tags())
    assert (_host(ab) == exp).all() and list(exp) == [0, 1, 0, 0]
    pool.close()


def test_fused_check_fails_closed(lib, dev):
    """The fused check + append writes only into pages it checked: a request
    whose new token lies outside the context it was checked for (the token at
    a page boundary left out of ctx, a position past ctx, a negative position)
    aborts and writes nothing; a length near INT32_MAX aborts as the oracle's
    check does (its page count does not wrap)."""
    w = workloads.custom("failclosed", [31, 47, 63, 64, 100, 20], Hq=8, Hkv=2, seed=11)
    st = dev.build(w, num_workers=8)
    ctx = w.ctx_lens.copy()
    pos = w.ctx_before.astype(np.int32).copy()
    ctx[3] = 64            # token 64 opens page 4, which a 64-token context never checks
    pos[1] = -1
    ctx[2] = 2 ** 31 - 2
    pos[4] = ctx[4]        # one past the context
    st.ctx_lens.copy_(torch.from_numpy(ctx))
    st.token_pos.copy_(torch.from_numpy(pos))
    K0, V0 = _host(st.K).copy(), _host(st.V).copy()
    lib.verify_append(st.desc, st.K, st.V, st.k_scale, st.v_scale, st.k_new, st.v_new,
                      st.token_pos, st.page_table, st.expected_tags, st.ctx_lens, st.pool_tags,
                      abort=st.abort)
    ab = _host(st.abort)
    check = oracle.verify(w.page_table, w.expected_tags, ctx, w.pool_tags)
    inside = (pos >= 0) & (pos.astype(np.int64) + 1 <= ctx)
    assert (ab == (check | ~inside)).all() and ab.tolist() == [0, 1, 1, 1, 1, 0]
    # the separate check agrees on the lengths alone
    assert (_host(lib.verify_tags(st.page_table, st.expected_tags, st.ctx_lens,
                                  st.pool_tags)) == check).all() and check[2] == 1
    # only requests 0 and 5 wrote their token: every other byte is unchanged
    K1, V1 = _host(st.K), _host(st.V)
    written = np.zeros(K0.size, bool)
    for b in (0, 5):
        page = int(w.page_table[b, pos[b] // 16])
        for h in range(w.Hkv):
            for dim in range(128):
                for is_v in (0, 1):
                    written[lib.cache_offset(st.desc, is_v, page, h, int(pos[b]) % 16, dim)] = True
    assert (K1[~written] == K0[~written]).all() and (V1[~written] == V0[~written]).all()
    # attention without the tracker never reads past a length the table cannot hold
    out = _host(lib.decode_attention(st.desc, st.K, st.V, st.k_scale, st.v_scale, st.q,
                                     st.page_table, st.ctx_lens, out_dtype=lib.OUT_F32,
                                     num_workers=8))
    assert (out[2].view(np.uint32) == 0).all()
    # several new tokens per request: all of them inside the context, or abort
    B = w.B
    kq = torch.stack([st.k_new, st.k_new], 1).contiguous()
    vq = torch.stack([st.v_new, st.v_new], 1).contiguous()
    first = torch.from_numpy(w.ctx_lens - 2).to(st.token_pos.device)
    first[0] = int(w.ctx_lens[0]) - 1          # its second token would be at ctx
    st.ctx_lens.copy_(torch.from_numpy(w.ctx_lens))
    abq = _host(lib.verify_append_q(st.desc, st.K, st.V, st.k_scale, st.v_scale, kq, vq, first,
                                    st.page_table, st.expected_tags, st.ctx_lens, st.pool_tags))
    assert abq.tolist() == [1] + [0] * (B - 1)
