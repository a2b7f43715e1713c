"""Page pool (free list + generation tags) and fault injection on the CPU.

The integrity scheme: every physical page's tag changes whenever the page is
handed out again; a request keeps the (page, tag) pairs it was given, and a
stale pair must make the tag check abort that request only.  Properties are
checked against a plain Python model; the scenarios of the commentary page's
advice on fault injection (cancellation, page reclamation, batch reordering,
concurrent releases) are replayed through the pool and the oracle's check.
"""
import random

import numpy as np
import pytest

import decode_attention_paged_fp8kv_amd as fp8kv
import oracle


def test_random_alloc_free_against_model():
    rng = random.Random(1)
    for trial in range(20):
        N = rng.randint(1, 60)
        pool = fp8kv.Pool(N, seed=trial)
        tags = {i: int(t) for i, t in enumerate(pool.tags())}
        live, free = set(), list(range(N))
        for step in range(300):
            if rng.random() < 0.55:
                n = rng.randint(0, 6)
                if n > len(free):
                    with pytest.raises(fp8kv.Fp8kvError) as e:
                        pool.alloc(n)
                    assert e.value.status == -3
                    continue
                ids, tg = pool.alloc(n)
                exp_ids = free[:n]
                del free[:n]
                assert list(ids) == exp_ids                 # first in, first out
                for i, t in zip(ids, tg):
                    assert int(i) not in live
                    tags[int(i)] = (tags[int(i)] + 1) & 0xFFFFFFFF   # new lifetime, new tag
                    assert int(t) == tags[int(i)] == pool.tag(int(i))
                    live.add(int(i))
            else:
                if live and rng.random() < 0.8:
                    k = rng.randint(1, len(live))
                    ids = rng.sample(sorted(live), k)
                    pool.free(ids)
                    for i in ids:
                        live.remove(i)
                        free.append(i)
                else:
                    # invalid frees change nothing
                    cand = rng.choice([[-1], [N], list(live)[:1] * 2, [i for i in range(N) if i not in live][:1]])
                    if not cand or (len(cand) == 1 and cand[0] in live):
                        continue
                    with pytest.raises(fp8kv.Fp8kvError):
                        pool.free(cand)
            assert pool.num_free == len(free)
            assert all(int(pool.tag(i)) == tags[i] for i in range(N))
        pool.close()


def test_pool_create_rejects_bad_size():
    with pytest.raises(fp8kv.Fp8kvError):
        fp8kv.Pool(0)


def _check(pool, reqs, P):
    """Run the oracle's tag check for a list of (pages, tags, ctx_len)."""
    B = len(reqs)
    pt = np.full((B, P), -1, np.int32)
    et = np.zeros((B, P), np.uint32)
    cl = np.zeros(B, np.int32)
    for b, (pages, tg, ctx) in enumerate(reqs):
        pt[b, :len(pages)] = pages
        et[b, :len(tg)] = tg
        cl[b] = ctx
    return oracle.verify(pt, et, cl, pool.tags())


def test_fault_injection_scenarios():
    pool = fp8kv.Pool(64, seed=5)
    a_ids, a_tags = pool.alloc(4)      # request A: 4 pages (up to 64 tokens)
    b_ids, b_tags = pool.alloc(3)      # request B
    reqs = [(a_ids, a_tags, 60), (b_ids, b_tags, 40)]
    assert (_check(pool, reqs, 4) == [0, 0]).all()

    # cancellation of B: its pages go back; nothing about A changes
    pool.free(b_ids)
    assert (_check(pool, [reqs[0]], 4) == [0]).all()

    # page reclamation: A's last page is reclaimed and handed to request C
    pool.free(a_ids[3:])
    _ = pool.alloc(pool.num_free - 1)   # drain the free list down to A's old page
    c_ids, c_tags = pool.alloc(1)
    assert c_ids[0] == a_ids[3]         # FIFO: A's page was the last one freed
    # A still believes it owns the page: stale tag -> A aborts, C is fine
    ab = _check(pool, [(a_ids, a_tags, 60), (c_ids, c_tags, 10)], 4)
    assert list(ab) == [1, 0]
    # ... but only if A actually reads that page this step
    ab = _check(pool, [(a_ids, a_tags, 48), (c_ids, c_tags, 10)], 4)
    assert list(ab) == [0, 0]

    # batch reordering does not change which request aborts
    ab = _check(pool, [(c_ids, c_tags, 10), (a_ids, a_tags, 60)], 4)
    assert list(ab) == [0, 1]

    # concurrent release of a page two requests both think they hold
    pool.free(c_ids)
    d_ids, d_tags = pool.alloc(1)
    assert d_ids[0] == c_ids[0] and d_tags[0] == c_tags[0] + 1
    ab = _check(pool, [(c_ids, c_tags, 5), (d_ids, d_tags, 5), (a_ids[:1], a_tags[:1], 16)], 4)
    assert list(ab) == [1, 0, 0]


def test_tag_wraps_around():
    pool = fp8kv.Pool(1, seed=0)
    t0 = int(pool.tags()[0])
    for k in range(5):
        ids, tg = pool.alloc(1)
        assert int(tg[0]) == (t0 + k + 1) & 0xFFFFFFFF
        pool.free(ids)


def test_random_alloc_share_free_against_model():
    """Reference counts: a page returns to the free list when its last holder
    frees it; sharing never changes a tag; only re-allocation does."""
    rng = random.Random(7)
    for trial in range(20):
        N = rng.randint(1, 40)
        pool = fp8kv.Pool(N, seed=100 + trial)
        tags = {i: int(t) for i, t in enumerate(pool.tags())}
        refs = {i: 0 for i in range(N)}
        free = list(range(N))
        for step in range(400):
            op = rng.random()
            held = [i for i in range(N) if refs[i] > 0]
            if op < 0.35:
                n = rng.randint(0, 4)
                if n > len(free):
                    with pytest.raises(fp8kv.Fp8kvError):
                        pool.alloc(n)
                    continue
                ids, tg = pool.alloc(n)
                assert list(ids) == free[:n]
                del free[:n]
                for i, t in zip(ids, tg):
                    tags[int(i)] = (tags[int(i)] + 1) & 0xFFFFFFFF
                    refs[int(i)] = 1
                    assert int(t) == tags[int(i)]
            elif op < 0.65 and held:
                ids = rng.sample(held, rng.randint(1, len(held)))
                got = pool.share(ids)
                for i, t in zip(ids, got):
                    refs[i] += 1
                    assert int(t) == tags[i]            # same tag for the new holder
            elif held and rng.random() < 0.85:
                ids = rng.sample(held, rng.randint(1, len(held)))
                pool.free(ids)
                for i in ids:
                    refs[i] -= 1
                    if refs[i] == 0:
                        free.append(i)
            else:
                bad = rng.choice([[-1], [N], [i for i in range(N) if refs[i] == 0][:1],
                                  held[:1] * 2])
                if not bad or (len(bad) == 1 and 0 <= bad[0] < N and refs[bad[0]] > 0):
                    continue
                before = [pool.refcount(i) for i in range(N)]
                with pytest.raises(fp8kv.Fp8kvError):
                    (pool.share if rng.random() < 0.5 else pool.free)(bad)
                assert [pool.refcount(i) for i in range(N)] == before   # all-or-nothing
            assert pool.num_free == len(free)
            assert all(pool.refcount(i) == refs[i] for i in range(N))
            assert all(int(pool.tag(i)) == tags[i] for i in range(N))
        pool.close()


def test_shared_prefix_isolation():
    """Two requests share a prefix; cancelling one leaves the other valid; once
    the last holder is gone the page is reissued with a new tag and any stale
    holder aborts while the new owner does not."""
    pool = fp8kv.Pool(16, seed=9)
    pre_ids, pre_tags = pool.alloc(2)                 # request A: prefix (2 full pages)
    a_tail, a_ttag = pool.alloc(1)                    # ... and its own last page
    b_tags = pool.share(pre_ids)                      # request B maps the same prefix
    assert (b_tags == pre_tags).all()
    b_tail, b_ttag = pool.alloc(1)
    A = (np.r_[pre_ids, a_tail], np.r_[pre_tags, a_ttag], 40)
    B = (np.r_[pre_ids, b_tail], np.r_[b_tags, b_ttag], 36)
    assert list(_check(pool, [A, B], 3)) == [0, 0]
    # A is cancelled: its pages are released, the shared ones stay with B
    pool.free(np.r_[pre_ids, a_tail])
    assert [pool.refcount(int(i)) for i in pre_ids] == [1, 1]
    assert list(_check(pool, [B], 3)) == [0]
    # B finishes too: the prefix pages go back to the pool ...
    pool.free(np.r_[pre_ids, b_tail])
    assert pool.num_free == 16
    # ... and are handed out again with new tags (FIFO: drain down to them)
    pool.alloc(pool.num_free - 4)
    c_ids, c_tags = pool.alloc(4)
    assert set(int(i) for i in pre_ids) <= set(int(i) for i in c_ids)
    C = (c_ids[:3], c_tags[:3], 48)
    # a holder that kept its old view of the prefix is caught; the new owner is not
    assert list(_check(pool, [B, C], 3)) == [1, 0]
