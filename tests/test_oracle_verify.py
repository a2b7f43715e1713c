"""Pins for the oracle's page-tag check (CPU only).

The check is pinned by (a) hand cases written from the rule of the
commentary page's section "Giving Every Physical Cache Page a 'Generation
Number'" (tests/golden/verify_cases.txt) and (b) the same rule restated as a
set comparison, run on random cases with stale entries planted.  The rule: a
request may go on only if every page it expects to read still carries the
tag the request recorded for it; any other case (a changed tag, a page id
the allocator does not know) aborts the request.
"""
import os

import numpy as np

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden", "verify_cases.txt")


def _load_cases():
    pool = None
    cases = []
    for line in open(GOLD):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("pool"):
            pool = {int(k): int(v) for k, v in (t.split(":") for t in line.split()[1:])}
            continue
        name, ctx, ids, tags, exp = [t.strip() for t in line.split("|")]
        cases.append((name, int(ctx), [int(x) for x in ids.split()],
                      [int(x) for x in tags.split()], int(exp)))
    return pool, cases


def test_golden_hand_cases():
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
    # the "len_exceeds_tbl" case needs its table row to be exactly 2 wide;
    # check each case on its own table of its own width too.
    got = oracle.verify(pt, et, cl, tags)
    for b, (name, ctx, ids, tg, exp) in enumerate(cases):
        row = oracle.verify(np.array([ids], np.int32), np.array([tg], np.uint32),
                            np.array([ctx], np.int32), tags)
        assert row[0] == exp, name
        if name != "len_exceeds_tbl":
            assert got[b] == exp, name


def restated_rule(request_pages, current_tags: dict) -> int:
    """1 if the request must abort: the (page id, recorded tag) pairs it expects
    are not all among the allocator's (page id, current tag) pairs."""
    expected = set(request_pages)
    known = {(pid, current_tags[pid]) for pid, _ in expected if pid in current_tags}
    return 0 if expected <= known else 1


def test_matches_restated_rule_random():
    rng = np.random.default_rng(3)
    for trial in range(40):
        N = int(rng.integers(1, 300))
        tags = rng.integers(0, 2 ** 32, N, dtype=np.uint64).astype(np.uint32)
        B = int(rng.integers(1, 20))
        P = int(rng.integers(1, 12))
        pt = rng.integers(-2, N + 2, size=(B, P)).astype(np.int32)
        et = np.where((pt >= 0) & (pt < N), tags[np.clip(pt, 0, N - 1)], 0).astype(np.uint32)
        flip = rng.random((B, P)) < 0.05
        et = np.where(flip, et + np.uint32(1), et).astype(np.uint32)
        cl = rng.integers(0, P * 16 + 1, B).astype(np.int32)
        got = oracle.verify(pt, et, cl, tags)

        current = {i: int(tags[i]) for i in range(N)}
        for b in range(B):
            n = (int(cl[b]) + 15) // 16
            pages = [(int(pt[b, i]), int(et[b, i])) for i in range(n)]
            assert got[b] == restated_rule(pages, current), (trial, b)


def test_workload_stale_entries_abort_exactly():
    w = workloads.make(5, batch=64)
    got = oracle.verify(w.page_table, w.expected_tags, w.ctx_lens, w.pool_tags)
    assert (got == w.expected_abort).all()
    assert 0 < got.sum() < w.B


def test_all_valid_workloads_pass():
    for cfg in (1,):
        w = workloads.make(cfg)
        got = oracle.verify(w.page_table, w.expected_tags, w.ctx_lens, w.pool_tags)
        assert (got == 0).all()
