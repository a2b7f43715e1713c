"""GPU: the multi-step decode loop (prompt in the cache, one token per step,
a page taken from the pool every 16 tokens) against the oracle replaying the
same token streams.

Cache bytes of every page a request holds must match bit for bit after the
run; the last step's output within the f32 tolerance; the no-op tracker gives
the same bits as the tracker; a request whose remembered tag goes stale is
aborted at the next step and retired while the others continue exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from _helpers import SM_SCALE, check_outputs, unswizzle
from workloads import bf16_bits_to_f32, scales_from_amax
from workloads.decode_loop import token_bits

pytestmark = pytest.mark.gpu

B, P, T, HQ, HKV, SEED = 3, 37, 20, 8, 2, 11   # positions 37..56: pages open at 48


@pytest.fixture(scope="module")
def fp8kv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_paged_fp8kv_amd as m
    return m


def _loop(fp8kv, tracker):
    from workloads.decode_loop import DecodeLoop
    return DecodeLoop(B, P, T, HQ, HKV, tracker=tracker, seed=SEED, out_dtype=fp8kv.OUT_F32)


def _tokens(which, b, n):
    return token_bits(SEED, which, b, 0, n, HKV)


def _scales(which):
    am = np.zeros(HKV, np.float32)
    for b in range(B):
        x = bf16_bits_to_f32(_tokens(which, b, P + T))
        am = np.maximum(am, np.abs(x).max(axis=(0, 2)))
    return scales_from_amax(am)


def _oracle_run(loop, upto, live):
    """Oracle caches after `upto` steps for the live requests, with the loop's
    page table (ids and their order come from the pool, not from the GPU's
    arithmetic)."""
    ks, vs = _scales("k"), _scales("v")
    K, V = oracle.new_cache(loop.num_pages, HKV)
    pt = loop.pt_host.numpy().copy()
    for b in range(B):
        if not live[b]:
            continue
        n = P + upto
        oracle.append(K, V, ks, vs, _tokens("k", b, n), _tokens("v", b, n),
                      np.full(n, b, np.int32), np.arange(n, dtype=np.int32), pt)
    return K, V, ks, vs, pt


def _check_cache(loop, K, V, live):
    kh = loop.K.cpu().numpy()
    vh = loop.V.cpu().numpy()
    for b in range(B):
        if not live[b]:
            continue
        pages = loop.pages[b]
        assert (unswizzle(kh, HKV, 0, pages, False) == K[pages]).all(), b
        assert (unswizzle(vh, HKV, 0, pages, True) == V[pages]).all(), b


def test_loop_matches_oracle(fp8kv):
    loop = _loop(fp8kv, tracker=True)
    assert np.array_equal(loop.k_scale.cpu().numpy(), _scales("k"))
    assert np.array_equal(loop.v_scale.cpu().numpy(), _scales("v"))
    loop.run()
    assert all(len(p) == -(-(P + T) // 16) for p in loop.pages)
    assert loop.abort.cpu().numpy().sum() == 0
    K, V, ks, vs, pt = _oracle_run(loop, T, [True] * B)
    _check_cache(loop, K, V, [True] * B)
    q = np.stack([token_bits(SEED, "q", b, T - 1, T, HQ)[0] for b in range(B)])
    ref, _ = oracle.attention(K, V, ks, vs, q, pt, np.full(B, P + T, np.int32), SM_SCALE)
    out = loop.out.cpu().numpy()
    err = check_outputs(out, None, ref)
    print(f"loop B={B} P={P} T={T}: max abs err {err:.3e}")
    # the tags that went up with the tables are the pool's
    assert np.array_equal(loop.tags.cpu().numpy().view(np.uint32), loop.pool.tags())
    loop.close()


def test_noop_tracker_gives_the_same_bits(fp8kv):
    on, off = _loop(fp8kv, True), _loop(fp8kv, False)
    for _ in range(T):
        on.step()
        off.step()
        assert torch.equal(on.out, off.out)
    assert all(a == b for a, b in zip(on.pages, off.pages))
    assert torch.equal(on.K, off.K) and torch.equal(on.V, off.V)
    on.close()
    off.close()


def test_stale_tag_aborts_only_that_request(fp8kv):
    loop = _loop(fp8kv, tracker=True)
    loop.run(6)
    free_before = loop.pool.num_free
    held = len(loop.pages[1])
    loop.corrupt_expected(1, 0)
    loop.step()                                    # step 6 (position 43): request 1 aborts
    ab = loop.abort.cpu().numpy()
    assert list(ab) == [0, 1, 0]
    assert not loop.live[1] and loop.pool.num_free == free_before + held
    assert (loop.out[1] == 0).all()
    loop.run(T - 7)                                # the others run to the end
    assert loop.live == [True, False, True]
    live = [True, False, True]
    K, V, ks, vs, pt = _oracle_run(loop, T, live)
    _check_cache(loop, K, V, live)
    q = np.stack([token_bits(SEED, "q", b, T - 1, T, HQ)[0] for b in range(B)])
    cl = np.array([P + T, 0, P + T], np.int32)
    ref, _ = oracle.attention(K, V, ks, vs, q, pt, cl, SM_SCALE,
                              abort=np.array([0, 1, 0], np.uint8))
    out = loop.out.cpu().numpy()
    assert (out[1] == 0).all()
    check_outputs(out[[0, 2]], None, ref[[0, 2]])
    loop.close()


def test_page_reclaimed_through_the_pool_aborts_its_holder(fp8kv):
    """The pool gives one of request 0's prompt pages to another holder (its
    tag changes); the new tag reaches the device with the tables and the next
    step aborts request 0 only; the page stays with its new holder."""
    loop = _loop(fp8kv, tracker=True)
    loop.run(4)
    pid = loop.pages[0][1]
    old_tag = loop.pool.tag(pid)
    loop.reclaim(0, 1)
    assert loop.pool.tag(pid) != old_tag and loop.pool.refcount(pid) == 1
    assert np.array_equal(loop.tags.cpu().numpy().view(np.uint32), loop.pool.tags())
    loop.step()
    assert list(loop.abort.cpu().numpy()) == [1, 0, 0]
    assert loop.live == [False, True, True] and loop.pool.refcount(pid) == 1
    assert (loop.out[0] == 0).all()
    loop.run(T - 5)
    live = [False, True, True]
    K, V, ks, vs, pt = _oracle_run(loop, T, live)
    _check_cache(loop, K, V, live)
    q = np.stack([token_bits(SEED, "q", b, T - 1, T, HQ)[0] for b in range(B)])
    cl = np.array([0, P + T, P + T], np.int32)
    ref, _ = oracle.attention(K, V, ks, vs, q, pt, cl, SM_SCALE,
                              abort=np.array([1, 0, 0], np.uint8))
    out = loop.out.cpu().numpy()
    assert (out[0] == 0).all()
    check_outputs(out[[1, 2]], None, ref[[1, 2]])
    loop.close()


def test_layers_share_the_page_table(fp8kv):
    """Two layers: one tag check per step, append and attention per layer, each
    layer's pool addressed by the same page ids (same inputs, so both caches
    and the last layer's output match the single-layer oracle)."""
    from workloads.decode_loop import DecodeLoop
    loop = DecodeLoop(B, P, T, HQ, HKV, tracker=True, seed=SEED, out_dtype=fp8kv.OUT_F32,
                      layers=2)
    loop.run()
    K, V, ks, vs, pt = _oracle_run(loop, T, [True] * B)
    for layer in range(2):
        loop.K, loop.V = loop.Ks[layer], loop.Vs[layer]
        _check_cache(loop, K, V, [True] * B)
    q = np.stack([token_bits(SEED, "q", b, T - 1, T, HQ)[0] for b in range(B)])
    ref, _ = oracle.attention(K, V, ks, vs, q, pt, np.full(B, P + T, np.int32), SM_SCALE)
    check_outputs(loop.out.cpu().numpy(), None, ref)
    loop.close()


def _pair(fp8kv, tracker, layers=2):
    from workloads.decode_loop import DecodeLoop
    return [DecodeLoop(B, P, T, HQ, HKV, tracker=tracker, seed=SEED, out_dtype=fp8kv.OUT_F32,
                       layers=layers, graph=g) for g in (False, True)]


def _same_state(a, b):
    assert all(x == y for x, y in zip(a.pages, b.pages))
    for ka, kb, va, vb in zip(a.Ks, b.Ks, a.Vs, b.Vs):
        assert torch.equal(ka, kb) and torch.equal(va, vb)
    assert torch.equal(a.abort, b.abort)


@pytest.mark.parametrize("tracker", [True, False])
def test_graph_replay_gives_the_eager_bits(fp8kv, tracker):
    """Every step replays a captured graph (two layers); each replay's output,
    with the loop's eager host work in between, equals the eager step's."""
    eager, graph = _pair(fp8kv, tracker)
    for s in range(T):
        eager.step()
        graph.step()
        assert torch.equal(eager.out, graph.out), s
    _same_state(eager, graph)
    eager.close()
    graph.close()


def test_graph_replay_stale_tag(fp8kv):
    """A stale remembered tag aborts the request under graph replay too; the
    retired request's lengths and table are changed in device memory that the
    graph reads, and the other requests continue with the eager bits."""
    eager, graph = _pair(fp8kv, True)
    for lp in (eager, graph):
        lp.run(6)
        lp.corrupt_expected(1, 0)
        lp.step()
    assert list(graph.abort.cpu().numpy()) == [0, 1, 0]
    assert graph.live == [True, False, True]
    for s in range(T - 7):
        eager.step()
        graph.step()
        assert torch.equal(eager.out, graph.out), s
    assert (graph.out[1] == 0).all()
    _same_state(eager, graph)
    eager.close()
    graph.close()
