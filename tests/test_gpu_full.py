"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (default decode workers, fused tag check + append).

Every row and every byte: the oracle builds the whole cache of the workload
itself (history and appended token of every request, from the host backend
of the input generator, encoded by the oracle's own encoder), runs the tag
check on the same tables and attends in binary64 for every (request, q-head)
row.  The test then requires
  * abort flags equal for every request;
  * every byte of both pools equal (each page the step reads, and the pages
    nobody reads, which both sides leave zero) -- so an aborted request's new
    token is written nowhere;
  * every output row within the tolerance of the 2e-3 bound (f32 rows, and
    bf16 rows as their round-to-nearest-even), aborted rows +0 bit for bit;
and prints the largest error and the number of bf16 elements that differ
from the oracle's own bf16 rounding.

Aborting a request must leave every other request of the batch exact (the
commentary page "Kimi and GLM Reasoning Slimming: Hands-On Test", section
"What Developers Should Learn from This", item 4): the capacity workloads
check the surviving rows against an oracle that never saw the aborted ones'
new tokens, and a ragged batch with one planted stale tag is compared the
same way.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import SM_SCALE, bf16_differences, check_outputs, tile_index

pytestmark = pytest.mark.gpu

PAGES_PER_CHUNK = 4096


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from workloads import device
    return device


def host_scales(w):
    """The workloads' calibration, on the host: fl32(amax / 448) per kv-head over
    every generated value (history and new token; the saturating overrides of
    the long workload excluded)."""
    # the magnitude bits of non-NaN bf16 values order as the magnitudes do
    am = {"k": np.zeros(w.Hkv, np.uint16), "v": np.zeros(w.Hkv, np.uint16)}
    for b in range(w.B):
        n = int(w.ctx_before[b]) + 1
        for which in "kv":
            x = w.kv_tokens(which, b, 0, n, backend="host", with_saturation=False)
            am[which] = np.maximum(am[which], (x & np.uint16(0x7FFF)).max(axis=(0, 2)))
    return tuple(workloads.scales_from_amax(workloads.bf16_bits_to_f32(am[c])) for c in "kv")


def oracle_cache(w, ks, vs, cache_dtype, abort):
    """The oracle's logical K/V pools after the step: every request's history
    (written before the step, aborted or not) and the new token of every
    request the check let through."""
    K, V = oracle.new_cache(w.num_pages, w.Hkv, cache_dtype)
    for b in range(w.B):
        L = int(w.ctx_before[b])
        kb = w.kv_tokens("k", b, 0, L + 1, backend="host")
        vb = w.kv_tokens("v", b, 0, L + 1, backend="host")
        if L > 0:
            oracle.append(K, V, ks, vs, kb[:L], vb[:L], np.full(L, b, np.int32),
                          np.arange(L, dtype=np.int32), w.page_table, cache_dtype=cache_dtype)
        oracle.append(K, V, ks, vs, kb[L:], vb[L:], np.array([b], np.int32),
                      np.array([L], np.int32), w.page_table, abort=abort,
                      cache_dtype=cache_dtype)
    return K, V


def compare_pools(st, K, V):
    """Every byte of the device pools against the oracle's logical pools."""
    w = st.w
    eb = 1 if st.cache_dtype == 0 else 2
    dt = np.uint8 if eb == 1 else np.uint16
    te = 16 * 128
    for X, ref, is_v in ((st.K, K, False), (st.V, V, True)):
        dev = _host(X).view(dt).reshape(w.num_pages, w.Hkv, te)
        idx = tile_index(is_v, eb).ravel()
        for p0 in range(0, w.num_pages, PAGES_PER_CHUNK):
            p1 = min(w.num_pages, p0 + PAGES_PER_CHUNK)
            got = np.take(dev[p0:p1], idx, axis=2)
            exp = ref[p0:p1].reshape(p1 - p0, w.Hkv, te)
            if not np.array_equal(got, exp):
                bad = np.argwhere(got != exp)[0]
                raise AssertionError(f"{'V' if is_v else 'K'} pool differs at page "
                                     f"{p0 + bad[0]}, kv-head {bad[1]}, element {bad[2]}")


def full_check(st, expected_abort=None, label=""):
    """One step on the device, then the oracle over the whole workload."""
    import decode_attention_paged_fp8kv_amd as fp8kv
    w = st.w
    out16 = _host(st.step(check_tags=True).view(torch.int16)).copy()
    out32 = _host(st.decode(out_dtype=fp8kv.OUT_F32)).copy()
    ab = _host(st.abort).copy()
    etag = _host(st.expected_tags).view(np.uint32)
    tags = _host(st.pool_tags).view(np.uint32)
    exp_ab = oracle.verify(w.page_table, etag, w.ctx_lens, tags)
    assert (ab == exp_ab).all(), f"abort flags differ at {np.flatnonzero(ab != exp_ab)[:8]}"
    if expected_abort is not None:
        assert (exp_ab == expected_abort).all()
    ks, vs = host_scales(w)
    assert (ks == st.k_scale_host).all() and (vs == st.v_scale_host).all()
    K, V = oracle_cache(w, ks, vs, st.cache_dtype, exp_ab)
    compare_pools(st, K, V)
    ref64, ref16 = oracle.attention(K, V, ks, vs, w.q_bits(), w.page_table, w.ctx_lens,
                                    SM_SCALE, abort=exp_ab, cache_dtype=st.cache_dtype)
    dead = exp_ab == 1
    assert (out32[dead].view(np.uint32) == 0).all() and (out16[dead] == 0).all()
    err = check_outputs(out32, out16, ref64)
    nd = bf16_differences(out16, ref16)
    print(f"{w.name}{label}: {w.B - int(dead.sum())}/{w.B} requests live, "
          f"{int(w.ctx_lens[~dead].sum())} tokens; {w.num_pages} pages x {w.Hkv} heads "
          f"bit-exact; max abs err (f32) {err:.3e}; bf16 elements differing from the "
          f"oracle's rounding: {nd} of {out16.size}", flush=True)
    return exp_ab


def test_uniform_32x8192_e4m3(dev):
    st = dev.build(workloads.make(2))
    ab = full_check(st)
    assert (ab == 0).all()


def test_uniform_32x8192_bf16_cache(dev):
    st = dev.build(workloads.make(2), cache_dtype=1)
    ab = full_check(st, label=" (bf16 cache)")
    assert (ab == 0).all()


def test_ragged_64(dev):
    st = dev.build(workloads.make(3))
    ab = full_check(st)
    assert (ab == 0).all()


def test_ragged_64_one_stale_tag(dev):
    """One request's expected tag made stale in its last page (the page that
    receives its new token): it aborts, writes nothing, gives +0 rows, and the
    63 others stay exact."""
    w = workloads.make(3)
    st = dev.build(w)
    b = 17
    i = int(w.n_pages[b]) - 1
    etag = w.expected_tags.copy()
    etag[b, i] ^= 1
    st.expected_tags.copy_(torch.from_numpy(etag.view(np.int32)).to(st.expected_tags.device))
    exp = np.zeros(w.B, np.uint8)
    exp[b] = 1
    full_check(st, expected_abort=exp, label=" (request 17 stale)")


def test_long_4x131072_outliers_saturation(dev):
    w = workloads.make(4)
    st = dev.build(w)
    full_check(st)
    # the appended token's +-25 values saturate to +-448 * scale (codes 0x7E / 0xFE)
    idx = tile_index(False, 1)
    K = _host(st.K).reshape(w.num_pages, w.Hkv, -1)
    for b in range(w.B):
        L = int(w.ctx_before[b])
        tile = K[w.page_table[b, L // 16], 0][idx[L % 16]]
        assert tile[5] == 0x7E and tile[40] == 0xFE and tile[77] == 0x7E and tile[120] == 0xFE


@pytest.mark.parametrize("mode", ["entries", "requests"])
def test_capacity_256_stale_tags(dev, mode):
    w = workloads.make(5, stale_mode=mode)
    st = dev.build(w)
    ab = full_check(st, expected_abort=w.expected_abort, label=f" ({mode})")
    assert 0 < ab.sum() < w.B


def test_capacity_256_stale_through_the_pool(dev):
    """Staleness made the way a server makes it: every page handed out by the
    library's pool, the stale pages freed and handed out again (their tags move
    on), the requests keeping the tags they recorded; the device tags are
    uploaded by the pool's own sync.  The oracle's inputs are the pool model
    (a page's tag goes up by one on each allocation), checked against the pool."""
    import decode_attention_paged_fp8kv_amd as fp8kv
    w = workloads.make(5)
    st = dev.build(w)
    pool = fp8kv.Pool(w.num_pages, seed=55)
    tags0 = pool.tags()
    ids, tags1 = pool.alloc(w.num_pages)
    assert (ids == np.arange(w.num_pages)).all()
    assert (tags1 == tags0 + np.uint32(1)).all()
    used = w.page_table >= 0
    etag = np.zeros(w.page_table.shape, np.uint32)
    etag[used] = tags1[w.page_table[used]]
    stale_pages = w.page_table[w.stale]
    pool.free(stale_pages)                    # the pages go back ...
    ids2, tags2 = pool.alloc(stale_pages.size)  # ... and to someone else
    assert (ids2 == stale_pages).all()
    model = tags1.copy()
    model[stale_pages] += np.uint32(1)
    assert (pool.tags() == model).all() and (tags2 == model[stale_pages]).all()
    st.expected_tags.copy_(torch.from_numpy(etag.view(np.int32)).to(st.expected_tags.device))
    pool.sync(st.pool_tags)
    torch.cuda.synchronize()
    assert (_host(st.pool_tags).view(np.uint32) == model).all()
    assert (oracle.verify(w.page_table, etag, w.ctx_lens, model) == w.expected_abort).all()
    full_check(st, expected_abort=w.expected_abort, label=" (stale through the pool)")
    pool.close()
