"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (default decode workers, fused tag check + append).

The oracle recomputes sampled (request, kv-head) pairs exactly: it regenerates
that head's inputs with the numpy generator, encodes them itself and attends
in binary64.  Cache bytes of the sampled pages must match bit for bit, abort
flags for every request, outputs within the f32/bf16 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import SM_SCALE, check_outputs, tile_index

pytestmark = pytest.mark.gpu


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from workloads import device
    return device


def _oracle_head(w, b, g, ks, vs, cache_dtype, aborted, q):
    """Oracle cache (kv-head g only) and output rows of request b."""
    L = int(w.ctx_before[b])
    K, V = oracle.new_cache(w.num_pages, 1, cache_dtype)
    kb = w.kv_tokens_head("k", b, 0, L + 1, g)[:, None, :]
    vb = w.kv_tokens_head("v", b, 0, L + 1, g)[:, None, :]
    pt = w.page_table[b:b + 1]
    sk, sv = ks[g:g + 1], vs[g:g + 1]
    if L > 0:
        oracle.append(K, V, sk, sv, kb[:L], vb[:L], np.zeros(L, np.int32),
                      np.arange(L, dtype=np.int32), pt, cache_dtype=cache_dtype)
    ab = np.array([1 if aborted else 0], np.uint8)
    oracle.append(K, V, sk, sv, kb[L:], vb[L:], np.zeros(1, np.int32), np.array([L], np.int32),
                  pt, abort=ab, cache_dtype=cache_dtype)
    G = w.G
    out64, _ = oracle.attention(K, V, sk, sv, q[b:b + 1, g * G:(g + 1) * G], pt,
                                w.ctx_lens[b:b + 1], SM_SCALE, abort=ab, cache_dtype=cache_dtype)
    return K, V, out64[0]


def _gpu_tiles(st, pages, g, is_v):
    """Logical [pages][16][128] view of kv-head g of the given pages (GPU bytes)."""
    w = st.w
    eb = 1 if st.cache_dtype == 0 else 2
    X = st.V if is_v else st.K
    tiles = X.view(w.num_pages, w.Hkv, -1)[torch.from_numpy(pages.astype(np.int64)).cuda(), g]
    host = _host(tiles).view(np.uint8 if eb == 1 else np.uint16)
    return host[:, tile_index(is_v, eb)]


def _check_pairs(st, pairs, out32, out16, ab):
    w = st.w
    q = w.q_bits()
    for b, g in pairs:
        K, V, ref = _oracle_head(w, b, g, st.k_scale_host, st.v_scale_host, st.cache_dtype,
                                 bool(ab[b]), q)
        pages = w.page_table[b, : w.n_pages[b]]
        assert (_gpu_tiles(st, pages, g, False) == K[pages, 0]).all(), (b, g)
        assert (_gpu_tiles(st, pages, g, True) == V[pages, 0]).all(), (b, g)
        rows = slice(g * w.G, (g + 1) * w.G)
        err = check_outputs(out32[b, rows], out16[b, rows], ref)
        print(f"{w.name} b={b} g={g} L={int(w.ctx_lens[b])} max abs err {err:.3e}")


def _run(st):
    out16 = _host(st.step(check_tags=True).view(torch.int16)).copy()
    import decode_attention_paged_fp8kv_amd as fp8kv
    out32 = _host(st.decode(out_dtype=fp8kv.OUT_F32)).copy()
    return out32, out16, _host(st.abort).copy()


def test_uniform_32x8192_e4m3(dev):
    w = workloads.make(2)
    st = dev.build(w)
    out32, out16, ab = _run(st)
    assert (ab == 0).all()
    _check_pairs(st, [(0, 3), (17, 6)], out32, out16, ab)


def test_uniform_32x8192_bf16_cache(dev):
    w = workloads.make(2)
    st = dev.build(w, cache_dtype=1)
    out32, out16, ab = _run(st)
    _check_pairs(st, [(5, 2)], out32, out16, ab)


def test_ragged_64(dev):
    w = workloads.make(3)
    st = dev.build(w)
    out32, out16, ab = _run(st)
    assert (ab == 0).all() and np.isfinite(out32).all()
    L = w.ctx_lens
    _check_pairs(st, [(int(L.argmax()), 0), (int(L.argmin()), 7), (11, 4)], out32, out16, ab)


def test_long_4x131072_outliers_saturation(dev):
    w = workloads.make(4)
    st = dev.build(w)
    out32, out16, ab = _run(st)
    assert np.isfinite(out32).all()
    # the appended token's +-25 values saturate to +-448 * scale (codes 0x7E / 0xFE)
    for b in range(w.B):
        L = int(w.ctx_before[b])
        page = np.array([w.page_table[b, L // 16]])
        tile = _gpu_tiles(st, page, 0, False)[0, L % 16]
        assert tile[5] == 0x7E and tile[40] == 0xFE and tile[77] == 0x7E and tile[120] == 0xFE
    _check_pairs(st, [(0, 0), (3, 5)], out32, out16, ab)


@pytest.mark.parametrize("mode", ["entries", "requests"])
def test_capacity_256_stale_tags(dev, mode):
    w = workloads.make(5, stale_mode=mode)
    st = dev.build(w)
    out32, out16, ab = _run(st)
    exp = oracle.verify(w.page_table, w.expected_tags, w.ctx_lens, w.pool_tags)
    assert (ab == exp).all() and (exp == w.expected_abort).all()
    assert (out32[ab == 1] == 0).all() and (out16[ab == 1] == 0).all()
    live = np.flatnonzero(ab == 0)
    L = w.ctx_lens
    pairs = [(int(live[L[live].argmax()]), 1), (int(live[L[live].argmin()]), 3)]
    _check_pairs(st, pairs, out32, out16, ab)
    # an aborted request: its new token was not written
    dead = int(np.flatnonzero(ab == 1)[0])
    Ld = int(w.ctx_before[dead])
    page = np.array([w.page_table[dead, Ld // 16]])
    K, _, _ = _oracle_head(w, dead, 2, st.k_scale_host, st.v_scale_host, 0, True, w.q_bits())
    assert (_gpu_tiles(st, page, 2, False)[0, Ld % 16] == K[page[0], 0, Ld % 16]).all()
