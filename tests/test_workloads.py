"""The seeded input generators: both backends agree bit for bit, and the
workloads have the stated shapes, lengths and integrity faults (CPU only)."""
import numpy as np
import torch

import workloads


def test_backends_bit_identical():
    for outl in (0, 66):
        for key in (1, 0xDEADBEEF, 2 ** 32 - 1):
            a = workloads.draw_bits(key, 12345, 50_000, "numpy", outlier_per_65536=outl)
            b = workloads.draw_bits(key, 12345, 50_000, "torch", "cpu", outlier_per_65536=outl)
            assert (a.view(np.int16) == b.numpy()).all()


def test_host_backend_matches_numpy():
    """The C backend (full-size oracle inputs) against the numpy definition:
    keys across the 32-bit range, counters that wrap past 2^32, outliers."""
    rng = np.random.default_rng(5)
    cases = [(1, 0, 10), (0xDEADBEEF, 12345, 70_001), (2 ** 32 - 1, 2 ** 32 - 5000, 9_000),
             (7, 3 * 2 ** 31, 4_096)]
    cases += [(int(rng.integers(0, 2 ** 32)), int(rng.integers(0, 2 ** 34)),
               int(rng.integers(1, 200_000))) for _ in range(12)]
    for key, start, count in cases:
        for outl, ob in ((0, workloads.BF16_20), (66, workloads.BF16_20), (4000, workloads.BF16_25)):
            a = workloads.draw_bits(key, start, count, "numpy", outlier_per_65536=outl,
                                    outlier_bits=ob)
            b = workloads.draw_bits(key, start, count, "host", outlier_per_65536=outl,
                                    outlier_bits=ob)
            assert a.dtype == b.dtype == np.uint16 and (a == b).all(), (key, start, count, outl)
    w = workloads.make(4, batch=2)
    L = int(w.ctx_before[1])
    for which in "kv":
        assert (w.kv_tokens(which, 1, L - 40, L + 1) ==
                w.kv_tokens(which, 1, L - 40, L + 1, backend="host")).all()
    s = workloads.shared_prompts([(3, 64)], plain=2)
    for b in range(s.B):
        n = int(s.ctx_before[b]) + 1
        assert (s.kv_tokens("k", b, 0, n) == s.kv_tokens("k", b, 0, n, backend="host")).all()


def test_workload_streams_bit_identical():
    w = workloads.make(4, batch=1)
    L = int(w.ctx_before[0])
    a = w.kv_tokens("k", 0, L - 20, L + 1)
    b = w.kv_tokens("k", 0, L - 20, L + 1, backend="torch", device="cpu")
    assert (a.view(np.int16) == b.numpy()).all()
    assert (w.q_bits().view(np.int16) == w.q_bits("torch", "cpu").numpy()).all()
    # saturating values sit on the appended token only
    f = workloads.bf16_bits_to_f32(a)
    assert np.abs(f[-1]).max() == 25.0 and np.abs(f[:-1]).max() <= 20.0


def test_distribution_is_roughly_standard_normal():
    x = workloads.bf16_bits_to_f32(workloads.draw_bits(77, 0, 1_000_000))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01


def test_configs():
    w1 = workloads.make(1)
    assert (w1.ctx_before == [17, 64, 100, 256]).all() and w1.num_pages == 64
    assert (w1.n_pages == [2, 5, 7, 17]).all() and w1.G == 4
    w3 = workloads.make(3)
    assert w3.B == 64 and w3.ctx_before.min() >= 1024 and w3.ctx_before.max() <= 32768
    assert w3.num_pages == int(w3.n_pages.sum())
    used = w3.page_table[w3.page_table >= 0]
    assert np.unique(used).size == used.size == w3.num_pages
    assert (w3.expected_abort == 0).all()
    w5 = workloads.make(5)
    assert w5.num_pages == 81250 and w5.Hq == 32 and w5.Hkv == 4
    frac = w5.stale.sum() / (w5.page_table >= 0).sum()
    assert abs(frac - 0.01) < 1e-4
    ab = w5.expected_abort
    assert 0.5 < ab.mean() < 0.95
    w5r = workloads.make(5, stale_mode="requests")
    assert w5r.expected_abort.sum() == round(0.01 * 256)


def test_scales_recipe():
    s = workloads.scales_from_amax(np.array([448.0, 0.0, 20.0], np.float32))
    assert s[0] == 1.0 and s[1] == 1.0 and s[2] == np.float32(20.0) / np.float32(448.0)


def test_keys_independent_of_integer_type():
    assert workloads.stream_key(np.int64(3), 2, np.int64(63)) == workloads.stream_key(3, 2, 63)
    w = workloads.make(1)
    a = w.kv_tokens("k", np.int64(2), 0, 5)
    b = w.kv_tokens("k", 2, 0, 5)
    assert (a == b).all()


def test_head_slice_generator_matches():
    for cfg in (1, 4):
        w = workloads.make(cfg, batch=2)
        L = int(w.ctx_before[1])
        full = w.kv_tokens("v", 1, max(0, L - 40), L + 1)
        for g in range(w.Hkv):
            assert (w.kv_tokens_head("v", 1, max(0, L - 40), L + 1, g) == full[:, g, :]).all()


def test_loop_token_streams_slice_and_backends_agree():
    import torch
    from workloads.decode_loop import token_bits
    full = token_bits(3, "k", 2, 0, 40, 4)
    part = token_bits(3, "k", 2, 17, 29, 4)
    assert full.shape == (40, 4, 128) and (full[17:29] == part).all()
    dev = token_bits(3, "k", 2, 17, 29, 4, "torch", "cpu")
    assert (dev.numpy().view(np.uint16) == part).all()
    # requests and tensors draw different streams
    assert not (token_bits(3, "k", 1, 0, 4, 4) == full[:4]).all()
    assert not (token_bits(3, "v", 2, 0, 4, 4) == full[:4]).all()


def test_multi_query_stream():
    """Speculative-verification queries: both backends agree, the newest query is
    the one-token step's Q, and the older ones continue the same Q stream."""
    w = workloads.make(1)
    q = w.q_bits_multi(3)
    assert q.shape == (w.B, 3, w.Hq, w.D)
    assert (q.view(np.int16) == w.q_bits_multi(3, "torch", "cpu").numpy()).all()
    assert (q[:, 2] == w.q_bits()).all()
    assert (q[:, :2] == w.q_bits_multi(3)[:, :2]).all()
    assert not (q[:, 0] == q[:, 2]).all()


def test_shared_prompt_workload():
    """A common prompt: one stream for tokens below prefix_len in every request
    (both backends, whole-token and per-head generators), own streams after it;
    shared pages are one set of ids with one tag, the private twin has distinct
    pages and the same lengths."""
    w = workloads.shared_prefix(B=5, prefix_len=48, suffix_max=40, Hq=8, Hkv=2)
    p = workloads.shared_prefix(B=5, prefix_len=48, suffix_max=40, Hq=8, Hkv=2, shared=False)
    assert (w.ctx_before == p.ctx_before).all() and (w.ctx_before >= 48 + 16).all()
    assert (w.page_table[:, :3] == w.page_table[0, :3]).all()
    assert (w.expected_tags[:, :3] == w.expected_tags[0, :3]).all()
    used = w.page_table[w.page_table >= 0]
    assert len(np.unique(used)) == w.num_pages == 3 + int((w.n_pages - 3).sum())
    pu = p.page_table[p.page_table >= 0]
    assert len(np.unique(pu)) == pu.size == p.num_pages
    assert (w.kv_tokens("v", 0, 0, 48) == w.kv_tokens("v", 4, 0, 48)).all()
    assert not (w.kv_tokens("v", 0, 48, 60) == w.kv_tokens("v", 4, 48, 60)).all()
    full = w.kv_tokens("k", 3, 0, int(w.ctx_lens[3]))
    assert (full == p.kv_tokens("k", 3, 0, int(w.ctx_lens[3]))).all()
    assert (full.view(np.int16) == w.kv_tokens("k", 3, 0, int(w.ctx_lens[3]), "torch", "cpu").numpy()).all()
    assert (w.kv_tokens_head("k", 3, 40, 60, 1) == full[40:60, 1]).all()
