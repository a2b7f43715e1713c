"""Pins for the oracle's quantize-on-append (CPU only).

  * every written byte equals E(fl32(x / scale)) with E the independent
    bit-level encoder of test_oracle_e4m3 and numpy's binary32 division
    (IEEE correctly rounded) -- the definition, computed another way;
  * closed form: x = DEC(c) * 2^k with scale 2^k re-encodes to c;
  * aborted requests, invalid page entries and tokens outside the table
    write nothing;
  * a BF16 cache stores the input bits unchanged.
"""
import numpy as np

import oracle
import workloads
from test_oracle_e4m3 import bitlevel_encode


def _one_step_inputs(seed=0, B=3, Hkv=2, N=12, D=128, S=16):
    rng = np.random.default_rng(seed)
    L = np.array([5, 16, 31][:B], np.int32)
    pt = np.full((B, 4), -1, np.int32)
    perm = rng.permutation(N).astype(np.int32)
    k = 0
    for b in range(B):
        n = (int(L[b]) + 1 + S - 1) // S
        pt[b, :n] = perm[k:k + n]
        k += n
    kn = workloads.draw_bits(123, 0, B * Hkv * D).reshape(B, Hkv, D)
    vn = workloads.draw_bits(456, 0, B * Hkv * D).reshape(B, Hkv, D)
    return L, pt, kn, vn


def test_append_equals_encoder_elementwise():
    L, pt, kn, vn = _one_step_inputs()
    B, Hkv, D = kn.shape
    ks = np.array([0.0071, 0.013], np.float32)
    vs = np.array([0.0042, 1.0], np.float32)
    K, V = oracle.new_cache(12, Hkv)
    seq = np.arange(B, dtype=np.int32)
    assert oracle.append(K, V, ks, vs, kn, vn, seq, L, pt) == 0
    for b in range(B):
        page, slot = pt[b, L[b] // 16], L[b] % 16
        for h in range(Hkv):
            xk = workloads.bf16_bits_to_f32(kn[b, h]) / ks[h]
            xv = workloads.bf16_bits_to_f32(vn[b, h]) / vs[h]
            assert xk.dtype == np.float32
            assert (K[page, h, slot] == bitlevel_encode(xk)).all()
            assert (V[page, h, slot] == bitlevel_encode(xv)).all()
    # nothing else was written
    written = np.zeros(K.shape[:3], bool)
    for b in range(B):
        written[pt[b, L[b] // 16], :, L[b] % 16] = True
    assert (K[~written] == 0).all() and (V[~written] == 0).all()


def test_closed_form_exact_values_reencode():
    tab = oracle.e4m3_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.int64)
    for k in (-7, 0, 5):
        vals = (tab[codes] * 2.0 ** k).astype(np.float32)   # exact, <= 4 significant bits
        bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
        assert (workloads.bf16_bits_to_f32(bits) == vals).all()
        n = bits.size
        pad = (-n) % 128
        kn = np.concatenate([bits, np.zeros(pad, np.uint16)]).reshape(-1, 1, 128)
        T = kn.shape[0]
        pt = np.arange(T, dtype=np.int32).reshape(T, 1)
        K, V = oracle.new_cache(T, 1)
        sc = np.array([2.0 ** k], np.float32)
        oracle.append(K, V, sc, sc, kn, kn, np.arange(T, dtype=np.int32),
                      np.zeros(T, np.int32), pt)
        got = K[:, 0, 0, :].ravel()[:n]
        exp = codes.astype(np.uint8)
        # -0.0 * 2^k is -0 -> 0x80; +0 -> 0x00
        assert (got == exp).all(), k


def test_abort_and_invalid_entries_skip():
    L, pt, kn, vn = _one_step_inputs()
    B, Hkv, D = kn.shape
    sc = np.ones(Hkv, np.float32)
    K, V = oracle.new_cache(12, Hkv)
    ab = np.array([0, 1, 0], np.uint8)
    pt2 = pt.copy()
    pt2[2, L[2] // 16] = 99                     # out of range: must be skipped
    skipped = oracle.append(K, V, sc, sc, kn, vn, np.arange(B, dtype=np.int32), L, pt2, abort=ab)
    assert skipped == 1
    assert (K[pt[1, L[1] // 16], :, L[1] % 16] == 0).all()   # aborted: untouched
    assert (K[pt[0, L[0] // 16], :, L[0] % 16] != 0).any()   # written
    assert K.sum() == K[pt[0, L[0] // 16]].sum()


def test_tokens_outside_the_table_skip():
    """A token whose request is not a row of the table (negative or past the
    last row) or whose position lies before 0 or past the table's width is
    skipped and counted; the valid tokens are written exactly as alone."""
    L, pt, kn, vn = _one_step_inputs()
    B, Hkv, D = kn.shape
    sc = np.ones(Hkv, np.float32)
    seq = np.array([0, -1, B, 2], np.int32)
    pos = np.array([L[0], 3, 3, 4 * 16], np.int32)       # the last one: past the table
    k4 = np.concatenate([kn, kn[:1]])
    v4 = np.concatenate([vn, vn[:1]])
    K, V = oracle.new_cache(12, Hkv)
    assert oracle.append(K, V, sc, sc, k4, v4, seq, pos, pt) == 3
    K1, V1 = oracle.new_cache(12, Hkv)
    oracle.append(K1, V1, sc, sc, kn[:1], vn[:1], seq[:1], pos[:1], pt)
    assert (K == K1).all() and (V == V1).all()


def test_bf16_cache_copies_bits():
    L, pt, kn, vn = _one_step_inputs()
    B, Hkv, D = kn.shape
    K, V = oracle.new_cache(12, Hkv, cache_dtype=1)
    sc = np.full(Hkv, 3.0, np.float32)
    oracle.append(K, V, sc, sc, kn, vn, np.arange(B, dtype=np.int32), L, pt, cache_dtype=1)
    for b in range(B):
        assert (K[pt[b, L[b] // 16], :, L[b] % 16] == kn[b]).all()
        assert (V[pt[b, L[b] // 16], :, L[b] % 16] == vn[b]).all()


def test_slot_named_twice_keeps_the_later_token():
    """Tokens are written in order: when two tokens name the same slot the
    cache holds the later one (the plain loop's result, whatever the threads)."""
    L, pt, kn, vn = _one_step_inputs()
    B, Hkv, D = kn.shape
    sc = np.ones(Hkv, np.float32)
    seq = np.array([0, 2, 0, 1, 0], np.int32)
    pos = np.array([L[0], L[2], L[0], L[1], L[0]], np.int32)
    kk = np.stack([kn[0], kn[2], kn[1], kn[1], kn[2]])
    vv = np.stack([vn[0], vn[2], vn[1], vn[1], vn[2]])
    K, V = oracle.new_cache(12, Hkv)
    oracle.append(K, V, sc, sc, kk, vv, seq, pos, pt)
    K1, V1 = oracle.new_cache(12, Hkv)
    for t in range(5):   # one token per call: the order is explicit
        oracle.append(K1, V1, sc, sc, kk[t:t + 1], vv[t:t + 1], seq[t:t + 1], pos[t:t + 1], pt)
    assert (K == K1).all() and (V == V1).all()
    page, slot = pt[0, L[0] // 16], L[0] % 16
    for h in range(Hkv):
        assert (K[page, h, slot] == bitlevel_encode(workloads.bf16_bits_to_f32(kn[2, h]))).all()
