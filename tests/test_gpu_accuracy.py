"""GPU: the FP8-vs-BF16 accuracy study measures quantization error, not
kernel error.

The study (`bench.py --accuracy`) reports the difference between the FP8-cache
and the BF16-cache outputs of the same kernel on the same inputs.  Here, on
inputs small enough for the oracle, each of the two outputs matches the
oracle's binary64 attention over its own cache, so the GPU difference equals
the oracle's difference (the error e4m3 storage adds) up to the two parity
errors; the FP8 error itself is printed.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import SM_SCALE, check_outputs, oracle_state

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,batch", [(1, None), (2, 2), (4, 1)])
def test_fp8_minus_bf16_is_the_quantization_error(cfg, batch):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_paged_fp8kv_amd as fp8kv
    from workloads import device
    w = workloads.make(cfg, batch=batch)
    q = w.q_bits()
    gpu, ref = {}, {}
    for cd in (fp8kv.E4M3, fp8kv.BF16):
        st = device.build(w, cache_dtype=cd)
        st.step(check_tags=True)
        gpu[cd] = st.decode(out_dtype=fp8kv.OUT_F32).cpu().numpy().astype(np.float64)
        K, V = oracle_state(w, st.k_scale_host, st.v_scale_host, cache_dtype=cd)
        ref[cd], _ = oracle.attention(K, V, st.k_scale_host, st.v_scale_host, q, w.page_table,
                                      w.ctx_lens, SM_SCALE, cache_dtype=cd)
        check_outputs(gpu[cd], None, ref[cd])
        del st
        torch.cuda.empty_cache()
    d_gpu = gpu[fp8kv.E4M3] - gpu[fp8kv.BF16]
    d_ref = ref[fp8kv.E4M3] - ref[fp8kv.BF16]
    gap = np.abs(d_gpu - d_ref).max()
    # the two parity errors: ~1e-7 (e4m3 cache) and ~7e-6 (bf16 cache, whose
    # P enters PV as two bf16 terms, 16 bits)
    assert gap <= 1e-4, gap
    rel = np.linalg.norm(d_ref) / np.linalg.norm(ref[fp8kv.BF16])
    print(f"{w.name} B={w.B}: FP8-vs-BF16 max abs {np.abs(d_ref).max():.3e}, rel L2 {rel:.3e}; "
          f"GPU vs oracle difference {gap:.2e}")
    # the quantization error is real (e4m3 keeps 3 mantissa bits) and small
    assert 1e-4 < rel < 0.1, rel


def test_values_exact_in_e4m3_give_the_bf16_cache_result():
    """Invariant: an e4m3 cache holding values that are exactly code x scale
    (scale a power of two, so every value is a bf16 number) gives the result
    of a bf16 cache holding the same values.  The append writes exactly the
    planted codes, and both kernels agree with the oracle and with each
    other to within their parity errors."""
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_paged_fp8kv_amd as fp8kv
    from _helpers import unswizzle
    w = workloads.custom("exact_e4m3", [33, 200, 511, 1000, 16], Hq=16, Hkv=2, seed=12)
    rng = np.random.default_rng(4)
    tab = oracle.e4m3_table()
    n_tok = int(w.ctx_lens.sum())
    # codes of magnitude below 16 (exponent field <= 10), so values stay below 2
    pick = np.array([x for x in range(256) if ((x >> 3) & 15) <= 10], np.uint8)
    codes = {c: rng.choice(pick, size=(n_tok, w.Hkv, 128)) for c in "kv"}
    scale = np.float32(2.0 ** -3)
    bits = {c: ((tab[codes[c]] * scale).astype(np.float32).view(np.uint32) >> 16)
            .astype(np.uint16) for c in "kv"}
    assert all((workloads.bf16_bits_to_f32(bits[c]) ==
                (tab[codes[c]] * scale).astype(np.float32)).all() for c in "kv")
    seq = np.repeat(np.arange(w.B, dtype=np.int32), w.ctx_lens)
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in w.ctx_lens])
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    q = w.q_bits()
    sc = dev(np.full(w.Hkv, scale, np.float32))
    pt = dev(w.page_table)
    out = {}
    for cd in (fp8kv.E4M3, fp8kv.BF16):
        d = fp8kv.desc(w.num_pages, w.Hkv, cd)
        K, V = fp8kv.new_cache(d)
        fp8kv.append(d, K, V, sc, sc, dev(bits["k"].view(np.int16)), dev(bits["v"].view(np.int16)),
                     dev(seq), dev(pos), pt)
        out[cd] = fp8kv.decode_attention(d, K, V, sc, sc, dev(q.view(np.int16)), pt,
                                         dev(w.ctx_lens), out_dtype=fp8kv.OUT_F32)
        torch.cuda.synchronize()
        if cd == fp8kv.E4M3:
            used = np.unique(w.page_table[w.page_table >= 0])
            Kc = unswizzle(K.cpu().numpy(), w.Hkv, 0, used, False)
            Ko = np.zeros((w.num_pages, w.Hkv, 16, 128), np.uint8)
            for t in range(n_tok):
                Ko[w.page_table[seq[t], pos[t] // 16], :, pos[t] % 16] = codes["k"][t]
            assert (Kc == Ko[used]).all()       # the append stored exactly the codes
    a, b = out[fp8kv.E4M3].cpu().numpy(), out[fp8kv.BF16].cpu().numpy()
    K, V = oracle.new_cache(w.num_pages, w.Hkv)
    oracle.append(K, V, np.full(w.Hkv, scale), np.full(w.Hkv, scale), bits["k"], bits["v"], seq,
                  pos, w.page_table)
    ref, _ = oracle.attention(K, V, np.full(w.Hkv, scale), np.full(w.Hkv, scale), q,
                              w.page_table, w.ctx_lens, SM_SCALE)
    check_outputs(a, None, ref)
    check_outputs(b, None, ref)
    gap = np.abs(a.astype(np.float64) - b).max()
    print(f"e4m3 cache vs bf16 cache on e4m3-exact values: max abs difference {gap:.2e}")
    assert gap <= 2e-5, gap
