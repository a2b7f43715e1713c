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
    assert gap <= 4e-3, gap
    rel = np.linalg.norm(d_ref) / np.linalg.norm(ref[fp8kv.BF16])
    print(f"{w.name} B={w.B}: FP8-vs-BF16 max abs {np.abs(d_ref).max():.3e}, rel L2 {rel:.3e}; "
          f"GPU vs oracle difference {gap:.2e}")
    # the quantization error is real (e4m3 keeps 3 mantissa bits) and small
    assert 1e-4 < rel < 0.1, rel
