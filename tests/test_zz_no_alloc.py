"""The allocation-free decode entry point (fp8kv_decode_attention_noalloc)
against the workspace form it shares its kernels with: the same outputs bit
for bit (same inputs, same worker count), on two calls in a row, the second
smaller than the first, whatever the shared scratch holds from earlier calls;
sizes above the scratch are refused before anything runs; the call recorded in
a HIP graph replays to the eager bits."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from _helpers import SM_SCALE, check_outputs

pytestmark = pytest.mark.gpu


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _both(fp8kv, st, out_dtype, num_workers=0):
    """(workspace form, allocation-free form) outputs of one decode."""
    ref = st.decode(out_dtype=out_dtype, num_workers=num_workers).clone()
    out = torch.empty_like(ref)
    got = fp8kv.decode_attention_noalloc(st.desc, st.K, st.V, st.k_scale, st.v_scale, st.q,
                                         st.page_table, st.ctx_lens, out, abort=st.abort,
                                         out_dtype=out_dtype, num_workers=num_workers)
    assert got is out
    return _host(ref.view(torch.int32) if ref.dtype == torch.float32 else ref.view(torch.int16)), \
        _host(got.view(torch.int32) if got.dtype == torch.float32 else got.view(torch.int16))


def test_noalloc_equals_workspace_form_twice_shrinking():
    import decode_attention_paged_fp8kv_amd as fp8kv
    from workloads import device
    assert torch.cuda.is_available()
    # 1: the ragged 64-request workload (about 5 MB of partial states)
    big = device.build(workloads.make(3))
    big.step(check_tags=True)
    for od in (fp8kv.OUT_BF16, fp8kv.OUT_F32):
        a, b = _both(fp8kv, big, od)
        assert np.array_equal(a, b), od
    # 2: a smaller batch right after, with stale tags (aborted rows), checked
    #    against the workspace form and against the oracle
    w = workloads.make(5, batch=40)
    small = device.build(w)
    small.step(check_tags=True)
    ab = _host(small.abort)
    assert (ab == w.expected_abort).all() and 0 < ab.sum() < w.B
    for nw in (0, 64):
        for od in (fp8kv.OUT_BF16, fp8kv.OUT_F32):
            a, b = _both(fp8kv, small, od, nw)
            assert np.array_equal(a, b), (nw, od)
    from _helpers import oracle_state
    Ko, Vo = oracle_state(w, small.k_scale_host, small.v_scale_host, abort=ab)
    ref, _ = oracle.attention(Ko, Vo, small.k_scale_host, small.v_scale_host, w.q_bits(),
                              w.page_table, w.ctx_lens, SM_SCALE, abort=ab)
    out = torch.empty(w.B, w.Hq, 128, dtype=torch.float32, device="cuda")
    fp8kv.decode_attention_noalloc(small.desc, small.K, small.V, small.k_scale, small.v_scale,
                                   small.q, small.page_table, small.ctx_lens, out,
                                   abort=small.abort, out_dtype=fp8kv.OUT_F32)
    err = check_outputs(_host(out), None, ref)
    print(f"allocation-free decode: bit-identical to the workspace form; max abs err vs "
          f"oracle {err:.3e}", flush=True)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    """A batch whose partial states exceed the scratch is refused on the host
    (nothing is enqueued); an empty batch is a no-op."""
    import decode_attention_paged_fp8kv_amd as fp8kv
    lib = fp8kv.raw_library()
    B, Hq, Hkv = 4096, 64, 8
    d = fp8kv.desc(64, Hkv)
    assert fp8kv.decode_workspace_size(d, B, Hq) > fp8kv.NOALLOC_SCRATCH_BYTES
    fake = 256   # never dereferenced: the call fails before any device work
    st = lib.fp8kv_decode_attention_noalloc(
        __import__("ctypes").byref(d), fake, fake, fake, fake, fake, Hq, fake, 4, fake, B,
        __import__("ctypes").c_float(SM_SCALE), None, fake, 0, 0, None)
    assert st == -4
    assert fp8kv.decode_workspace_size(d, 64, Hq) <= fp8kv.NOALLOC_SCRATCH_BYTES
    out = torch.empty(0, Hq, 128, dtype=torch.bfloat16, device="cuda")
    z = torch.empty(0, dtype=torch.int32, device="cuda")
    kc = torch.zeros(fp8kv.cache_bytes(d), dtype=torch.uint8, device="cuda")
    sc = torch.ones(Hkv, dtype=torch.float32, device="cuda")
    fp8kv.decode_attention_noalloc(d, kc, kc, sc, sc,
                                   torch.empty(0, Hq, 128, dtype=torch.bfloat16, device="cuda"),
                                   z.view(0, 0), z, out)
    torch.cuda.synchronize()


def test_noalloc_call_recorded_in_a_graph():
    """The callers the entry point is for: a HIP graph records the call
    (nothing to allocate at capture or at replay); three replays, with eager
    calls of the workspace form and a cleared output in between, each equal
    to the eager result bit for bit."""
    import decode_attention_paged_fp8kv_amd as fp8kv
    from workloads import device
    w = workloads.make(5, batch=40)
    st = device.build(w, num_workers=64)
    st.step(check_tags=True)
    torch.cuda.synchronize()
    ref = st.decode(num_workers=64).clone()
    out = torch.empty_like(ref)

    def call():
        fp8kv.decode_attention_noalloc(st.desc, st.K, st.V, st.k_scale, st.v_scale, st.q,
                                       st.page_table, st.ctx_lens, out, abort=st.abort,
                                       num_workers=64)
    call()                      # the first call on the device looks up the scratch address
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()                  # marshalled inside the capture: it names the capturing stream
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
        st.decode(num_workers=64)   # eager work between replays
        torch.cuda.synchronize()
