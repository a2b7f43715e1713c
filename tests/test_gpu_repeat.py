"""GPU: every attention entry point gives bit-identical results when it is
called again on the same inputs, whatever its workspace held before (random
bytes are written over it before each call).  No result may depend on timing
or on memory a call did not write itself."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

REPEATS = 25


def _repeat(call, ws, what):
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    first = None
    for i in range(REPEATS):
        ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device=ws.device, generator=g))
        o = call()
        torch.cuda.synchronize()
        o = o.cpu().numpy().view(np.uint32).copy()
        if first is None:
            first = o
            assert np.isfinite(o.view(np.float32)).all()
        else:
            assert np.array_equal(o, first), f"{what}: call {i}: {(o != first).sum()} elements differ"
    print(f"{what}: {REPEATS} calls bit-identical", flush=True)


def _state(ctx_before, Hq, Hkv, cd):
    import workloads
    from workloads import device
    w = workloads.custom("repeat", ctx_before, Hq, Hkv, seed=11)
    st = device.build(w, cache_dtype=cd)
    st.step(check_tags=True)
    torch.cuda.synchronize()
    return w, st


@pytest.mark.parametrize("cd", [0, 1])
def test_plain_and_multi_query_calls_repeat(cd):
    import decode_attention_paged_fp8kv_amd as fp8kv
    from workloads import device
    w, st = _state([5, 40, 300, 1000, 2047, 16, 3000, 129], 64, 8, cd)
    for nw in (0, 64):
        ws = torch.empty(max(fp8kv.decode_workspace_size(st.desc, w.B, w.Hq, nw), 1),
                         dtype=torch.uint8, device="cuda")
        _repeat(lambda: fp8kv.decode_attention(st.desc, st.K, st.V, st.k_scale, st.v_scale, st.q,
                                               st.page_table, st.ctx_lens, abort=st.abort,
                                               out_dtype=fp8kv.OUT_F32, num_workers=nw,
                                               workspace=ws),
                ws, f"plain cache={cd} workers={nw}")
    for q_len in (2, 4):
        sp = device.build_spec(st, q_len)
        _repeat(lambda: sp.decode(out_dtype=fp8kv.OUT_F32), sp.workspace,
                f"q_len={q_len} cache={cd}")


@pytest.mark.parametrize("cd", [0, 1])
@pytest.mark.parametrize("groups,Hq,Hkv", [
    (((5, 48),), 64, 8),                    # one group, one column tile per wave
    (((20, 64),), 64, 8),                   # one group, two column tiles per wave
    (((5, 64), (2, 32), (9, 160)), 16, 4),  # three groups and ungrouped requests
])
def test_shared_prompt_calls_repeat(cd, groups, Hq, Hkv):
    import decode_attention_paged_fp8kv_amd as fp8kv
    import workloads
    from workloads import device
    w = workloads.shared_prompts(list(groups), plain=3, suffix_max=70, Hq=Hq, Hkv=Hkv)
    st = device.build(w, cache_dtype=cd)
    st.step(check_tags=True)
    torch.cuda.synchronize()
    gs = np.concatenate([[0], np.cumsum([r for r, _ in groups])]).tolist()
    pl = [p for _, p in groups]
    for nw in (0, 12):
        need = fp8kv.decode_workspace_size_shared(st.desc, w.B, w.Hq, w.max_pages, gs, pl, nw)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        _repeat(lambda: fp8kv.decode_attention_shared(st.desc, st.K, st.V, st.k_scale, st.v_scale,
                                                      st.q, st.page_table, st.ctx_lens, gs, pl,
                                                      abort=st.abort, out_dtype=fp8kv.OUT_F32,
                                                      num_workers=nw, workspace=ws),
                ws, f"shared groups={groups} cache={cd} workers={nw}")
