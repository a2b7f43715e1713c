#!/usr/bin/env python3
"""Benchmark of one decode step of FP8 paged attention with page-tag integrity.

A step = tag check (separate batched kernel) + quantize-on-append of each
request's new token + paged attention over the e4m3 cache (+ split merge),
for one layer, all requests, one stream.  Inputs are synthetic and already
resident in HBM when timing starts.

Default workload: 64 requests with context lengths uniform in [1024, 32768],
64 query / 8 kv heads, head_dim 128, 16-token pages, pages a seeded random
permutation of the pool, tag check on.

Prints ONE JSON line (rank 0, one GPU).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8 paged decode attn: tokens/s and achieved HBM GB/s (% of 8 TB/s) @1 GPU"
PEAK_GBPS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "decode_attention_paged_fp8kv_amd", "csrc", "fp8kv_kernels.hip")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "decode_ragged64_hbm_counters.txt")


def kernel_source_hash() -> str:
    import hashlib
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()


def counter_traffic():
    """HBM bytes per decode call from the committed counter summary, or None
    when it is missing or was taken on a different kernel source."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    fields = {}
    for line in open(PMC_SUMMARY):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(float(fields["traffic_bytes_per_decode_call"]))
    except (KeyError, ValueError):
        return None


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def alg_bytes(w, cache_dtype: int, tag_check: bool, active=None):
    """Algorithmic HBM bytes of one step and of the attention kernel alone.

    KV reads 2*Hkv*D*(L_b+1)*E per active request (E = 1 e4m3, 2 bf16);
    Q read and O write 2*Hq*D bytes each; append reads 2*Hkv*D*2 bytes and
    writes 2*Hkv*D*E; page ids 4*n_b; the tag check 12*n_b (id, expected
    tag, current tag) when enabled.  Split-K partials are overhead, not
    counted."""
    import numpy as np
    E = 1 if cache_dtype == 0 else 2
    D = 128
    act = np.ones(w.B, bool) if active is None else active
    L1 = w.ctx_lens.astype(np.int64)
    n = w.n_pages.astype(np.int64)
    kv = int((2 * w.Hkv * D * L1 * E)[act].sum())
    qo = int(act.sum()) * w.Hq * D * 2 * 2
    ids = int((4 * n)[act].sum())
    attn = kv + qo + ids
    append = int(act.sum()) * (2 * w.Hkv * D * 2 + 2 * w.Hkv * D * E)
    verify = int((12 * n).sum()) if tag_check else 0
    return attn + append + verify, attn


def time_steps(fn, steps: int):
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def warm_up(fns, min_seconds: float = 0.1):
    """Run the steps in turn for at least min_seconds of wall time.  Right
    after a state is built the first tens of milliseconds of GPU work run
    slower (a multi-query step measured 410 us first, 371 us later), so the
    studies that compare several steps warm each up this way and interleave
    their timed rounds."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_seconds:
        for f in fns:
            f()
        torch.cuda.synchronize()


def interleaved_steps(fns, steps: int, rounds: int = 4):
    """Seconds per step of each fn: rounds of steps // rounds steps each,
    the fns alternating round by round; the median round of each."""
    per = max(1, steps // rounds)
    out = [[] for _ in fns]
    for r in range(rounds):
        order = list(range(len(fns))) if r % 2 == 0 else list(range(len(fns)))[::-1]
        for i in order:
            out[i].append(time_steps(fns[i], per))
    return [statistics.median(v) for v in out]


def event_times(fns, steps: int):
    """Per-stage HIP-event durations (ms) on the current stream."""
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        ev[k][0].record()
        for i, f in enumerate(fns):
            f()
            ev[k][i + 1].record()
    torch.cuda.synchronize()
    return [[ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(steps)] for i in range(len(fns))]


def capture_graphs(st, fns):
    """One captured HIP graph per function; each replay is checked bit for bit
    against an eager call (with eager work in between) before it is timed."""
    import torch
    outs = lambda: (st.out.clone(), st.abort.clone())  # noqa: E731
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(side)
    graphs = []
    for f in fns:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            f()
        graphs.append(g)
    torch.cuda.synchronize()
    fns[0]()
    ref = outs()
    for _ in range(3):
        graphs[0].replay()
        torch.cuda.synchronize()
        got = outs()
        if not all(torch.equal(a, b) for a, b in zip(got, ref)):
            raise RuntimeError("graph replay of the step differs from the eager step")
        fns[0]()
    return [g.replay for g in graphs]


def loop_study(args):
    """Multi-step decode with the tag tracker on vs the no-op tracker: prompts of
    8,192 tokens, 1,000 generated tokens, concurrency 1/2/4/8, 1 and 32 layers of
    the ragged workload's shape (64 q-heads / 8 kv-heads), launched eagerly or as
    one captured HIP graph per step.  Runs of the two tracker modes alternate;
    each run restarts from the prompt.  A step's latency is its wall time
    including the host work (page allocation, tag upload, launches or graph
    replay) and the read-back of the abort flags, synchronized at the end of
    every step."""
    import numpy as np
    import torch
    from workloads.decode_loop import DecodeLoop

    rng = np.random.default_rng(0)
    per = {}
    for launch, nl, c in [(g, nl, c) for g in args.loop_launch for nl in args.loop_layers
                          for c in args.loop_concurrency]:
        log(f"bench: decode loop, {launch} launches, {nl} layer(s), concurrency {c}")
        loops = {m: DecodeLoop(c, args.loop_prompt, args.loop_steps, tracker=(m == "on"), seed=c,
                               step_sets=16, layers=nl, graph=(launch == "graph"))
                 for m in ("on", "off")}
        for lp in loops.values():
            lp.run(min(20, args.loop_steps))
            lp.reset()
        tot = {"on": [], "off": []}
        lat = {"on": [], "off": []}
        for r in range(args.loop_rounds):
            for m in (("on", "off") if r % 2 == 0 else ("off", "on")):
                x = loops[m].run()
                loops[m].reset()
                tot[m].append(float(x.sum()))
                lat[m].append(x)
        d = np.array([(a - b) / b for a, b in zip(tot["on"], tot["off"])])
        boots = [rng.choice(d, d.size).mean() for _ in range(2000)]
        # p95 step latency per round, on against off in the same round pair
        d95 = np.array([np.percentile(a, 95) / np.percentile(b, 95) - 1
                        for a, b in zip(lat["on"], lat["off"])])
        boots95 = [rng.choice(d95, d95.size).mean() for _ in range(2000)]
        res = {}
        for m in ("on", "off"):
            allx = np.concatenate(lat[m])
            res[m] = {"tokens_s": round(c * args.loop_steps / float(np.median(tot[m])), 1),
                      "step_ms_p50": round(float(np.percentile(allx, 50)) * 1e3, 4),
                      "step_ms_p95": round(float(np.percentile(allx, 95)) * 1e3, 4)}
        res["overhead_pct"] = {"mean": round(100 * float(d.mean()), 3),
                               "ci95": [round(100 * float(np.percentile(boots, 2.5)), 3),
                                        round(100 * float(np.percentile(boots, 97.5)), 3)]}
        res["overhead_us_per_step"] = round(
            1e6 * (float(np.median(tot["on"])) - float(np.median(tot["off"]))) / args.loop_steps, 2)
        res["p95_overhead_pct"] = {"mean": round(100 * float(d95.mean()), 3),
                                   "ci95": [round(100 * float(np.percentile(boots95, 2.5)), 3),
                                            round(100 * float(np.percentile(boots95, 97.5)), 3)]}
        per.setdefault(launch, {}).setdefault(f"{nl}_layers", {})[str(c)] = res
        for lp in loops.values():
            lp.close()
        del loops
        torch.cuda.empty_cache()
    top = per[args.loop_launch[0]][f"{args.loop_layers[0]}_layers"][str(max(args.loop_concurrency))]
    print(json.dumps({
        "metric": "decode loop (8192-token prompts, 1000 generated tokens): tokens/s and p95 "
                  "step latency, tag tracker on vs the no-op tracker",
        "value": top["on"]["tokens_s"], "unit": "tokens/s", "n_gpus": 1,
        "higher_is_better": True, "data": "synthetic",
        "config": {"workload": "decode_loop", "prompt_tokens": args.loop_prompt,
                   "generated_tokens": args.loop_steps, "q_heads": 64, "kv_heads": 8,
                   "head_dim": 128, "page_tokens": 16, "kv_cache": "e4m3",
                   "rounds": args.loop_rounds, "layers": args.loop_layers},
        "value_is": f"tracker on, {args.loop_launch[0]} launches, {args.loop_layers[0]} "
                    f"layer(s), concurrency {max(args.loop_concurrency)}",
        "by_launch_layers_and_concurrency": per}), flush=True)


def accuracy_study(args):
    """FP8 cache vs BF16 cache on the same inputs through the same kernel (f32
    outputs): the difference is the error the e4m3 storage adds, since the
    BF16-cache output agrees with binary64 attention to ~1e-6 (parity tests).
    Uniform, ragged and long-context workloads (the last with ±20 outliers,
    so scale = 20/448, and ±25 values on the new token that saturate)."""
    import numpy as np
    import torch

    import decode_attention_paged_fp8kv_amd as fp8kv
    import workloads
    from workloads import device

    res = {}
    for cfg in args.accuracy_configs:
        w = workloads.make(cfg)
        log(f"bench: accuracy, workload {w.name}")
        outs = {}
        for cd in (fp8kv.E4M3, fp8kv.BF16):
            st = device.build(w, cache_dtype=cd)
            st.step(check_tags=True)
            outs[cd] = st.decode(True, out_dtype=fp8kv.OUT_F32).double()
            torch.cuda.synchronize()
            del st
            torch.cuda.empty_cache()
        def metrics(ref, got):
            err = got - ref
            cos = torch.nn.functional.cosine_similarity(got.reshape(-1, got.shape[-1]),
                                                        ref.reshape(-1, ref.shape[-1]), dim=1)
            return {"max_abs_err": float(err.abs().max()),
                    "mean_abs_err": float(err.abs().mean()),
                    "rel_l2_err": float(err.norm() / ref.norm()),
                    "min_cosine": float(cos.min()),
                    "output_rms": float(ref.pow(2).mean().sqrt()),
                    "output_max_abs": float(ref.abs().max())}
        ref, got = outs[fp8kv.BF16], outs[fp8kv.E4M3]
        res[w.name] = metrics(ref, got)
        # kv-head 0 carries the long workload's saturating values on the new token;
        # the other kv-heads' q-heads show the error of in-range values alone
        res[w.name]["kv_head_0"] = metrics(ref[:, :w.G], got[:, :w.G])
        res[w.name]["other_kv_heads"] = metrics(ref[:, w.G:], got[:, w.G:])
        del outs, ref, got
        torch.cuda.empty_cache()
    print(json.dumps({
        "metric": "FP8 e4m3 cache vs BF16 cache: attention output error (same inputs, same "
                  "kernel, f32 outputs)",
        "value": max(r["rel_l2_err"] for r in res.values()), "unit": "relative L2 error (max over "
                 "workloads)", "n_gpus": 1, "higher_is_better": False, "data": "synthetic",
        "config": {"workload": "accuracy", "workloads": list(res)},
        "by_workload": res}), flush=True)


def spec_study(args):
    """q_len new tokens per request checked in one step (speculative
    verification) on the chosen workload: tag check and append of the q_len
    tokens (one launch), one multi-query attention launch.  The request's context after the
    step is the workload's own (L_b + 1), so the pages read are the same as the
    one-token step's; verified tokens per second count live requests x q_len.
    The one-token step over the same cache is timed in the same run."""
    import numpy as np
    import torch

    import workloads
    from workloads import device

    cfg = {"tiny": 1, "uniform": 2, "ragged": 3, "long": 4, "capacity": 5}[args.workload]
    cache = 0 if args.cache == "e4m3" else 1
    w = workloads.make(cfg)
    log(f"bench: speculative verification, workload {w.name}, q_len {args.qlen}")
    base = device.build(w, cache_dtype=cache, num_workers=args.num_workers)
    sp = device.build_spec(base, args.qlen)
    sp.step(True)
    torch.cuda.synchronize()
    live = base.abort.cpu().numpy() == 0
    one_bytes, one_attn = alg_bytes(w, cache, True, active=live)
    # extra bytes of the q_len-token step: q_len-1 more Q rows and O rows per live
    # request, q_len-1 more appended tokens (2 reads of bf16, 1 write of E per value)
    E = 1 if cache == 0 else 2
    nl = int(live.sum())
    extra_qo = nl * (args.qlen - 1) * w.Hq * 128 * 2 * 2
    extra_app = nl * (args.qlen - 1) * 2 * w.Hkv * 128 * (2 + E)
    attn_bytes = one_attn + extra_qo
    step_bytes = one_bytes + extra_qo + extra_app
    for _ in range(args.warmup):
        sp.step(True)
        base.step(True)
    warm_up([lambda: sp.step(True), lambda: base.step(True)])
    t_spec, t_one = interleaved_steps([lambda: sp.step(True), lambda: base.step(True)], args.steps)
    nev = max(20, args.steps // 2)
    # the calls on their own, through the steps' prepared launches where there are
    # (a context shorter than q_len takes the two-launch form, unprepared)
    spec_dec = (lambda: sp.prepared()[1]()) if sp.k_new_q is not None else (lambda: sp.decode(True))
    td_spec, td_one = event_times([spec_dec, lambda: base.prepared(True)[1]()], nev)
    ta = event_times([lambda: sp.prepared()[0]() if sp.k_new_q is not None else sp.append(True)],
                     nev)[0]
    td_spec = statistics.median(td_spec) * 1e-3
    td_one = statistics.median(td_one) * 1e-3
    gbps = attn_bytes / td_spec / 1e9
    print(json.dumps({
        "metric": "speculative verification step: new tokens checked per second (q_len per "
                  "request; tag check + append + multi-query attention)",
        "value": round(nl * args.qlen / t_spec, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_spec * 1e3, 4),
        "higher_is_better": True, "data": "synthetic",
        "dtype": f"{args.cache} cache; bf16/f16 MFMA, f32 accumulate",
        "config": {"workload": w.name, "requests": w.B, "live_requests": nl, "q_len": args.qlen,
                   "q_heads": w.Hq, "kv_heads": w.Hkv, "columns": w.G * args.qlen,
                   "head_dim": 128, "page_tokens": 16, "kv_cache": args.cache,
                   "attended_tokens_last_query": int(w.ctx_lens.sum())},
        "step_alg_bytes": step_bytes, "hbm_gbps": round(step_bytes / t_spec / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": "fp8kv_decode_attention_q call",
                     "achieved": round(gbps, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_GBPS, 4), "traffic": None,
                     "alg_bytes_per_launch": attn_bytes, "avg_launch_us": round(td_spec * 1e6, 2)},
        "tag_check_append_us": round(statistics.median(ta) * 1e3, 2),
        "tag_check_append": "one launch" if sp.k_new_q is not None else "two launches",
        "one_token_step": {"ms_per_step": round(t_one * 1e3, 4),
                           "tokens_s": round(nl / t_one, 1),
                           "decode_us": round(td_one * 1e6, 2)},
        "step_time_ratio_vs_one_token": round(t_spec / t_one, 4)}), flush=True)


def shared_study(args):
    """Cache reuse: 64 requests continuing one 16,384-token prompt (U[16, 2048]
    own tokens each), the prompt's pages mapped by every request (shared) vs a
    private copy per request.  Same values, lengths and work partition, so the
    plain call's outputs are bit-identical; what changes is how many distinct
    bytes the step reads.  With shared pages the shared-prompt call also reads
    each of the prompt's pages once for the whole batch.  Step = fused check +
    append, then attention."""
    import numpy as np
    import torch

    import workloads
    from workloads import device

    res = {}
    for shared in ((True,) if args.no_private else (True, False)):
        w = workloads.shared_prefix(shared=shared)
        log(f"bench: {w.name}")
        st = device.build(w)
        st.step(check_tags=True)
        torch.cuda.synchronize()
        live = st.abort.cpu().numpy() == 0
        step_bytes, attn_bytes = alg_bytes(w, 0, True, active=live)
        # distinct K/V bytes: the shared prompt once, every request's own tokens
        own = (w.ctx_lens - w.prefix_len).astype(np.int64)
        kv_tok = int(own[live].sum()) + (w.prefix_len if shared else w.prefix_len * int(live.sum()))
        unique_kv = 2 * w.Hkv * 128 * kv_tok
        for _ in range(args.warmup):
            st.step(check_tags=True)
        warm_up([lambda: st.step(check_tags=True)])
        t = time_steps(lambda: st.step(check_tags=True), args.steps)
        td = statistics.median(event_times([lambda: st.prepared(True)[1]()],
                                           max(20, args.steps // 2))[0]) * 1e-3
        res["shared" if shared else "private"] = {
            "workload": w.name, "pool_pages": w.num_pages, "ms_per_step": round(t * 1e3, 4),
            "tokens_s": round(int(live.sum()) / t, 1), "decode_us": round(td * 1e6, 2),
            "alg_bytes_per_decode": attn_bytes,
            "alg_gbps": round(attn_bytes / td / 1e9, 1),
            "distinct_kv_bytes": unique_kv,
            "distinct_kv_gbps": round(unique_kv / td / 1e9, 1)}
        res["out_" + ("shared" if shared else "private")] = st.decode(True, out_dtype=1).clone()
        if shared:
            # the shared-prompt call: the prompt's pages once for the whole batch
            import decode_attention_paged_fp8kv_amd as fp8kv
            groups = ([0, w.B], [w.prefix_len])
            ws = torch.zeros(fp8kv.decode_workspace_size_shared(st.desc, w.B, w.Hq, w.max_pages,
                                                                *groups),
                             dtype=torch.uint8, device="cuda")
            call = fp8kv.decode_attention_shared(st.desc, st.K, st.V, st.k_scale, st.v_scale,
                                                 st.q, st.page_table, st.ctx_lens, *groups,
                                                 abort=st.abort, workspace=ws, prepare=True)

            def cstep():
                st.verify_append()
                call()
            for _ in range(args.warmup):
                cstep()
            warm_up([cstep])
            tc = time_steps(cstep, args.steps)
            tdc = statistics.median(event_times([call], max(20, args.steps // 2))[0]) * 1e-3
            res["shared_call"] = {
                "ms_per_step": round(tc * 1e3, 4), "tokens_s": round(int(live.sum()) / tc, 1),
                "decode_us": round(tdc * 1e6, 2), "alg_gbps": round(attn_bytes / tdc / 1e9, 1),
                "distinct_kv_gbps": round(unique_kv / tdc / 1e9, 1)}
            out_c = fp8kv.decode_attention_shared(st.desc, st.K, st.V, st.k_scale, st.v_scale,
                                                  st.q, st.page_table, st.ctx_lens, *groups,
                                                  abort=st.abort, out_dtype=1, workspace=ws)
            res["shared_call"]["max_abs_diff_vs_plain_call"] = float(
                (out_c - res["out_shared"]).abs().max())
        del st
        torch.cuda.empty_cache()
    out_pr = res.pop("out_private", None)
    same = bool(torch.equal(res.pop("out_shared"), out_pr)) if out_pr is not None else None
    sh, pr, sc = res["shared"], res.get("private"), res["shared_call"]
    print(json.dumps({
        "metric": "shared-prompt decode step (64 requests, one 16,384-token prompt mapped by all "
                  "+ U[16, 2048] own tokens): tokens/s, shared pages vs private copies",
        "value": sc["tokens_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "data": "synthetic",
        "dtype": "e4m3 cache; bf16/f16 MFMA, f32 accumulate",
        "config": {"workload": sh["workload"], "requests": 64, "prompt_tokens": 16384,
                   "q_heads": 64, "kv_heads": 8, "head_dim": 128, "page_tokens": 16,
                   "kv_cache": "e4m3", "tag_check": True},
        "value_is": "shared pages, shared-prompt call (fp8kv_decode_attention_shared)",
        "shared_call": sc, "shared": sh, "private": pr,
        "step_speedup_shared_pages": round(pr["ms_per_step"] / sh["ms_per_step"], 3) if pr else None,
        "step_speedup_shared_call": round(pr["ms_per_step"] / sc["ms_per_step"], 3) if pr else None,
        "outputs_bit_identical": same}), flush=True)


def device_info():
    """What the numbers were measured on."""
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2**30, 1), "hip": torch.version.hip}


def device_copy(n_bytes: int = 2 << 30):
    """A plain device-to-device copy of 2 GiB (torch's copy kernel): read plus
    written bytes per second, the streaming rate a simple kernel reaches on this
    part, beside the 8 TB/s denominator."""
    import torch
    x = torch.ones(n_bytes, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    t = statistics.median(event_times([lambda: y.copy_(x)], 10)[0]) * 1e-3
    del x, y
    torch.cuda.empty_cache()
    return {"bytes_moved": 2 * n_bytes, "us": round(t * 1e6, 1),
            "gbps": round(2 * n_bytes / t / 1e9, 1)}


def stream_read(n_bytes: int = 4 << 30):
    """The library's streaming-read reference over 4 GiB: 16-byte nontemporal
    loads like the tile loads, no page indirection."""
    import torch
    import decode_attention_paged_fp8kv_amd as fp8kv
    x = torch.ones(n_bytes, dtype=torch.uint8, device="cuda")
    sink = fp8kv.debug_read_bandwidth(x)
    for _ in range(2):
        fp8kv.debug_read_bandwidth(x, sink)
    t = statistics.median(event_times([lambda: fp8kv.debug_read_bandwidth(x, sink)], 10)[0]) * 1e-3
    del x, sink
    torch.cuda.empty_cache()
    return {"bytes_read": n_bytes, "us": round(t * 1e6, 1), "gbps": round(n_bytes / t / 1e9, 1)}


def cpu_study(args):
    """The oracle as it stands on the host, single-threaded and on all cores,
    on bounded samples of the tiny, uniform, ragged and long workloads: context
    for the GPU figures, not a target."""
    import oracle
    import workloads
    res = {}
    all_threads = oracle.num_threads()
    for cfg in (1, 2, 3, 4):
        w = workloads.make(cfg)
        for threads in (1, all_threads):
            oracle.set_num_threads(threads)
            log(f"bench: CPU oracle, {w.name}, {threads} thread(s)")
            res.setdefault(w.name, {})[f"{threads}_threads"] = cpu_baseline(w, target_s=5.0)
    oracle.set_num_threads(all_threads)
    print(json.dumps({
        "metric": "CPU oracle (binary64, plain C + OpenMP over output rows): tokens/s and "
                  "algorithmic GB/s on bounded samples",
        "value": res[workloads.make(3).name][f"{all_threads}_threads"]["value"],
        "unit": "tokens/s", "n_gpus": 0, "higher_is_better": True, "data": "synthetic",
        "config": {"workload": "cpu_study", "threads": [1, all_threads]},
        "value_is": f"ragged workload, {all_threads} threads", "by_workload": res}), flush=True)


def cpu_baseline(w, target_s: float = 15.0):
    """The oracle as it stands, on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    import workloads
    from workloads import device  # noqa: F401

    rng_key = 0x5EED
    K, V = oracle.new_cache(w.num_pages, w.Hkv)

    def fill(b):
        pages = w.page_table[b, : w.n_pages[b]]
        nbytes = pages.size * w.Hkv * 16 * 128
        for X, k in ((K, rng_key + 2 * b), (V, rng_key + 2 * b + 1)):
            bits = workloads.draw_bits(k, 0, nbytes).astype(np.uint8)
            bits[(bits & 0x7F) == 0x7F] = 0x7E
            X[pages] = bits.reshape(pages.size, w.Hkv, 16, 128)

    ks = np.full(w.Hkv, 0.01, np.float32)
    vs = np.full(w.Hkv, 0.01, np.float32)
    q = w.q_bits()
    sm = np.float32(1.0 / np.sqrt(128.0))

    def run(reqs):
        reqs = np.asarray(reqs)
        t0 = time.perf_counter()
        ab = oracle.verify(w.page_table[reqs], w.expected_tags[reqs], w.ctx_lens[reqs], w.pool_tags)
        kn = np.stack([w.kv_tokens("k", b, int(w.ctx_before[b]), int(w.ctx_before[b]) + 1)[0]
                       for b in reqs])
        vn = np.stack([w.kv_tokens("v", b, int(w.ctx_before[b]), int(w.ctx_before[b]) + 1)[0]
                       for b in reqs])
        oracle.append(K, V, ks, vs, kn, vn, np.arange(len(reqs), dtype=np.int32),
                      w.ctx_before[reqs].astype(np.int32), w.page_table[reqs], abort=ab)
        oracle.attention(K, V, ks, vs, q[reqs], w.page_table[reqs], w.ctx_lens[reqs], sm, abort=ab)
        return time.perf_counter() - t0

    fill(0)
    t1 = run([0])
    per_tok = t1 / max(1, int(w.ctx_lens[0]))
    reqs, est = [0], t1
    for b in range(1, w.B):
        if est >= target_s:
            break
        fill(b)
        reqs.append(b)
        est += per_tok * int(w.ctx_lens[b])
    t = run(reqs)
    mask = np.zeros(w.B, bool)
    mask[reqs] = True
    step_bytes, _ = alg_bytes(w, 0, False, active=mask)
    return {"value": len(reqs) / t, "unit": "tokens/s", "cores": oracle.num_threads(),
            "alg_gbps": round(step_bytes / t / 1e9, 4),
            "kind": "oracle",
            "sample": f"requests 0..{len(reqs) - 1} of the workload ({int(w.ctx_lens[reqs].sum())} "
                      f"attended tokens, all {w.Hq} q-heads): tag check + append + fp64 attention, "
                      f"one step in {t:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--num-workers", type=int, default=0, help="decode waves (0 = device default)")
    ap.add_argument("--workload", default="ragged",
                    choices=["tiny", "uniform", "ragged", "long", "capacity"],
                    help="which synthetic workload (the headline is 'ragged')")
    ap.add_argument("--cache", default="e4m3", choices=["e4m3", "bf16"])
    ap.add_argument("--q-heads", type=int, default=0,
                    help="query heads per request instead of the workload's own (same kv-heads): "
                         "the GQA group size G = q-heads / kv-heads, e.g. 8 for G = 1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip bf16 variant and tag overhead")
    ap.add_argument("--overhead-rounds", type=int, default=20)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM counters)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="cycle the steps over R copies of the workload's device state so a "
                         "step's reads are not served by the 256 MB last-level cache (0 = 2 for "
                         "the uniform workload, whose cache is 538 MB, else 1)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a captured HIP graph of the step (no host launch "
                         "cost; for workloads whose GPU time is below the binding's)")
    ap.add_argument("--accuracy", action="store_true",
                    help="measure the FP8 cache's output error against the BF16 cache instead")
    ap.add_argument("--accuracy-configs", type=int, nargs="+", default=[2, 3, 4])
    ap.add_argument("--shared-prefix", action="store_true",
                    help="cache reuse study: a prompt's pages shared by 64 requests vs copies")
    ap.add_argument("--no-private", action="store_true",
                    help="--shared-prefix: skip the private-copies workload (shared pages only)")
    ap.add_argument("--cpu-study", action="store_true",
                    help="the oracle on the host, 1 thread and all cores, tiny/uniform/ragged/long")
    ap.add_argument("--qlen", type=int, default=1,
                    help="q_len > 1: speculative-verification study (q_len new tokens per "
                         "request checked in one step)")
    ap.add_argument("--loop", action="store_true",
                    help="run the multi-step decode study (tracker on vs off) instead")
    ap.add_argument("--loop-concurrency", type=int, nargs="+", default=[1, 2, 4, 8])
    ap.add_argument("--loop-prompt", type=int, default=8192)
    ap.add_argument("--loop-steps", type=int, default=1000)
    ap.add_argument("--loop-rounds", type=int, default=6)
    ap.add_argument("--loop-launch", nargs="+", default=["graph", "eager"],
                    choices=["graph", "eager"],
                    help="each step replays one captured HIP graph, or launches eagerly")
    ap.add_argument("--loop-layers", type=int, nargs="+", default=[1, 32],
                    help="layers per model step (one tag check per step, attention per layer)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus "
              f"{args.gpus}", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import decode_attention_paged_fp8kv_amd as fp8kv
    import workloads
    from workloads import device

    if args.cpu_study:
        cpu_study(args)
        return
    torch.cuda.set_device(0)
    if args.loop:
        loop_study(args)
        return
    if args.accuracy:
        accuracy_study(args)
        return
    if args.qlen > 1:
        spec_study(args)
        return
    if args.shared_prefix:
        shared_study(args)
        return
    if args.calibrate_copy:
        n = 1 << 30
        x = torch.ones(n, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                          "launches": 3}), flush=True)
        return
    cfg = {"tiny": 1, "uniform": 2, "ragged": 3, "long": 4, "capacity": 5}[args.workload]
    cache = 0 if args.cache == "e4m3" else 1
    w = workloads.make(cfg)
    if args.q_heads:
        if args.q_heads % w.Hkv:
            sys.exit(f"--q-heads {args.q_heads} is not a multiple of {w.Hkv} kv-heads")
        w.Hq = args.q_heads
        w.name = f"{w.name}_{w.Hq}q{w.Hkv}kv"
    R = args.rotate if args.rotate > 0 else (2 if cfg == 2 else 1)
    log(f"bench: building workload {w.name} ({w.B} requests, {args.cache} cache, {R} cop"
        f"{'y' if R == 1 else 'ies'})")
    states = [device.build(w, cache_dtype=cache, num_workers=args.num_workers) for _ in range(R)]
    st = states[0]
    st.step(check_tags=True)
    torch.cuda.synchronize()
    live = st.abort.cpu().numpy() == 0        # aborted requests read nothing
    step_bytes, attn_bytes = alg_bytes(w, cache, True, active=live)

    def cycle(fns):
        """A callable that runs the next copy's function on each call."""
        k = [0]

        def run():
            fns[k[0] % len(fns)]()
            k[0] += 1
        return run

    steps_ = [lambda s=s: s.step(check_tags=True) for s in states]
    # the step's two calls on their own, through the step's prepared launches
    # (for the current stream: a graph capture prepares its own)
    vas = [lambda s=s: s.prepared(True)[0]() for s in states]
    decs = [lambda s=s: s.prepared(True)[1]() for s in states]
    if args.graph:
        caps = [capture_graphs(s, [a, b, c]) for s, a, b, c in zip(states, steps_, vas, decs)]
        steps_, vas, decs = ([c[i] for c in caps] for i in range(3))
    step, verify_append, decode = cycle(steps_), cycle(vas), cycle(decs)
    verify_only = cycle([s.verify for s in states])
    for _ in range(args.warmup):
        step()
    log(f"bench: timing {args.steps} steps")
    t_step = time_steps(step, args.steps)
    per_step = sorted(event_times([step], args.steps)[0])
    p50 = per_step[len(per_step) // 2]
    p95 = per_step[min(len(per_step) - 1, int(0.95 * len(per_step)))]
    # per-kernel HIP-event times on the launch stream
    nev = max(20, args.steps // 2)
    tva, td = event_times([verify_append, decode], nev)
    tv = event_times([verify_only], nev)[0]
    t_dec = statistics.median(td) * 1e-3
    t_ver = statistics.median(tva) * 1e-3
    tokens_s = int(live.sum()) / t_step
    gbps = step_bytes / t_step / 1e9
    attn_gbps = attn_bytes / t_dec / 1e9
    res = {
        "metric": METRIC, "value": round(tokens_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"{args.cache} cache; bf16/f16 MFMA, f32 accumulate", "data": "synthetic",
        "config": {"workload": w.name, "requests": w.B, "live_requests": int(live.sum()),
                   "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": 128, "page_tokens": 16, "kv_cache": args.cache, "tag_check": True,
                   "attended_tokens": int(w.ctx_lens.sum()),
                   "decode_waves": fp8kv.decode_num_workers(st.num_workers), "parallelism": "none (1 GPU)"},
        "step_us_p50": round(p50 * 1e3, 2), "step_us_p95": round(p95 * 1e3, 2),
        "hbm_gbps": round(gbps, 1), "pct_of_8tbps": round(100 * gbps / PEAK_GBPS, 2),
        "step_alg_bytes": step_bytes,
        "roofline": {"bound": "hbm",
                     "kernel": "fp8kv_decode_attention call (decode_kernel + merge pass)",
                     "achieved": round(attn_gbps, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(attn_gbps / PEAK_GBPS, 4),
                     "traffic": counter_traffic() if (cfg == 3 and cache == 0) else None,
                     "alg_bytes_per_launch": attn_bytes,
                     "avg_launch_us": round(t_dec * 1e6, 2)},
        "tag_check_append_us": round(t_ver * 1e6, 2),
        # HIP events around one call: for kernels this short the figure includes the
        # host's launch time; the kernel-trace summaries hold the GPU times
        "tag_check_alone_us": round(statistics.median(tv) * 1e3, 2),
        "state_copies": R,
        "launch": "hip graph replay" if args.graph else "eager",
        "device": device_info(),
    }
    if not args.no_extras and cfg == 3:
        log("bench: tag-check overhead (interleaved on/off)")
        # both forms run prepared launches (one C call per kernel, no per-call
        # argument checks); enough steps per round that the host's latency
        # before a round's first kernel is amortised
        step = lambda: st.step(check_tags=True)  # noqa: E731
        off = lambda: st.step(check_tags=False)  # noqa: E731
        warm_up([step, off])
        deltas = []
        M = 50
        for r in range(args.overhead_rounds):
            a = time_steps(step, M)
            b = time_steps(off, M)
            deltas.append((a - b) / b)
        rng = np.random.default_rng(0)
        d = np.array(deltas)
        boots = [rng.choice(d, d.size).mean() for _ in range(2000)]
        res["tag_check_overhead"] = {"mean_pct": round(100 * d.mean(), 3),
                                     "ci95_pct": [round(100 * float(np.percentile(boots, 2.5)), 3),
                                                  round(100 * float(np.percentile(boots, 97.5)), 3)],
                                     "rounds": args.overhead_rounds, "steps_per_round": M}
        del st, states, steps_, vas, decs, step, verify_append, decode, verify_only
        torch.cuda.empty_cache()
        log("bench: uniform 32x8192, e4m3 vs bf16 cache")
        w2 = workloads.make(2)
        var = {}
        for cd, name in ((0, "e4m3"), (1, "bf16")):
            # two copies, alternated, as in the uniform workload's own line
            c2 = [device.build(w2, cache_dtype=cd) for _ in range(2)]
            st2 = cycle([lambda s=s: s.step(True) for s in c2])
            for _ in range(10):
                st2()
            warm_up([st2])
            t2 = time_steps(st2, 100)
            b2, a2 = alg_bytes(w2, cd, True)
            td2 = statistics.median(
                event_times([cycle([lambda s=s: s.prepared(True)[1]() for s in c2])], 50)[0]) * 1e-3
            var[name] = {"ms_per_step": round(t2 * 1e3, 4), "tokens_s": round(w2.B / t2, 1),
                         "hbm_gbps": round(b2 / t2 / 1e9, 1),
                         "attn_gbps": round(a2 / td2 / 1e9, 1)}
            del c2, st2
            torch.cuda.empty_cache()
        res["uniform_32x8192"] = var
        res["device_copy"] = device_copy()
        res["stream_read"] = stream_read()
    if not args.no_cpu_baseline and cfg == 3:
        log("bench: CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
