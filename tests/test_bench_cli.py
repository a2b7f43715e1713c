"""Host: bench.py's contract that needs no GPU.  Asked for more than one GPU
it stops at once with a message (it has no multi-GPU path) and before it
imports torch or touches a device; the committed HBM counter summaries it
reports from stay within 10% of the algorithmic bytes."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n),
                        "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and f"--gpus {n}" in r.stderr
    assert r.stdout == ""      # no JSON line for a run that did not happen


def test_committed_hbm_counters_match_the_algorithmic_bytes():
    """The HBM counter summaries in profiles/ (FETCH_SIZE + WRITE_SIZE of the
    decode call, calibrated on a plain copy) stay within 10% of the call's
    algorithmic bytes on every workload of 0.5 GB or more: no re-reads.  Each
    names the kernel source it was taken on, and the benchmark reports the
    ragged workload's figure only while that source is current."""
    import glob
    import re
    import bench
    files = glob.glob(os.path.join(ROOT, "profiles", "*_hbm_counters.txt"))
    assert files
    ratios = []
    for f in files:
        text = open(f).read()
        assert re.search(r"^kernel_source_sha256: [0-9a-f]{64}$", text, re.M), f
        ratios += [float(x) for x in re.findall(r"^traffic_over_algorithmic: ([0-9.]+)$", text, re.M)]
    assert len(ratios) >= 5 and all(0.9 <= r <= 1.1 for r in ratios), ratios
    import workloads
    t = bench.counter_traffic()
    attn = bench.alg_bytes(workloads.make(3), 0, True)[1]
    assert t is None or 0.9 <= t / attn <= 1.1
