"""GPU: one decode step driven through the C ABI alone -- a C program
(tests/c/fp8kv_c_step.c) that takes pages from the library's pool, uploads
their tags, appends prompts, runs the fused check + append of a new token per
request and the attention, and compares abort flags, every cache byte (through
fp8kv_cache_offset) and every output row with the oracle's C functions.  No
Python or torch sits between the program and the library."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "build", "fp8kv_c_step")


def test_c_program_step_matches_oracle():
    if not os.path.exists(BIN):
        pytest.skip("tests/c/build/fp8kv_c_step is not built (__graft_entry__.build() builds it)")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "fp8kv C step: ok (abort 010" in r.stdout
