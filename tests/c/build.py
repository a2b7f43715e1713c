"""Build the C-ABI step test (tests/c/fp8kv_c_step.c) with gcc against the
built libfp8kv.so, the oracle's library and the HIP runtime.  Needs both
libraries built first; the binary lands in tests/c/build/."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "fp8kv_c_step.c")
OUT_DIR = os.path.join(HERE, "build")
BIN = os.path.join(OUT_DIR, "fp8kv_c_step")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    pkg = os.path.join(ROOT, "decode_attention_paged_fp8kv_amd")
    orc = os.path.join(ROOT, "oracle")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"),
           "-o", BIN + ".tmp", SRC,
           "-L" + pkg, "-lfp8kv", "-L" + orc, "-loracle", "-L" + os.path.join(ROCM, "lib"),
           "-lamdhip64", "-lm",
           # found next to the binary wherever the tree is copied
           "-Wl,-rpath,$ORIGIN/../../../decode_attention_paged_fp8kv_amd",
           "-Wl,-rpath,$ORIGIN/../../../oracle", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
