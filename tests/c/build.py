"""Build the C test programs with gcc: the exhaustive e4m3 encoder pin
(tests/c/e4m3_every_binary32.c, against the oracle's library) and the C-ABI
step test (tests/c/fp8kv_c_step.c, against the built libfp8kv.so, the oracle's
library and the HIP runtime).  Needs the libraries built first; the binaries
land in tests/c/build/."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "fp8kv_c_step.c")
OUT_DIR = os.path.join(HERE, "build")
BIN = os.path.join(OUT_DIR, "fp8kv_c_step")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


E4M3_SRC = os.path.join(HERE, "e4m3_every_binary32.c")
E4M3_BIN = os.path.join(OUT_DIR, "e4m3_every_binary32")


def build_e4m3(verbose: bool = False) -> str:
    """The exhaustive encoder pin (CPU only: gcc + OpenMP + the oracle's library)."""
    os.makedirs(OUT_DIR, exist_ok=True)
    orc = os.path.join(ROOT, "oracle")
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-Wall", "-Wextra",
           "-o", E4M3_BIN + ".tmp", E4M3_SRC, "-L" + orc, "-loracle", "-lm",
           "-Wl,-rpath,$ORIGIN/../../../oracle"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(E4M3_BIN + ".tmp", E4M3_BIN)
    return E4M3_BIN


def build(verbose: bool = False) -> str:
    build_e4m3(verbose)
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
