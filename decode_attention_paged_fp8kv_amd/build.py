"""Build libfp8kv.so (HIP, gfx950) in-tree with hipcc.

Flags: -O3 for gfx950 only; packed-fp32 instruction selection disabled;
correctly rounded fp32 division (quantize-on-append relies on it); no
fast-math.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8kv.so")
SOURCES = [os.path.join(CSRC, "fp8kv_kernels.hip"), os.path.join(CSRC, "fp8kv_pool.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    # keep MFMA accumulators in ordinary VGPRs: the online-softmax rescale
    # multiplies them on the VALU, and AGPR accumulators would be copied
    # back and forth around every MFMA
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def build(verbose: bool = False, extra=None, out: str = LIB) -> str:
    cmd = [HIPCC] + FLAGS + (extra or []) + ["-x", "hip"] + SOURCES + ["-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msg)
    if verbose and msg:
        print(msg, flush=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
