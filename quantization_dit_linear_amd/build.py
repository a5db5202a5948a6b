"""Build liborbitquant.so in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-fp32 instruction selection turned
off (no v_pk_{add,mul,fma}_f32 in the output).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liborbitquant.so")
SOURCES = ["oq_host.cpp", "rotate_quantize.hip", "rotate_quantize_fast.hip", "linear.hip"]
ARCH = os.environ.get("OQ_OFFLOAD_ARCH", "gfx950")


def build(verbose: bool = False, extra=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    cmd = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *extra, *srcs, "-o", OUT + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError("hipcc failed")
    if verbose and err.strip():
        sys.stderr.write(err + "\n")
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
