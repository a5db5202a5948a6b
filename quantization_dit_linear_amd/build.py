"""Build liborbitquant.so in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-fp32 instruction selection turned
off (no v_pk_{add,mul,fma}_f32 in the output).
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liborbitquant.so")
SOURCES = ["oq_host.cpp", "rotate_quantize.hip", "rotate_quantize_fast.hip", "linear.hip",
           "adaln_rtn4.hip", "diag.hip"]
# per-source extra flags: the rotate kernel keeps its MFMA results in
# ordinary VGPRs (no accumulation-register round trip per value)
PER_SOURCE = {"rotate_quantize_fast.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = os.environ.get("OQ_OFFLOAD_ARCH", "gfx950")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("'-packed-fp32-ops' is not a recognized feature for this target",
             "argument unused during compilation: '--hip-link'")
    err = "\n".join(l for l in res.stderr.splitlines() if not any(n in l for n in noise))
    if res.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))
    if verbose and err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source to an object (per-source flags), link the .so."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(BUILD_DIR, exist_ok=True)
    common = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wall", "-Wno-unused-function",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC, *extra]
    objs = [os.path.join(BUILD_DIR, s + ".o") for s in SOURCES]
    cmds = [common + PER_SOURCE.get(s, []) + ["-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    # the sources compile independently: one hipcc per source, in parallel
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "8"))))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", OUT + ".tmp"],
         verbose)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
