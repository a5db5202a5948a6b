"""Benchmark of the OrbitQuant online quantized-linear path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload image_qkv]

A step is one pass of the whole path over one batch of synthetic input
resident in HBM: offline weight preparation of W (rotate + quantize the
weight rows), online rotate + quantize of the activation tokens, and the
W4A4 low-bit linear.  The codebook and rotation plan are host-side
precomputations cached by the library after the first call (warmup).

Prints ONE JSON line with the throughput of the whole step (in the linear's
FLOP-equivalent TFLOP/s), per-kernel rates, the roofline of the dominant
kernel (the linear, bound by fp16 MFMA) and of rotate + quantize (bound by
HBM), and the fp64 CPU oracle timed on a bounded sample of the same
workload on this host's cores.

Inputs: seeded synthetic activations shaped like an image-DiT fused QKV
projection (2 CFG branches x 4608 tokens, d = 3072 -> 9216, 1% outlier
channels x50, per-token log-normal(0, 1.5) scale) and N(0, 0.02^2) weights,
drawn by the `workloads` generators.  Four input buffer sets are cycled so
the working set exceeds the 256 MB Infinity Cache.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, 2.5 PFLOP/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="image_qkv")
    p.add_argument("--linear", default=None, help="linear name inside the workload")
    p.add_argument("--bits", default=None, help="w,a bits (default: the workload's first pair)")
    p.add_argument("--sets", type=int, default=4, help="input buffer sets cycled")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=9216)
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="before the steps, copy a buffer of this many MiB once (untimed), "
                        "as the known-size reference for HBM byte counters")
    return p.parse_args()


def src_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "quantization_dit_linear_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, digest):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(kernel)
    if not e or e.get("source_digest") != digest:
        return None
    return e.get("bytes_per_launch")


def to_dev(x):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def cpu_baseline(cfg, lin, bw, ba, rows_n):
    """The fp64 oracle, as it stands, on a bounded sample: weight prep of all
    N weight rows, rotate + quantize and the linear for `rows_n` of the M
    token rows; the full step is extrapolated linearly in token rows."""
    import oracle
    import workloads as wl
    M, N, K = lin.act.M, lin.weight.N, lin.act.d
    rows = wl.sample_rows(M, rows_n, 5)
    x = wl.activations(cfg, lin.name, rows)
    W = wl.weights(cfg, lin.name)
    t0 = time.perf_counter()
    wc, wn, _ = oracle.rotate_quantize(W, lin.weight.dtype, K, lin.seed, bw)
    t1 = time.perf_counter()
    ac, an, _ = oracle.rotate_quantize(x, lin.act.dtype, K, lin.seed, ba)
    t2 = time.perf_counter()
    oracle.linear(ac, an, ba, wc, wn, bw, K)
    t3 = time.perf_counter()
    scale = M / len(rows)
    t_step = (t1 - t0) + ((t2 - t1) + (t3 - t2)) * scale
    flops = 2.0 * M * N * K
    return {
        "value": flops / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"weight prep of all {N} weight rows + rotate-quantize and linear of "
                   f"{len(rows)} of {M} token rows (seeded sample), fp64; full step "
                   f"extrapolated linearly in token rows"),
        "seconds_measured": round(t3 - t0, 3),
        "step_seconds_extrapolated": round(t_step, 3),
    }


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}): this build has no "
              "multi-GPU path; see the sharding notes in DESIGN.md", flush=True)
        return 2
    import torch
    import quantization_dit_linear_amd as q
    import workloads as wl

    cfg = a.workload
    lin = wl.CONFIGS[cfg]["linears"][0] if a.linear is None else wl.get_linear(cfg, a.linear)
    bw, ba = lin.bit_pairs[0] if a.bits is None else tuple(int(v) for v in a.bits.split(","))
    M, N, K = lin.act.M, lin.weight.N, lin.act.d
    torch.cuda.set_device(0)

    x_np = wl.activations(cfg, lin.name)
    W_np = wl.weights(cfg, lin.name)
    xs = [to_dev(x_np)]
    Ws = [to_dev(W_np)]
    for i in range(1, a.sets):
        # distinct buffers with the same distribution: circular row shifts
        xs.append(torch.roll(xs[0], shifts=97 * i, dims=0).contiguous())
        Ws.append(torch.roll(Ws[0], shifts=89 * i, dims=0).contiguous())
    dev = xs[0].device
    wc = [torch.empty((N, K * bw // 8), dtype=torch.uint8, device=dev) for _ in range(a.sets)]
    wn = [torch.empty((N,), dtype=torch.float32, device=dev) for _ in range(a.sets)]
    ac = [torch.empty((M, K * ba // 8), dtype=torch.uint8, device=dev) for _ in range(a.sets)]
    an = [torch.empty((M,), dtype=torch.float32, device=dev) for _ in range(a.sets)]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        s = i % a.sets
        if ev is not None:
            ev[0].record(stream)
        q.prepare_weights(Ws[s], lin.seed, bw, out=wc[s], norms=wn[s])
        if ev is not None:
            ev[1].record(stream)
        q.rotate_quantize(xs[s], lin.seed, ba, out=ac[s], norms=an[s])
        if ev is not None:
            ev[2].record(stream)
        q.linear(ac[s], an[s], ba, wc[s], wn[s], bw, K, out=y)
        if ev is not None:
            ev[3].record(stream)

    if a.calib_copy_mib > 0:
        n = a.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(a.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(a.steps):
        step(i, evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / a.steps
    t_prep = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    t_rot = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    t_lin = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))

    flops = 2.0 * M * N * K
    in_b = 2 if lin.act.dtype == wl.BF16 else 4
    rot_bytes = M * (K * in_b + K * ba / 8 + 4)
    prep_bytes = N * (K * (2 if lin.weight.dtype == wl.BF16 else 4) + K * bw / 8 + 4)
    lin_tflops = flops / (t_lin * 1e-3) / 1e12
    rot_gbs = rot_bytes / (t_rot * 1e-3) / 1e9
    prep_gbs = prep_bytes / (t_prep * 1e-3) / 1e9

    lin_digest = src_digest("linear.hip")
    rot_digest = src_digest("rotate_quantize.hip", "rotate_quantize_fast.hip") if os.path.exists(
        os.path.join(ROOT, "quantization_dit_linear_amd", "csrc", "rotate_quantize_fast.hip")) \
        else src_digest("rotate_quantize.hip")

    out = {
        "metric": "rotate+quant GB/s and W4A4 linear TFLOP/s, as % of HBM / MFMA peak",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "dtype_detail": "linear: fp16 MFMA operands (unit-variance levels), fp32 accumulate, "
                        "bf16 output; rotate+quantize: fp32",
        "data": "synthetic",
        "config": {"workload": f"{cfg}/{lin.name}: {M} tokens, d_in {K} -> d_out {N}, "
                               f"W{bw}A{ba}, activations "
                               f"{'bf16' if lin.act.dtype == wl.BF16 else 'fp32'}",
                   "M": M, "N": N, "K": K, "w_bits": bw, "a_bits": ba},
        "kernels": {
            "linear": {"ms": round(t_lin, 4), "TFLOP/s": round(lin_tflops, 2),
                       "frac_of_mfma_fp16_peak": round(lin_tflops / MFMA_FP16_PEAK_TFLOPS, 4)},
            "rotate_quantize": {"ms": round(t_rot, 4), "GB/s": round(rot_gbs, 1),
                                "frac_of_hbm_peak": round(rot_gbs / HBM_PEAK_GBS, 4)},
            "prepare_weights": {"ms": round(t_prep, 4), "GB/s": round(prep_gbs, 1),
                                "frac_of_hbm_peak": round(prep_gbs / HBM_PEAK_GBS, 4)},
        },
        "roofline": {"bound": "mfma", "achieved": round(lin_tflops, 2),
                     "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(lin_tflops / MFMA_FP16_PEAK_TFLOPS, 4),
                     "traffic": stored_traffic("linear", lin_digest)},
        "roofline_rotate_quantize": {"bound": "hbm", "achieved": round(rot_gbs, 1),
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(rot_gbs / HBM_PEAK_GBS, 4),
                                     "traffic": stored_traffic("rotate_quantize", rot_digest)},
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, lin, bw, ba, a.cpu_rows)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
