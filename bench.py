"""Benchmark of the OrbitQuant online quantized-linear path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload video_block]

A step is one pass of the online path over one batch of synthetic input
resident in HBM: rotate + quantize of the activation tokens, then the W4A4
low-bit linear against weight codes prepared offline.  Weight preparation
(rotate + quantize of the weight rows) runs once before the timed region,
as it would when a layer is loaded, and is timed on its own.  The codebook
and rotation plan are host-side precomputations cached by the library after
the first call.  Before the W warm-up steps, untimed settle steps run for
about --settle-ms (200 ms by default), so the timed steps see the clocks of
a GPU under this load rather than of one just out of idle.

Prints ONE JSON line with the throughput of the step (in the linear's
FLOP-equivalent TFLOP/s), per-kernel rates, the roofline of the dominant
kernel (the linear, bound by fp16 MFMA) and of rotate + quantize (bound by
HBM), the same step on the image-DiT QKV shape, and the fp64 CPU oracle
timed on a bounded sample of the same workload on this host's cores.

Inputs: seeded synthetic activations shaped like a video-DiT block's fused
QKV projection (21 x 30 x 52 = 32760 latent tokens, d = 5120 -> 15360, 1%
outlier channels x50, per-token log-normal(0, 2) scale) and N(0, 0.02^2)
weights, drawn by the `workloads` generators.  Activation buffer sets are
cycled so rotate + quantize reads its input from HBM, not the 256 MB
Infinity Cache (the linear's 1 GB output also evicts it every step).

Other modes:
    python bench.py --sweep           every workload instance and bit pair at
                                      full size, one JSON line each
    python bench.py --summarize-profiles KT FETCH WRITE [--profile-counters ...]
                                      rocprofv3 output -> profiles/ summaries
                                      and the workload's traffic.json entry
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
# Untimed steps before the warm-up steps, in ms of load.  From idle the
# part's clocks need tens of milliseconds of this load to settle: at
# 9216 x 9216 x 3072 the linear's first calls took 480 us, the next ten
# 550-600 us, and it settled at 447 us after about 50 ms.
SETTLE_MS = 200.0
MFMA_FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, 2.5 PFLOP/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="video_block")
    p.add_argument("--linear", default=None, help="linear name inside the workload")
    p.add_argument("--bits", default=None, help="w,a bits (default: the workload's first pair)")
    p.add_argument("--sets", type=int, default=2, help="activation buffer sets cycled")
    p.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                   help="before the warm-up steps, untimed steps for about this long, so the "
                        "clocks settle at their loaded state (0: none)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=3072,
                   help="token rows of the oracle's sample (rotate + quantize and the linear)")
    p.add_argument("--no-second-shape", action="store_true",
                   help="skip the same step on the image-DiT QKV shape")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="before the steps, copy a buffer of this many MiB once (untimed), "
                        "as the known-size reference for HBM byte counters")
    p.add_argument("--no-ref-gemm", action="store_true",
                   help="skip timing the library fp16 GEMM of the linear's shape and the "
                        "fake-quantization path")
    p.add_argument("--summarize-profiles", nargs=3, metavar=("KT_DIR", "FETCH_DIR", "WRITE_DIR"),
                   help="no benchmark: turn rocprofv3 output of this workload (kernel trace, "
                        "FETCH_SIZE and WRITE_SIZE runs) into the summaries under profiles/")
    p.add_argument("--profile-command", default="",
                   help="with --summarize-profiles: the rocprofv3 commands, recorded verbatim")
    p.add_argument("--profile-counters", nargs="*", default=[],
                   help="with --summarize-profiles: rocprofv3 --pmc output folders whose "
                        "per-kernel counter averages go into profiles/<workload>_counters.txt")
    p.add_argument("--profile-bench-log", default=None,
                   help="with --summarize-profiles: output of the traced bench.py run, whose "
                        "own per-kernel event timings are compared with the trace")
    p.add_argument("--prep-launches", type=int, default=None,
                   help="with --summarize-profiles: leading rotate-kernel dispatches that "
                        "prepared weights (default: what bench.py launches, 1 + 5)")
    p.add_argument("--profile-out", default=os.path.join(ROOT, "profiles"),
                   help="with --summarize-profiles: folder for the summaries and traffic.json")
    p.add_argument("--sweep", action="store_true",
                   help="no step benchmark: time rotate+quantize and the linear of every "
                        "workload instance and bit pair at full size, one JSON line each")
    return p.parse_args()


# sources of the kernels whose counters profiles/traffic.json records: the
# linear, and the bf16 fast rotate kernel that every recorded workload runs
# (with the header of constants both share with the host)
LIN_SRC = ("linear.hip", "oq_internal.h")
ROT_SRC = ("rotate_quantize_fast.hip", "oq_internal.h")


def src_digest(*names):
    """Digest of kernel sources with comments and blank lines dropped, so
    stored counter data stays valid across comment-only edits and goes
    stale on any code change."""
    import re
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "quantization_dit_linear_amd", "csrc", n)) as f:
            txt = f.read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        txt = re.sub(r"//[^\n]*", "", txt)
        h.update("\n".join(l.rstrip() for l in txt.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def stored_traffic(tag, kernel, digest):
    """HBM bytes per launch from the committed counter summary of workload
    `tag`, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(tag, {}).get(kernel)
    if not e or e.get("source_digest") != digest:
        return None
    return e.get("bytes_per_launch")


def to_dev(x):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def _oracle_stages(cfg, lin, bw, ba, w_rows, x_rows, lin_rows):
    """Seconds of the oracle's three stages on seeded samples: weight prep
    of w_rows weight rows, rotate + quantize of x_rows token rows, and the
    linear of the first lin_rows of those token rows against all N rows."""
    import oracle
    import workloads as wl
    M, N, K = lin.act.M, lin.weight.N, lin.act.d
    rows = wl.sample_rows(M, x_rows, 5)
    x = wl.activations(cfg, lin.name, rows)
    W = wl.weights(cfg, lin.name)
    Wp = W if w_rows >= N else W[:w_rows]
    t0 = time.perf_counter()
    wc, wn, _ = oracle.rotate_quantize(Wp, lin.weight.dtype, K, lin.seed, bw)
    t1 = time.perf_counter()
    ac, an, _ = oracle.rotate_quantize(x, lin.act.dtype, K, lin.seed, ba)
    t2 = time.perf_counter()
    if wc.shape[0] < N:  # the linear needs every weight row: tile the sample
        reps = -(-N // wc.shape[0])
        wc, wn = np.tile(wc, (reps, 1))[:N], np.tile(wn, reps)[:N]
    oracle.linear(ac, an, ba, wc, wn, bw, K, rows=np.arange(min(lin_rows, len(rows))))
    t3 = time.perf_counter()
    return len(Wp), len(rows), min(lin_rows, len(rows)), t1 - t0, t2 - t1, t3 - t2


def cpu_baseline(cfg, lin, bw, ba, rows_n):
    """The fp64 oracle, as it stands, on a bounded sample of the same
    workload: weight prep of all N weight rows (offline, reported on its
    own), then rotate + quantize and the linear for a seeded sample of
    `rows_n` of the M token rows; the online step is extrapolated linearly
    in token rows.  Also the per-stage rates (weight prep and rotate +
    quantize in GB/s over the same algorithmic bytes as the GPU figures,
    the linear in GFLOP/s), and the same on one thread on a smaller
    sample."""
    import oracle
    import workloads as wl
    M, N, K = lin.act.M, lin.weight.N, lin.act.d
    e_w = 2 if lin.weight.dtype == wl.BF16 else 4
    e_a = 2 if lin.act.dtype == wl.BF16 else 4

    def rates(nw, nx, nl, tw, tx, tl):
        return {"prepare_weights_GB/s": round(nw * (K * e_w + K * bw / 8 + 4) / tw / 1e9, 3),
                "rotate_quantize_GB/s": round(nx * (K * e_a + K * ba / 8 + 4) / tx / 1e9, 3),
                "linear_GFLOP/s": round(2.0 * nl * N * K / tl / 1e9, 2)}

    nw, nx, nl, tw, tx, tl = _oracle_stages(cfg, lin, bw, ba, N, rows_n, rows_n)
    t_step = tx * (M / nx) + tl * (M / nl)
    out = {
        "value": 2.0 * M * N * K / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"rotate-quantize and linear (against all {N} weight rows) of {nx} of "
                   f"{M} token rows (seeded sample), fp64; the online step extrapolated "
                   f"linearly in token rows; weight prep of all {N} rows timed apart"),
        "seconds_measured": round(tw + tx + tl, 3),
        "step_seconds_extrapolated": round(t_step, 3),
        "prepare_weights_seconds": round(tw, 3),
        "stages": rates(nw, nx, nl, tw, tx, tl),
    }
    threads = oracle.num_threads()
    try:
        oracle.set_threads(1)
        one = _oracle_stages(cfg, lin, bw, ba, min(N, 1024), min(M, 256), 8)
    finally:
        oracle.set_threads(threads)
    out["one_thread"] = dict(rates(*one), sample=(
        f"{one[0]} weight rows, {one[1]} token rows rotated, {one[2]} token rows through "
        f"the linear"), seconds_measured=round(sum(one[3:]), 3))
    return out


def library_fp16_gemm(M, N, K, iters=10):
    """Context, not part of the path: the vendor library's dense fp16 GEMM
    (torch.matmul) on the linear's shape, fp16 in and out, random operands.
    It does no decoding, so it is a practical ceiling for the linear."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    x = torch.randn((M, K), generator=g, device="cuda").to(torch.float16)
    w = torch.randn((N, K), generator=g, device="cuda").to(torch.float16)
    for _ in range(2):
        y = x @ w.t()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        y = x @ w.t()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    del x, w, y
    return {"what": "torch.matmul fp16 x fp16 -> fp16, same M, N, K (vendor library GEMM)",
            "ms": round(ms, 4), "TFLOP/s": round(2.0 * M * N * K / ms / 1e9, 1)}


def fake_quant_path(q, x, W, seed, ba, bw, iters=10):
    """Context: the pages' own evaluation path on the same inputs -- the
    weights fake-quantized offline to bf16 by the library (oq_rotate_quantize
    with OQ_OUT_BF16_DEQUANT, then transposed once), and per step the tokens
    fake-quantized the same way followed by the vendor bf16 GEMM."""
    import torch
    M, K = x.shape
    N = W.shape[0]
    xh = torch.empty((M, K), dtype=torch.bfloat16, device=x.device)
    xn = torch.empty((M,), dtype=torch.float32, device=x.device)
    wh, _ = q.fake_quantize(W, seed, bw)
    wt = wh.t().contiguous()
    del wh

    def run():
        q.fake_quantize(x, seed, ba, out=xh, norms=xn)
        return torch.mm(xh, wt)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    del wt, xh, xn
    return {"what": "fake-quantize x to bf16 (library) and a vendor bf16 GEMM against the "
                    "weights fake-quantized and transposed offline",
            "ms": round(ms, 4)}


def w8a8_path(q, x, W, seed, iters=10):
    """The same online step at 8 bits on both sides (W8A8, the top of the
    pages' bit range): rotate + quantize to byte codes and the W8A8 linear
    against weights prepared offline; per-kernel times from events on the
    launch stream."""
    import torch
    M, K = x.shape
    N = W.shape[0]
    ac = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    an = torch.empty((M,), dtype=torch.float32, device=x.device)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    wc, wn = q.prepare_weights(W, seed, 8)
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(iters)]

    def run(e=None):
        if e is not None:
            e[0].record(stream)
        q.rotate_quantize(x, seed, 8, out=ac, norms=an)
        if e is not None:
            e[1].record(stream)
        q.linear(ac, an, 8, wc, wn, 8, K, out=y)
        if e is not None:
            e[2].record(stream)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    for i in range(iters):
        run(ev[i])
    torch.cuda.synchronize()
    t_step = float(np.median([e[0].elapsed_time(e[2]) for e in ev]))
    t_rot = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    t_lin = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
    in_b = x.element_size()
    rot_gbs = M * (K * in_b + K + 4) / (t_rot * 1e-3) / 1e9
    lin_tf = 2.0 * M * N * K / (t_lin * 1e-3) / 1e12
    del ac, an, y, wc, wn
    return {"what": "W8A8 online step on the same inputs (medians over launches)",
            "step_ms": round(t_step, 4),
            "linear": {"ms": round(t_lin, 4), "TFLOP/s": round(lin_tf, 1),
                       "frac_of_mfma_fp16_peak": round(lin_tf / MFMA_FP16_PEAK_TFLOPS, 4)},
            "rotate_quantize": {"ms": round(t_rot, 4), "GB/s": round(rot_gbs, 1),
                                "frac_of_hbm_peak": round(rot_gbs / HBM_PEAK_GBS, 4)}}


def measured_ceilings(q):
    """The ceilings measured on this GPU beside the datasheet peaks: the
    library's matrix-core probe (back-to-back independent fp16 MFMAs, no
    memory traffic) and a 1 GiB device-to-device copy (HBM read + write)."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 2 * cus
    sink = torch.empty((blocks * 512,), dtype=torch.float32, device="cuda")
    q.diag_mfma_f16(blocks, 100, sink)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    iters = 4000
    e0.record()
    flop = q.diag_mfma_f16(blocks, iters, sink)
    e1.record()
    torch.cuda.synchronize()
    mfma_tf = flop / (e0.elapsed_time(e1) * 1e-3) / 1e12
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    reps = 5
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * (1 << 30) / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    del src, dst, sink
    return {"mfma_f16_probe_TFLOP/s": round(mfma_tf, 1),
            "copy_1GiB_GB/s": round(copy_gbs, 1),
            "what": "fp16 MFMA probe (orbitquant_diag.h, 2 workgroups per CU, 32 independent "
                    "accumulators per wave) and a 1 GiB device copy counted as read + write"}


def adaln_rtn4(q, name, iters=50):
    """The AdaLN modulation projection of the same model size with INT4
    weight-only RTN weights (oq_rtn4_linear), HBM-bound: weight nibbles +
    scales + activations + outputs per launch."""
    import torch
    import workloads as wl
    x_np, W_np = wl.adaln_inputs(name)
    x, W = to_dev(x_np), to_dev(W_np)
    q4, sc = q.rtn4_prepare_weights(W)
    M, K = x.shape
    N = W.shape[0]
    # four copies of the prepared weights (4 x 78.6 MB at the video shape),
    # cycled, so a launch does not find its weights in the 256 MB Infinity
    # Cache left there by the launch before
    sets = [(q4, sc)] + [(q4.clone(), sc.clone()) for _ in range(3)]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    for i in range(3):
        q.rtn4_linear(x, *sets[i % len(sets)], out=y)
    torch.cuda.synchronize()
    # a launch takes a few microseconds on the GPU and more on the host side
    # (Python, ctypes): replay the launches from a captured HIP graph so the
    # timing is the GPU's
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(iters):
            q.rtn4_linear(x, *sets[i % len(sets)], out=y)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 4
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (iters * reps)
    byts = N * K / 2 + 4 * N + 2 * M * K + 2 * M * N
    gbs = byts / (ms * 1e-3) / 1e9
    return {"shape": f"{M} x {K} -> {N} ({name} DiT block)", "ms": round(ms, 5),
            "timing": "HIP graph of back-to-back launches over 4 weight copies",
            "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


LINEAR_KERNELS = ("linear_kernel", "tail_reduce_kernel")  # the kernels of one linear call


def _short_kernel_name(name):
    n = name.replace("(anonymous namespace)::", "").replace("oq::", "")
    if "(" in n:
        n = n[:n.index("(")]
    return n.replace("void ", "").strip()


def _step_launches(line):
    """Activation launches of the steps one bench line ran: settle, warm-up
    and timed steps (None for a line without step counts)."""
    if "steps" not in line or "warmup" not in line:
        return None
    return int(line["steps"]) + int(line["warmup"]) + int(line.get("settle", {}).get("steps", 0))


def _split_rotate(rows, n_prep, n_act=None):
    """Rotate-kernel rows of a rocprofv3 csv in dispatch order -> (weight
    preparation rows, activation rows): the first n_prep dispatches of the
    workload's rotate kernel prepared the weights (bench.py launches them
    before any activation); with n_act, only the next n_act dispatches (the
    steps' own launches, not the back-to-back ones timed after them) count
    as activation rows."""
    order = sorted(rows, key=lambda r: int(r.get("Dispatch_Id") or 0))
    disp = sorted({int(r.get("Dispatch_Id") or i) for i, r in enumerate(order)})
    prep_ids = set(disp[:n_prep])
    act_ids = set(disp[n_prep:] if n_act is None else disp[n_prep:n_prep + n_act])
    prep = [r for i, r in enumerate(order) if int(r.get("Dispatch_Id") or i) in prep_ids]
    act = [r for i, r in enumerate(order) if int(r.get("Dispatch_Id") or i) in act_ids]
    return prep, act


def summarize_profiles(a):
    """Write profiles/<workload>_kernel_stats.txt, _traffic.txt and the
    traffic table bench.py reads, from rocprofv3 csv output."""
    import csv
    import glob
    import workloads as wl
    cfg = a.workload
    lin = wl.CONFIGS[cfg]["linears"][0] if a.linear is None else wl.get_linear(cfg, a.linear)
    bw, ba = lin.bit_pairs[0] if a.bits is None else tuple(int(v) for v in a.bits.split(","))
    M, N, K = lin.act.M, lin.weight.N, lin.act.d
    in_b = 2 if lin.act.dtype == wl.BF16 else 4
    tag = f"{cfg}_w{bw}a{ba}"
    n_prep = (1 + PREP_TIMED) if a.prep_launches is None else a.prep_launches
    kt_dir, f_dir, w_dir = a.summarize_profiles

    def one(pattern, d, required=True):
        files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
        if not files:
            if required:
                raise SystemExit(f"no {pattern} under {d}")
            return None
        return files[0]

    rows = list(csv.DictReader(open(one("*kernel_stats.csv", kt_dir))))
    lines = []
    for r in rows:
        lines.append((_short_kernel_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                      float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    # one linear call: the full-round kernel, plus (when a sparse last round
    # of tiles is cut into K ranges) the pieces' kernel and their reduction
    lin_parts = [n for n, *_ in lines if n.startswith(LINEAR_KERNELS)]
    lin_name = " + ".join(lin_parts)
    rot_name = next(n for n, *_ in lines if n.startswith(f"rq_fast_kernel<{K},")
                    or n.startswith("rq_"))
    # per-dispatch durations of the rotate kernel: weight preparation apart
    trace = one("*kernel_trace.csv", kt_dir, required=False)
    rot_act_us = rot_prep_us = None
    if trace:
        tr = [r for r in csv.DictReader(open(trace))
              if _short_kernel_name(r["Kernel_Name"]) == rot_name]
        n_act = None
        if a.profile_bench_log:  # the steps' own launches
            jl = json.loads([l for l in open(a.profile_bench_log) if l.startswith("{")][-1])
            n_act = _step_launches(jl)
        prep, act = _split_rotate(tr, n_prep, n_act)
        dur = lambda rs: [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs]
        if act:
            rot_act_us = float(np.mean(dur(act)))
        if prep:
            rot_prep_us = float(np.mean(dur(prep)))
    with open(os.path.join(a.profile_out, f"{tag}_kernel_stats.txt"), "w") as f:
        f.write(f"Kernel timing on one MI355X (gfx950), workload {cfg}/{lin.name}: {M} tokens, "
                f"d_in {K} -> d_out {N}, W{bw}A{ba}.\nCommands (repository root on the GPU "
                f"host):\n{a.profile_command}\n\n")
        f.write(f"{'kernel':70s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} "
                f"{'pct':>6s}\n")
        for n, c, av, mn, mx, pc in lines:
            f.write(f"{n[:70]:70s} {c:6d} {av:9.1f} {mn:9.1f} {mx:9.1f} {pc:6.2f}\n")
        lin_sum = sum(av for n, c, av, *_ in lines if n in lin_parts)
        f.write(f"\nlinear call = {lin_name}: {lin_sum:.1f} us per call; 2*{M}*{N}*{K} = "
                f"{2.0 * M * N * K:.4g} flop per call -> "
                f"{2.0 * M * N * K / (lin_sum * 1e-6) / 1e12:.1f} TFLOP/s\n")
        rot_alg = M * (K * in_b + K * ba / 8 + 4)
        f.write(f"{rot_name}: {M} activation rows x ({K}*{in_b} + {K}*{ba}/8 + 4) = "
                f"{rot_alg:.4g} algorithmic bytes per launch")
        if rot_act_us is not None:
            f.write(f"; activation launches of the steps (after the first {n_prep} "
                    f"dispatches, which prepared the {N} weight rows) average "
                    f"{rot_act_us:.1f} us -> "
                    f"{rot_alg / (rot_act_us * 1e-6) / 1e9:.1f} GB/s")
            if rot_prep_us is not None:
                f.write(f"; weight preparation {rot_prep_us:.1f} us")
        f.write("\n")
        if a.profile_bench_log:
            line = [l for l in open(a.profile_bench_log) if l.startswith("{")][-1]
            kb = json.loads(line)["kernels"]
            f.write(f"\nAgreement: in the traced run bench.py's own HIP events (on the stream "
                    f"the kernels run on) averaged {kb['linear']['ms'] * 1e3:.1f} us per linear "
                    f"call vs {lin_sum:.1f} us of its kernels in the trace; rotate+quantize "
                    f"{kb['rotate_quantize']['ms'] * 1e3:.1f} us"
                    + (f" vs {rot_act_us:.1f} us" if rot_act_us is not None else "")
                    + " (events include the gaps between launches).\n")

    def counters(d, cname):
        per = {}
        for r in csv.DictReader(open(one("*counter_collection.csv", d))):
            if r["Counter_Name"] != cname:
                continue
            per.setdefault(r["Kernel_Name"], []).append(r)
        return per

    fetch, write = counters(f_dir, "FETCH_SIZE"), counters(w_dir, "WRITE_SIZE")

    def calib(per):
        copies = [(int(r["Grid_Size"]), float(r["Counter_Value"]))
                  for k, vals in per.items() if "copyBuffer" in k for r in vals]
        if not copies:
            raise SystemExit("no copy kernel in the counter run (use --calib-copy-mib)")
        return max(copies)[1]  # the largest copy: the calibration buffer

    f_ref, w_ref = calib(fetch), calib(write)
    copy_kib = 1024 * 1024  # 1 GiB read and written by the calibration copy
    f_scale, w_scale = copy_kib / f_ref, copy_kib / w_ref

    def kib_per_call(per, prefixes):
        # every kernel of a call runs once per call: the sum of their means
        names = {_short_kernel_name(k) for k in per if _short_kernel_name(k).startswith(prefixes)}
        return sum(float(np.mean([float(r["Counter_Value"]) for k, vs in per.items()
                                  if _short_kernel_name(k) == n for r in vs])) for n in names)

    def rot_act(per):
        rs = [r for k, vs in per.items() if _short_kernel_name(k) == rot_name for r in vs]
        return float(np.mean([float(r["Counter_Value"])
                              for r in _split_rotate(rs, n_prep)[1]]))

    lin_fetch = kib_per_call(fetch, LINEAR_KERNELS) * 1024 * f_scale
    lin_write = kib_per_call(write, LINEAR_KERNELS) * 1024 * w_scale
    rot_fetch = rot_act(fetch) * 1024 * f_scale
    rot_write = rot_act(write) * 1024 * w_scale
    lin_alg_r = M * K * ba / 8 + N * K * bw / 8 + 4 * (M + N)
    lin_alg_w = 2 * M * N
    rot_alg_r = M * K * in_b
    rot_alg_w = M * (K * ba / 8 + 4)
    lin_digest = src_digest(*LIN_SRC)
    rot_digest = src_digest(*ROT_SRC)
    table = {
        "linear": {"kernel": lin_name, "source_digest": lin_digest,
                   "bytes_per_launch": int(lin_fetch + lin_write), "fetch_bytes": int(lin_fetch),
                   "write_bytes": int(lin_write), "algorithmic_read_bytes": int(lin_alg_r),
                   "algorithmic_write_bytes": int(lin_alg_w)},
        "rotate_quantize": {"kernel": rot_name, "source_digest": rot_digest,
                            "bytes_per_launch": int(rot_fetch + rot_write),
                            "fetch_bytes": int(rot_fetch), "write_bytes": int(rot_write),
                            "algorithmic_read_bytes": int(rot_alg_r),
                            "algorithmic_write_bytes": int(rot_alg_w),
                            "note": f"activation launches only (the first {n_prep} "
                                    f"dispatches prepared the weights)"},
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)}
    # one entry per workload, so summaries of several workloads coexist
    tpath = os.path.join(a.profile_out, "traffic.json")
    allt = {}
    if os.path.exists(tpath):
        with open(tpath) as f:
            allt = json.load(f)
        if "workload" in allt:  # older single-workload layout
            allt = {}
    allt[tag] = table
    with open(tpath, "w") as f:
        json.dump(allt, f, indent=1)
    with open(os.path.join(a.profile_out, f"{tag}_traffic.txt"), "w") as f:
        f.write(f"HBM-side traffic per launch from rocprofv3 counters, workload {cfg}/{lin.name} "
                f"({M} x {K} -> {N}, W{bw}A{ba}).\nCommands (repository root on the GPU host):\n"
                f"{a.profile_command}\n\n")
        f.write(f"reference: the calibration copy of 1 GiB: FETCH_SIZE {f_ref:.0f} KiB -> scale "
                f"{f_scale:.4f}; WRITE_SIZE {w_ref:.0f} KiB -> scale {w_scale:.4f}\n\n")
        for key in ("linear", "rotate_quantize"):
            e = table[key]
            f.write(f"{e['kernel']}: fetch {e['fetch_bytes'] / 1e6:.1f} MB (algorithmic reads "
                    f"{e['algorithmic_read_bytes'] / 1e6:.1f} MB); write "
                    f"{e['write_bytes'] / 1e6:.1f} MB (algorithmic writes "
                    f"{e['algorithmic_write_bytes'] / 1e6:.1f} MB)\n")
    if a.profile_counters:
        write_counter_summary(a, tag, lin_parts, rot_name, M, N, K, ba, bw, in_b, n_prep)
    print(json.dumps(table))
    return 0


def write_counter_summary(a, tag, lin_parts, rot_name, M, N, K, ba, bw, in_b, n_prep):
    """Per-kernel averages of SQ/GRBM counters from rocprofv3 --pmc runs,
    with the derived rates the kernels are tuned by."""
    import csv
    import glob
    per = {}
    for d in a.profile_counters:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows = [r for r in csv.DictReader(open(f))
                    if _short_kernel_name(r["Kernel_Name"]) in (*lin_parts, rot_name)]
            rot = [r for r in rows if _short_kernel_name(r["Kernel_Name"]) == rot_name]
            # activation launches of the rotate kernel only (weight prep apart)
            keep = {id(r) for r in _split_rotate(rot, n_prep)[1]}
            for r in rows:
                k = _short_kernel_name(r["Kernel_Name"])
                if k == rot_name and id(r) not in keep:
                    continue
                per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
    lines = [f"SQ/GRBM counters per launch (rocprofv3 --pmc), workload {tag} "
             f"({M} x {K} -> {N}).", "Commands (repository root on the GPU host):",
             a.profile_command, ""]
    n_mfma = 2.0 * M * N * K / 16384  # 16x16x32 f16 MFMAs of the linear
    mfma_call = sum(float(np.mean(per[k]["SQ_INSTS_MFMA"])) for k in lin_parts
                    if "SQ_INSTS_MFMA" in per.get(k, {}))
    for k in (*lin_parts, rot_name):
        c = {n: float(np.mean(v)) for n, v in per.get(k, {}).items()}
        if not c:
            continue
        lines.append(k)
        for n in sorted(c):
            lines.append(f"  {n:30s} {c[n]:.6g}")
        gui = c.get("GRBM_GUI_ACTIVE")
        if k in lin_parts and k.startswith("linear_kernel"):
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c and gui:
                lines.append(f"  MFMA busy per SIMD (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / "
                             f"(GRBM_GUI_ACTIVE / 8 XCDs)): "
                             f"{c['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / (gui / 8):.3f}")
            if "SQ_INSTS_MFMA" in c:
                lines.append(f"  MFMA instructions: {c['SQ_INSTS_MFMA']:.4g}; all kernels of "
                             f"the call: {mfma_call:.4g} (2MNK/16384 = {n_mfma:.4g})")
            if "SQ_INSTS_VALU" in c and "SQ_INSTS_MFMA" in c:
                lines.append(f"  non-MFMA VALU instructions per MFMA: "
                             f"{(c['SQ_INSTS_VALU'] - c['SQ_INSTS_MFMA']) / c['SQ_INSTS_MFMA']:.2f}")
        elif k == rot_name:
            elems = float(M) * K  # activation launches
            for n in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT",
                      "SQ_LDS_IDX_ACTIVE"):
                if n in c:
                    lines.append(f"  {n} per coordinate: {c[n] / elems * 64:.3f}"
                                 + (" (wave instructions x 64 lanes)" if "INSTS" in n
                                    else " (cycles per 64 coordinates)"))
            if "SQ_ACTIVE_INST_VALU" in c and gui:
                lines.append(f"  VALU busy per SIMD: "
                             f"{c['SQ_ACTIVE_INST_VALU'] * 4 / 1024 / (gui / 8):.3f}")
        lines.append("")
    with open(os.path.join(a.profile_out, f"{tag}_counters.txt"), "w") as f:
        f.write("\n".join(lines))


def _median_ms(fn, n_sets, iters, settle_ms=SETTLE_MS):
    """Median of per-call HIP event times (current stream), cycling buffer
    sets, after two untimed rounds and untimed calls for about settle_ms."""
    import torch
    for i in range(2 * n_sets):
        fn(i % n_sets)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < settle_ms and i < 5000:
        fn(i % n_sets)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for i, (e0, e1) in enumerate(ev):
        e0.record()
        fn(i % n_sets)
        e1.record()
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))


def sweep(q, iters=20):
    """Every workload instance at full size: rotate+quantize of its
    activations (synthetic bf16 tokens; enough buffer sets to exceed twice
    the 256 MB Infinity Cache) and the linear for each of its bit pairs on
    the codes the library itself makes from synthetic tokens and weights
    (so the codes follow the Lloyd-Max cell frequencies, as in use), against
    the HBM and fp16 MFMA peaks."""
    import torch
    import workloads as wl
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    for cfg, c in wl.CONFIGS.items():
        if cfg == "tiny":
            continue
        for lin in c["linears"]:
            M, N, K = lin.act.M, lin.weight.N, lin.act.d
            e_in = 2 if lin.act.dtype == wl.BF16 else 4
            dt = torch.bfloat16 if e_in == 2 else torch.float32
            sets = max(1, min(4, -(-(512 << 20) // (M * K * e_in))))
            xs = [torch.randn((M, K), generator=g, device="cuda").to(dt) for _ in range(sets)]
            W = (0.02 * torch.randn((N, K), generator=g, device="cuda")).to(dt)
            rec = {"instance": f"{cfg}/{lin.name}", "M": M, "N": N, "K": K, "rotate_quantize": [],
                   "linear": []}
            acodes = {}
            for ba in sorted({b for _, b in lin.bit_pairs}):
                codes = [torch.empty((M, K * ba // 8), dtype=torch.uint8, device="cuda")
                         for _ in range(sets)]
                norms = [torch.empty((M,), dtype=torch.float32, device="cuda") for _ in range(sets)]
                ms = _median_ms(lambda i: q.rotate_quantize(xs[i], lin.seed, ba, out=codes[i],
                                                            norms=norms[i]), sets, iters)
                gbs = M * (K * e_in + K * ba / 8 + 4) / (ms * 1e-3) / 1e9
                rec["rotate_quantize"].append({"a_bits": ba, "us": round(ms * 1e3, 1),
                                               "GB/s": round(gbs, 1),
                                               "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
                acodes[ba] = (codes[0], norms[0])
                del codes[1:], norms[1:]
            del xs
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            for bw, ba in lin.bit_pairs:
                wc, wn = q.prepare_weights(W, lin.seed, bw)
                ac, an = acodes[ba]
                ms = _median_ms(lambda i: q.linear(ac, an, ba, wc, wn, bw, K, out=y), 1, iters)
                tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
                rec["linear"].append({"w_bits": bw, "a_bits": ba, "ms": round(ms, 4),
                                      "TFLOP/s": round(tf, 1),
                                      "frac_of_mfma_fp16_peak": round(tf / MFMA_FP16_PEAK_TFLOPS,
                                                                      4)})
                del wc, wn
            del y, W, acodes
            torch.cuda.empty_cache()
            print(json.dumps(rec), flush=True)
    return 0


class KernelEvent:
    """A HIP timing event recorded without the system-scope fence
    (hipEventDisableSystemFence), for the per-kernel events inside the timed
    steps: a default event makes the queue write back and invalidate the
    caches when it is recorded, which after the linear's 1 GB of output put
    about 10 us between it and the next launch (the untimed steps run back
    to back with no gap).  Made through the HIP runtime the process already
    uses (the libamdhip64 torch mapped, found in /proc/self/maps); read only
    after a device synchronisation."""
    FLAGS = 0x20000000  # hipEventDisableSystemFence
    _hip = None

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes
            # the copy already mapped into this process (torch's), so the
            # events belong to the runtime that owns the streams
            path = "libamdhip64.so.7"
            try:
                with open("/proc/self/maps") as f:
                    for line in f:
                        if "libamdhip64.so" in line:
                            path = line.split()[-1]
                            break
            except OSError:
                pass
            lib = ctypes.CDLL(path)
            P = ctypes.c_void_p
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [P, P]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
            lib.hipEventDestroy.argtypes = [P]
            cls._hip = lib
        return cls._hip

    def __init__(self):
        import ctypes
        self.h = ctypes.c_void_p()
        if self.hip().hipEventCreateWithFlags(ctypes.byref(self.h), self.FLAGS) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        import ctypes
        if self.hip().hipEventRecord(self.h, ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        if self.hip().hipEventElapsedTime(ctypes.byref(ms), self.h, end.h) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        if self._hip is not None and self.h:
            self._hip.hipEventDestroy(self.h)


PREP_TIMED = 5  # timed weight-preparation launches after the first one
LEAD_CYCLES = 500_000  # untimed spin before the timed region (about 200 us)
BACK_TO_BACK = 20  # rotate+quantize launches timed alone after the steps


def online_step(q, lin, cfg, bw, ba, steps, warmup, sets, calib_copy_mib=0, settle_ms=0.0):
    """Times the online step of one linear: weight codes prepared once
    (offline; 1 + PREP_TIMED launches, the first untimed, before anything
    else touches the rotate kernel), then untimed settle steps for about
    `settle_ms` of wall time, `warmup` untimed and
    `steps` timed steps of rotate + quantize (activation set i mod sets)
    followed by the linear, with one fence-free HIP event on the launch
    stream between consecutive kernels and the whole timed region bracketed
    by device synchronisations."""
    import torch
    import workloads as wl
    M, N, K = lin.act.M, lin.weight.N, lin.act.d
    x_np = wl.activations(cfg, lin.name)
    xs = [to_dev(x_np)]
    del x_np
    for i in range(1, sets):
        # distinct buffers with the same distribution: circular row shifts
        xs.append(torch.roll(xs[0], shifts=97 * i, dims=0).contiguous())
    W = to_dev(wl.weights(cfg, lin.name))
    dev = xs[0].device
    stream = torch.cuda.current_stream()
    wc = torch.empty((N, K * bw // 8), dtype=torch.uint8, device=dev)
    wn = torch.empty((N,), dtype=torch.float32, device=dev)
    ac = [torch.empty((M, K * ba // 8), dtype=torch.uint8, device=dev) for _ in range(sets)]
    an = [torch.empty((M,), dtype=torch.float32, device=dev) for _ in range(sets)]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    if calib_copy_mib > 0:  # known-size reference for the HBM byte counters
        n = calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # offline weight preparation
    q.prepare_weights(W, lin.seed, bw, out=wc, norms=wn)
    torch.cuda.synchronize()
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(PREP_TIMED)]
    for e0, e1 in pev:
        e0.record(stream)
        q.prepare_weights(W, lin.seed, bw, out=wc, norms=wn)
        e1.record(stream)
    torch.cuda.synchronize()
    t_prep = float(np.median([e0.elapsed_time(e1) for e0, e1 in pev]))

    def step(i, mid=None, end=None):
        s = i % sets
        q.rotate_quantize(xs[s], lin.seed, ba, out=ac[s], norms=an[s])
        if mid is not None:
            mid.record(stream)
        q.linear(ac[s], an[s], ba, wc, wn, bw, K, out=y)
        if end is not None:
            end.record(stream)

    # every event of the timed region is made here, before the settle steps:
    # making them takes tens of milliseconds, and an idle device that long
    # starts the clock transient over.  One event between consecutive
    # kernels (each recorded event costs the queue a few microseconds):
    # mark 2i opens step i's rotate+quantize, 2i+1 separates it from the
    # linear, 2i+2 closes the step and opens the next
    marks = [KernelEvent() for _ in range(2 * steps + 1)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for e in (start, stop, s0, s1):  # torch makes its events at the first record
        e.record(stream)
    torch.cuda.synchronize()
    n_settle, settle_total = 0, 0.0
    if settle_ms > 0:
        s0.record(stream)
        t0 = time.perf_counter()
        while n_settle < 4000:
            step(n_settle)
            n_settle += 1
            if n_settle % 4 == 0:  # a short wait, the next launches follow at once
                torch.cuda.synchronize()
                if (time.perf_counter() - t0) * 1e3 >= settle_ms:
                    break
        s1.record(stream)
        torch.cuda.synchronize()
        settle_total = s0.elapsed_time(s1)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # untimed: a short spin kernel keeps the device busy while the host
    # queues the first steps, so the timed region starts with launches
    # already queued instead of the host's latency for the first one
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(LEAD_CYCLES)
    start.record(stream)
    marks[0].record(stream)
    for i in range(steps):
        step(i, marks[2 * i + 1], marks[2 * i + 2])
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    # after the timed region, not part of the step: the rotate+quantize
    # launch alone, BACK_TO_BACK times back to back (one event pair), so its
    # rate without a linear's output write-back beside it is on record too
    for i in range(2):
        q.rotate_quantize(xs[i % sets], lin.seed, ba, out=ac[i % sets], norms=an[i % sets])
    torch.cuda.synchronize()
    b0 = torch.cuda.Event(enable_timing=True)
    b1 = torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for i in range(BACK_TO_BACK):
        q.rotate_quantize(xs[i % sets], lin.seed, ba, out=ac[i % sets], norms=an[i % sets])
    b1.record(stream)
    torch.cuda.synchronize()
    r = {
        "t_rot_b2b": b0.elapsed_time(b1) / BACK_TO_BACK,
        "ms_step": total_ms / steps,
        "t_rot": float(np.mean([marks[2 * i].elapsed_time(marks[2 * i + 1])
                                for i in range(steps)])),
        "t_lin": float(np.mean([marks[2 * i + 1].elapsed_time(marks[2 * i + 2])
                                for i in range(steps)])),
        "per_step": np.array([marks[2 * i].elapsed_time(marks[2 * i + 2]) for i in range(steps)]),
        "lin_steps": np.array([marks[2 * i + 1].elapsed_time(marks[2 * i + 2])
                               for i in range(steps)]),
        "rot_steps": np.array([marks[2 * i].elapsed_time(marks[2 * i + 1]) for i in range(steps)]),
        "t_prep": t_prep,
        "prep_launches": 1 + PREP_TIMED,
        "settle_steps": n_settle,
        "settle_ms": settle_total,
    }
    r["x0"], r["W"] = xs[0], W
    del xs[1:], ac, an, y, wc, wn
    return r


def b2b_entry(r, rt):
    """The rotate+quantize launch timed alone (after the steps, not in them)."""
    return {"what": f"the same launch {BACK_TO_BACK} times back to back after the timed "
                    "steps (one event pair): no linear's output write-back beside it",
            "ms": round(r["t_rot_b2b"], 4), "GB/s": round(rt["rot_b2b_gbs"], 1),
            "frac_of_hbm_peak": round(rt["rot_b2b_gbs"] / HBM_PEAK_GBS, 4)}


def step_rates(lin, bw, ba, r):
    import workloads as wl
    M, N, K = lin.act.M, lin.weight.N, lin.act.d
    in_b = 2 if lin.act.dtype == wl.BF16 else 4
    flops = 2.0 * M * N * K
    rot_bytes = M * (K * in_b + K * ba / 8 + 4)
    prep_bytes = N * (K * (2 if lin.weight.dtype == wl.BF16 else 4) + K * bw / 8 + 4)
    return {"lin_tflops": flops / (r["t_lin"] * 1e-3) / 1e12,
            "rot_gbs": rot_bytes / (r["t_rot"] * 1e-3) / 1e9,
            "rot_b2b_gbs": rot_bytes / (r["t_rot_b2b"] * 1e-3) / 1e9,
            "prep_gbs": prep_bytes / (r["t_prep"] * 1e-3) / 1e9,
            "value": flops / (r["ms_step"] * 1e-3) / 1e12}


def main():
    a = parse()
    if a.summarize_profiles:
        return summarize_profiles(a)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}): the library has no "
              "multi-GPU path; its kernels run one GPU's share of the work", flush=True)
        return 2
    if a.sweep:
        import torch
        import quantization_dit_linear_amd as q
        torch.cuda.set_device(0)
        return sweep(q)
    import torch
    import quantization_dit_linear_amd as q
    import workloads as wl

    cfg = a.workload
    lin = wl.CONFIGS[cfg]["linears"][0] if a.linear is None else wl.get_linear(cfg, a.linear)
    bw, ba = lin.bit_pairs[0] if a.bits is None else tuple(int(v) for v in a.bits.split(","))
    M, N, K = lin.act.M, lin.weight.N, lin.act.d
    tag = f"{cfg}_w{bw}a{ba}"
    torch.cuda.set_device(0)

    r = online_step(q, lin, cfg, bw, ba, a.steps, a.warmup, a.sets, a.calib_copy_mib,
                    a.settle_ms)
    rt = step_rates(lin, bw, ba, r)
    x0, W0 = r.pop("x0"), r.pop("W")
    ref_gemm = None if a.no_ref_gemm else library_fp16_gemm(M, N, K)
    fq_path = None if a.no_ref_gemm else fake_quant_path(q, x0, W0, lin.seed, ba, bw)
    w8 = None if a.no_ref_gemm else w8a8_path(q, x0, W0, lin.seed)
    adaln = None if a.no_ref_gemm else adaln_rtn4(q, "image" if K == 3072 else "video")
    ceil = None if a.no_ref_gemm else measured_ceilings(q)
    del x0, W0
    torch.cuda.empty_cache()
    second = None
    if not a.no_second_shape and cfg != "image_qkv":
        l2 = wl.CONFIGS["image_qkv"]["linears"][0]
        r2 = online_step(q, l2, "image_qkv", 4, 4, max(a.steps, 20), max(a.warmup, 3), 4,
                         settle_ms=a.settle_ms)
        r2.pop("x0"), r2.pop("W")
        rt2 = step_rates(l2, 4, 4, r2)
        second = {
            "workload": f"image_qkv/qkv: {l2.act.M} tokens, d_in {l2.act.d} -> d_out "
                        f"{l2.weight.N}, W4A4, activations bf16 (4 activation sets)",
            "ms_per_step": round(r2["ms_step"], 4), "value": round(rt2["value"], 3),
            "linear": {"ms": round(r2["t_lin"], 4), "TFLOP/s": round(rt2["lin_tflops"], 2),
                       "frac_of_mfma_fp16_peak": round(rt2["lin_tflops"] / MFMA_FP16_PEAK_TFLOPS,
                                                       4)},
            "rotate_quantize": {"ms": round(r2["t_rot"], 4), "GB/s": round(rt2["rot_gbs"], 1),
                                "frac_of_hbm_peak": round(rt2["rot_gbs"] / HBM_PEAK_GBS, 4),
                                "back_to_back": b2b_entry(r2, rt2)},
            "prepare_weights": {"ms": round(r2["t_prep"], 4), "GB/s": round(rt2["prep_gbs"], 1)},
        }
        torch.cuda.empty_cache()

    lin_digest = src_digest(*LIN_SRC)
    rot_digest = src_digest(*ROT_SRC)
    lin_tflops, rot_gbs, prep_gbs = rt["lin_tflops"], rt["rot_gbs"], rt["prep_gbs"]
    out = {
        "metric": "rotate+quant GB/s and W4A4 linear TFLOP/s, as % of HBM / MFMA peak",
        "value": round(rt["value"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "settle": {"what": "untimed steps before the warm-up steps, so the clocks settle at "
                           "their loaded state",
                   "steps": r["settle_steps"], "ms": round(r["settle_ms"], 1)},
        "ms_per_step": round(r["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "dtype_detail": "linear: fp16 MFMA operands (unit-variance levels), fp32 accumulate, "
                        "bf16 output; rotate+quantize: fp32",
        "data": "synthetic",
        "config": {"workload": f"{cfg}/{lin.name}: {M} tokens, d_in {K} -> d_out {N}, "
                               f"W{bw}A{ba}, activations "
                               f"{'bf16' if lin.act.dtype == wl.BF16 else 'fp32'}; step = "
                               f"rotate+quantize + linear, weights prepared offline",
                   "M": M, "N": N, "K": K, "w_bits": bw, "a_bits": ba},
        "step_ms_median": round(float(np.median(r["per_step"])), 4),
        "step_ms_iqr": [round(float(np.percentile(r["per_step"], 25)), 4),
                        round(float(np.percentile(r["per_step"], 75)), 4)],
        "kernels": {
            "linear": {"ms": round(r["t_lin"], 4), "TFLOP/s": round(lin_tflops, 2),
                       "ms_median": round(float(np.median(r["lin_steps"])), 4),
                       "frac_of_mfma_fp16_peak": round(lin_tflops / MFMA_FP16_PEAK_TFLOPS, 4)},
            "rotate_quantize": {"ms": round(r["t_rot"], 4), "GB/s": round(rot_gbs, 1),
                                "ms_median": round(float(np.median(r["rot_steps"])), 4),
                                "frac_of_hbm_peak": round(rot_gbs / HBM_PEAK_GBS, 4),
                                "back_to_back": b2b_entry(r, rt)},
        },
        "prepare_weights": {"what": "offline, once per layer: not in the step; median of "
                                    f"{PREP_TIMED} launches",
                            "ms": round(r["t_prep"], 4), "GB/s": round(prep_gbs, 1),
                            "frac_of_hbm_peak": round(prep_gbs / HBM_PEAK_GBS, 4),
                            "launches": r["prep_launches"],
                            "step_ms_with_it": round(r["ms_step"] + r["t_prep"], 4)},
        "roofline": {"bound": "mfma", "achieved": round(lin_tflops, 2),
                     "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(lin_tflops / MFMA_FP16_PEAK_TFLOPS, 4),
                     "traffic": stored_traffic(tag, "linear", lin_digest)},
        "roofline_rotate_quantize": {"bound": "hbm", "achieved": round(rot_gbs, 1),
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(rot_gbs / HBM_PEAK_GBS, 4),
                                     "traffic": stored_traffic(tag, "rotate_quantize",
                                                               rot_digest)},
    }
    if second is not None:
        out["image_qkv"] = second
    if ref_gemm is not None:
        out["reference_fp16_gemm"] = dict(ref_gemm, linear_over_reference=round(
            ref_gemm["ms"] / r["t_lin"], 3))
    if adaln is not None:
        out["adaln_rtn4"] = adaln
    if ceil is not None:
        out["measured_ceilings"] = dict(
            ceil, linear_frac_of_probe=round(lin_tflops / ceil["mfma_f16_probe_TFLOP/s"], 4),
            rotate_frac_of_copy=round(rot_gbs / ceil["copy_1GiB_GB/s"], 4))
    if w8 is not None:
        out["w8a8"] = w8
    if fq_path is not None:
        out["fake_quant_path"] = dict(fq_path, native_step_speedup=round(
            fq_path["ms"] / r["ms_step"], 3))
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, lin, bw, ba, a.cpu_rows)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
