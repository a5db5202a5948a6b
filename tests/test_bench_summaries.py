"""Host logic of bench.py's profile summaries: a linear call made of several
kernels (the full rounds, the K-split leftover pieces and their reduction)
is timed and counted as the sum of its kernels, the HBM counters are
scaled by the calibration copy, and traffic.json keeps one entry per
workload.  Fabricated rocprofv3 CSV files stand in for a GPU run."""
import csv
import json
import os
import sys

import pytest

import bench

LIN_BIG = ("void oq::(anonymous namespace)::linear_kernel<oq::(anonymous namespace)::"
           "Tile<256, 2, 4, 32, 1>, 4, 4>(unsigned char const*, float const*)")
LIN_SMALL = ("void oq::(anonymous namespace)::linear_kernel<oq::(anonymous namespace)::"
             "Tile<128, 2, 2, 16, 2>, 4, 4>(unsigned char const*, float const*)")
REDUCE = "oq::(anonymous namespace)::tail_reduce_kernel(float const*, int, int)"
ROT = "void oq::(anonymous namespace)::rq_fast_kernel<3072, 4, false, false>(unsigned short const*)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def _counters(path, name, per_kernel):
    """One row per dispatch; dispatch ids follow the listing order."""
    rows = []
    did = 0
    for kernel, values in per_kernel.items():
        for v in values:
            did += 1
            rows.append([did, kernel, name, float(v), 1024])
    _write(path, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Grid_Size"],
           rows)


@pytest.fixture
def runs(tmp_path):
    kt = tmp_path / "kt"
    _write(str(kt / "kt_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
            "StdDev"],
           [[LIN_BIG, 12, 6.0e6, 500000.0, 80.0, 480000.0, 520000.0, 1.0],
            [ROT, 24, 648000.0, 27000.0, 8.0, 22000.0, 30000.0, 1.0],
            [LIN_SMALL, 12, 240000.0, 20000.0, 3.0, 19000.0, 21000.0, 1.0],
            [REDUCE, 12, 96000.0, 8000.0, 1.0, 7000.0, 9000.0, 1.0],
            [COPY, 9, 30000.0, 3333.0, 0.4, 2000.0, 5000.0, 1.0]])
    # per-dispatch trace of the rotate kernel: one weight-preparation launch
    # (30 us) first, then activation launches of 25 and 27 us
    _write(str(kt / "kt_kernel_trace.csv"),
           ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [[5, ROT, 1000, 31000], [9, ROT, 50000, 75000], [12, ROT, 90000, 117000],
            [7, LIN_BIG, 40000, 45000]])
    # KiB per dispatch; the 1 GiB calibration copy reads 524288 and writes
    # 1048576, so the scales are 2.0 and 1.0
    _counters(str(tmp_path / "f" / "f_counter_collection.csv"), "FETCH_SIZE",
              {COPY: [1.0, 524288.0], LIN_BIG: [100000.0, 100000.0], LIN_SMALL: [8000.0],
               REDUCE: [16000.0], ROT: [27000.0, 29000.0, 30000.0]})
    _counters(str(tmp_path / "w" / "w_counter_collection.csv"), "WRITE_SIZE",
              {COPY: [1.0, 1048576.0], LIN_BIG: [170000.0], LIN_SMALL: [16000.0],
               REDUCE: [2000.0], ROT: [9000.0, 7000.0]})
    _counters(str(tmp_path / "s" / "s_counter_collection.csv"), "SQ_INSTS_MFMA",
              {LIN_BIG: [3.0e7], LIN_SMALL: [1.5e6], REDUCE: [0.0]})
    out = tmp_path / "out"
    out.mkdir()
    # a summary of another workload must survive
    with open(out / "traffic.json", "w") as f:
        json.dump({"other_w4a4": {"linear": {"bytes_per_launch": 7}}}, f)
    return tmp_path


def _summarize(tmp_path, monkeypatch):
    argv = ["bench.py", "--workload", "image_qkv", "--prep-launches", "1",
            "--summarize-profiles", str(tmp_path / "kt"), str(tmp_path / "f"),
            str(tmp_path / "w"), "--profile-counters", str(tmp_path / "s"),
            "--profile-out", str(tmp_path / "out"), "--profile-command", "cmd"]
    monkeypatch.setattr(sys, "argv", argv)
    assert bench.summarize_profiles(bench.parse()) == 0


def test_linear_call_is_the_sum_of_its_kernels(runs, monkeypatch):
    _summarize(runs, monkeypatch)
    txt = (runs / "out" / "image_qkv_w4a4_kernel_stats.txt").read_text()
    assert ("linear call = linear_kernel<Tile<256, 2, 4, 32, 1>, 4, 4> + linear_kernel"
            "<Tile<128, 2, 2, 16, 2>, 4, 4> + tail_reduce_kernel: 528.0 us per call") in txt


def test_traffic_per_call_and_scaling(runs, monkeypatch):
    _summarize(runs, monkeypatch)
    t = json.load(open(runs / "out" / "traffic.json"))
    assert t["other_w4a4"] == {"linear": {"bytes_per_launch": 7}}
    e = t["image_qkv_w4a4"]
    assert e["fetch_scale"] == 2.0 and e["write_scale"] == 1.0
    lin = e["linear"]
    assert lin["fetch_bytes"] == int((100000 + 8000 + 16000) * 1024 * 2.0)
    assert lin["write_bytes"] == int((170000 + 16000 + 2000) * 1024 * 1.0)
    assert lin["bytes_per_launch"] == lin["fetch_bytes"] + lin["write_bytes"]
    assert lin["source_digest"] == bench.src_digest(*bench.LIN_SRC)
    rot = e["rotate_quantize"]
    # the first dispatch prepared the weights: activation launches only
    assert rot["fetch_bytes"] == int(29500 * 1024 * 2.0)
    assert rot["write_bytes"] == int(7000 * 1024 * 1.0)
    assert rot["algorithmic_read_bytes"] == 9216 * 3072 * 2
    # algorithmic bytes of the workload: codes and norms in, bf16 out
    M = N = 9216
    K = 3072
    assert lin["algorithmic_read_bytes"] == M * K // 2 + N * K // 2 + 4 * (M + N)
    assert lin["algorithmic_write_bytes"] == 2 * M * N


def test_rotate_time_excludes_weight_preparation(runs, monkeypatch):
    _summarize(runs, monkeypatch)
    txt = (runs / "out" / "image_qkv_w4a4_kernel_stats.txt").read_text()
    assert "average 26.0 us" in txt and "weight preparation 30.0 us" in txt


def test_mfma_count_sums_the_call(runs, monkeypatch):
    _summarize(runs, monkeypatch)
    txt = (runs / "out" / "image_qkv_w4a4_counters.txt").read_text()
    assert "all kernels of the call: 3.15e+07" in txt


def test_source_digest_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "quantization_dit_linear_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "k.hip").write_text("int f() {\n  return 1;  // one\n}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.src_digest("k.hip")
    (src / "k.hip").write_text("/* header */\nint f() {\n\n  return 1;  // the value one\n}\n")
    assert bench.src_digest("k.hip") == d0
    (src / "k.hip").write_text("int f() {\n  return 2;  // one\n}\n")
    assert bench.src_digest("k.hip") != d0


def test_split_rotate_counts_only_the_steps_launches():
    """Rotate dispatches in launch order: the first n_prep prepared the
    weights, the next n_act belong to the steps, and any later ones (the
    launches timed back to back after the steps) are left out of both."""
    rows = [{"Dispatch_Id": str(i), "v": i} for i in (7, 3, 11, 5, 9, 1, 13, 15, 2)]
    prep, act = bench._split_rotate(rows, 2, 4)
    assert [int(r["Dispatch_Id"]) for r in prep] == [1, 2]
    assert [int(r["Dispatch_Id"]) for r in act] == [3, 5, 7, 9]
    prep, act = bench._split_rotate(rows, 2)
    assert [int(r["Dispatch_Id"]) for r in act] == [3, 5, 7, 9, 11, 13, 15]


def test_step_launches_count_settle_warmup_and_timed_steps():
    """The activation launches the summaries attribute to the steps: every
    step the bench line says it ran, settle steps included."""
    assert bench._step_launches({"steps": 10, "warmup": 2, "settle": {"steps": 45}}) == 57
    assert bench._step_launches({"steps": 10, "warmup": 2}) == 12
    assert bench._step_launches({"metric": "x"}) is None
