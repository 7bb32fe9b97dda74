"""bench.py's command line and its one-line JSON report.

The CPU test checks that a request for more than one GPU is refused before
anything touches a device; the GPU test runs a short benchmark in a child
process and checks every key of the line it prints."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
METRIC = "dispatch+combine GB/s (% of HBM peak) and mb_plan µs per MoE layer call"


def _bench(*args, timeout=240):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2", timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.gpu
def test_report_line_keys():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    r = _bench("--workload", "mixtral", "--steps", "3", "--warmup", "1")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    assert d["metric"] == METRIC and d["unit"] == "GB/s"
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["vs_baseline"] is None and d["data"] == "synthetic"
    assert d["dtype"] == "bf16" and d["config"]["workload"] == "mixtral"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # value: the step's algorithmic bytes over the step time
    nbytes = sum(d["algorithmic_bytes"].values())
    assert d["value"] == pytest.approx(nbytes / (d["ms_per_step"] * 1e6), rel=2e-3)
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-3)
    assert "traffic" in rf
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s"
    assert cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert d["plan_us"]["p50"] > 0
    assert d["graph_replay"] is None


@pytest.mark.gpu
def test_graph_replay_report():
    """--graph adds the steps replayed from HIP graphs beside the eager ones."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    r = _bench("--workload", "mixtral", "--steps", "3", "--warmup", "1", "--graph",
               "--skip-cpu-baseline")
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    g = d["graph_replay"]
    assert g["graphs"] >= 1 and g["ms_per_step"] > 0 and g["value"] > 0
    assert d["cpu_baseline"] is None


@pytest.mark.gpu
def test_fp8_and_drift_reports():
    """The fp8 decode workload with the dequantising combine, and the
    drift-gated sequence with its replan report."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    r = _bench("--workload", "decode_drift", "--combine-fp8", "--steps", "4", "--warmup", "1",
               "--skip-cpu-baseline")
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["dtype"] == "fp8" and d["config"]["workload"] == "decode_drift"
    assert d["config"]["expert_outputs"] == "fp8+scales"
    assert 0 < d["plan_us"]["p50"] <= d["plan_us"]["p99"]
    assert d["roofline"]["frac"] == pytest.approx(d["roofline"]["achieved"] / 8000.0, rel=1e-3)
    r = _bench("--workload", "drift_decode", "--warmup", "1", "--skip-cpu-baseline")
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    g = d["drift_gate"]
    assert d["steps"] == d["config"]["calls"] == g["calls"]
    s = g["settings"]
    gate = s["gate"]
    assert gate["replanned_calls"][0] == 0 and gate["same_every_rep"]
    assert 0 < gate["plan_us"]["kept_mean"] and 0 < gate["plan_us"]["replanned_mean"]
    assert gate["header"]["replans"] == gate["replans"] == len(gate["replanned_calls"])
    assert gate["header"]["guarded"] == gate["guard_replans"]
    assert len(gate["changes_per_call"]) == g["calls"]
    assert s["every_call"]["replans"] == g["calls"] and s["every_call"]["params"] is None
    for row in s.values():
        assert row["fatal_calls"] == 0
    assert g["replica_weight_bytes_avoided_by_gate"] == (
        s["every_call"]["replica_changes"] - gate["replica_changes"]) * g["weight_bytes_per_replica"]


@pytest.mark.gpu
def test_ceiling_report():
    """bench.py --ceiling: k_dispatch beside its reference kernels, each
    timed; the write-only scatter writes what its header says where pos says."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    r = _bench("--workload", "mixtral", "--ceiling", "--reps", "3")
    assert r.returncode == 0, r.stderr[-2000:]
    c = json.loads(r.stdout.strip().splitlines()[-1])["ceiling"]
    assert set(c["kernels"]) == {"k_dispatch", "k_scatter_write", "k_row_write", "k_fill",
                                 "k_read", "k_copy", "k_combine", "k_gather_xor"}
    for k in c["kernels"].values():
        assert k["us"] > 0 and 0 < k["frac_of_peak"] < 1.2
    import ctypes

    import bench

    L = bench._ceiling_lib()
    dev = torch.device("cuda:0")
    N, K, rows, rb = 300, 4, 1500, 2064  # rows of 129 lanes: a ragged second span
    pos = torch.randperm(rows, device=dev)[: N * K].to(torch.int32)
    pos[5] = -1  # skipped
    pos[7] = rows  # skipped
    for fn in (L.mbc_scatter_write, L.mbc_row_write):
        buf = torch.full((rows, rb // 4), -1, dtype=torch.int32, device=dev)
        rc = fn(ctypes.c_void_p(pos.data_ptr()), ctypes.c_void_p(buf.data_ptr()), N, K, rb, rows,
                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == 0
        torch.cuda.synchronize()
        b = buf.view(rows, rb // 16, 4).cpu()
        p = pos.cpu()
        hit = torch.zeros(rows, dtype=torch.bool)
        for j in range(N * K):
            r = int(p[j])
            if 0 <= r < rows:
                hit[r] = True
                assert bool((b[r, :, 0] == j // K).all())
                assert bool((b[r, :, 1] == torch.arange(rb // 16)).all())
        assert bool((b[~hit] == -1).all())
    # the gather: y row t = XOR of the rows pos[t][k] (skipped entries add nothing)
    ye = torch.randint(-2 ** 31, 2 ** 31 - 1, (rows, rb // 4), dtype=torch.int32, device=dev)
    y = torch.full((N, rb // 4), 7, dtype=torch.int32, device=dev)
    rc = L.mbc_gather_xor(ctypes.c_void_p(pos.data_ptr()), ctypes.c_void_p(ye.data_ptr()),
                          ctypes.c_void_p(y.data_ptr()), N, K, rb, rows,
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    p = pos.view(N, K).long()
    ok = (p >= 0) & (p < rows)
    g = ye[p.clamp(0, rows - 1)] * ok.unsqueeze(-1)
    exp = g[:, 0]
    for k in range(1, K):
        exp = exp ^ g[:, k]
    assert torch.equal(y, exp)
