"""Benchmark of the hot path: mb_plan + mb_dispatch + mb_combine per step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one MoE layer call of the chosen workload (default: the
DeepSeek-V3-like prefill layer, 32 logical ranks x 4096 tokens, 256 experts,
top-8, 1 replica slot per rank, bf16 rows of 7168): plan, dispatch every token
row to its K rows, combine the K expert-output rows of every token. Inputs are
seeded synthetic routing and rows, resident in HBM before timing starts.
Expert outputs are the dispatched rows (identity experts), written once
before timing into a buffer of their own.

A workload of several calls (the 61 layer calls of decode_drift) steps
through its calls, one per step (by default five passes, after one untimed
pass that settles the runtime's launch queues), so plan p50/p99 cover every
call five times. A workload whose row buffers are
smaller than the last-level cache runs on several buffer sets in turn (at
least 1 GiB in all), so no step reads what a recent step left in cache.

A workload planned with drift-gated replanning (drift_decode) steps through
its sequence of calls, one call per step, from a fresh drift state when the
timed steps begin; the line then also reports, per gate setting (none, the
workload's, a check every call, ViBE's tolerance 0.03, the region-size guard
alone), plan times over five fresh passes, replans, replica weight copies at
W = 3 H I b bytes each, and the rank imbalance.

Prints one JSON line. `value` is dispatch + combine algorithmic bytes per
step divided by the whole step time (plan included), from HIP events around
the timed steps; the steps are queued behind 30 ms of unrelated GPU work
(`backlog_ms`, inside the wall-clock bracket) so that the host's launch rate
does not idle the GPU between short steps. `roofline` refers to the
kernel with the larger share of the step (HIP events on the launch stream);
`cpu_baseline` times the CPU oracle (single thread) on half of the
tokens of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine GB/s (% of HBM peak) and mb_plan µs per MoE layer call"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
# committed counter summaries, one per workload: pmc_k_dispatch_k_combine_<workload>.md
PROFILE_PMC = os.path.join(ROOT, "profiles", "pmc_k_dispatch_k_combine_{}.md")
ROW_KERNEL_SOURCE = os.path.join(ROOT, "token_dispatch_mb_amd", "csrc", "rows.hip")


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(wl, combine_fp8: bool = False) -> dict:
    """Bytes the method itself must move per layer call (no padding, no
    staging): dispatch reads each row once and writes it K times, reading
    pos; combine reads K expert rows, pos and w per token and writes one row
    (with combine_fp8 the expert rows are fp8 plus a 4-byte scale per 128)."""
    N, K, H = wl.n_tokens, wl.top_k, wl.hidden
    b_in = {"f32": 4, "bf16": 2, "fp8": 1}[wl.dtype_in]
    b_out = {"f32": 4, "bf16": 2}[wl.dtype_out]
    row_in = H * b_in + (H // 128 * 4 if wl.dtype_in == "fp8" else 0)
    row_out = H * b_out
    row_exp = H + H // 128 * 4 if combine_fp8 else row_out
    dispatch = N * row_in + N * K * row_in + N * K * 4
    combine = N * K * row_exp + N * K * 8 + N * row_out
    return {"dispatch": dispatch, "combine": combine, "row_in": row_in, "row_out": row_out}


def source_hash() -> str:
    return hashlib.sha256(open(ROW_KERNEL_SOURCE, "rb").read()).hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the workload's committed
    rocprofv3 counter summary, or None if absent or taken on different kernel
    source."""
    path = PROFILE_PMC.format(workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^source_sha256_16:\s*(\w+)", text, re.M)
    if not m or m.group(1) != source_hash():
        return None
    m = re.search(r"^workload:\s*(\S+)", text, re.M)
    if not m or m.group(1) != workload:
        return None
    m = re.search(rf"^traffic_bytes_per_launch\.{kernel}:\s*([0-9.eE+]+)", text, re.M)
    return float(m.group(1)) if m else None


# Intermediate width I of one expert for the replica weight bytes W = 3 H I b
# (ISER-MoE, Key Formula: gate, up and down projections), the MoonEP
# benchmark's H' = 2048; b = 1 byte (fp8 weights, as the rows).
WEIGHT_I = 2048
WEIGHT_B = 1


_BACKLOG = {}  # the backlog's scratch buffer and its measured fill time


def _backlog(torch, dev, ms: float) -> None:
    """Queue about `ms` of GPU work (fills of a 2 GiB buffer, their rate
    measured once) on the current stream, so that the host can queue the
    work after it before the GPU reaches it: event pairs around that work
    then time the GPU alone, not the host's launch rate."""
    if "buf" not in _BACKLOG:
        _BACKLOG["buf"] = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        _BACKLOG["buf"].fill_(0)
        a.record()
        for _ in range(4):
            _BACKLOG["buf"].fill_(0)
        b.record()
        torch.cuda.synchronize()
        _BACKLOG["fill_ms"] = a.elapsed_time(b) / 4
    for _ in range(max(1, int(ms / _BACKLOG["fill_ms"]) + 1)):
        _BACKLOG["buf"].fill_(0)


def _time_plans(dims, ids_all, ws, bufs, speeds, repair, drift, reps, mb, torch, np):
    """The calls of ids_all planned `reps` times in turn (a drift state, if
    any, zero-filled before each pass), one HIP event pair around each plan,
    run twice: once to time the host's queueing, then behind a backlog of GPU
    work longer than that, so the plans run back to back on the GPU. Returns
    the µs of each plan [reps * calls] and each plan's replica slots and
    status word [reps, calls, ...]."""
    dev = bufs.status.device
    T, PR = ids_all.shape[0], bufs.rep_expert.numel()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps * T)]
    rep_d = torch.empty((reps * T, PR), dtype=torch.int32, device=dev)
    st_d = torch.empty((reps * T, 4), dtype=torch.int32, device=dev)

    def run():
        for r in range(reps):
            if drift is not None:
                drift[1].zero_()
            for c in range(T):
                i = r * T + c
                ev[i][0].record()
                mb.plan(dims, ids_all[c], ws, bufs, speeds=speeds, drift=drift, repair=repair)
                ev[i][1].record()
                rep_d[i].copy_(bufs.rep_expert.view(-1))
                st_d[i].copy_(bufs.status)

    torch.cuda.synchronize()
    h0 = time.perf_counter()
    run()
    host_ms = (time.perf_counter() - h0) * 1e3
    torch.cuda.synchronize()
    _backlog(torch, dev, 2 * host_ms + 5)
    run()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
    return us, rep_d.cpu().numpy().reshape(reps, T, PR), st_d.cpu().numpy().reshape(reps, T, 4)


def _drift_report(wl, dims, ids_all, ws, bufs, speeds, repair, mb, torch, np, reps=5):
    """Untimed against the step, timed per plan: the sequence of calls planned
    from a fresh state `reps` times under each gate setting (and with no
    gate: the greedy every call), one HIP event pair around each plan, the
    plans queued back to back. Per setting: plan µs (mean, p50, p99, and the
    replanned and kept calls' means), replans and guard replans per
    sequence, replica slots whose expert changed from the previous call
    (each a weight copy of W bytes) and calls that kept every slot, the rank
    imbalance max load / mean load after each call, and fatal calls (plans
    timed by _time_plans)."""
    dev = bufs.status.device
    T = wl.calls
    w_bytes = 3 * wl.hidden * WEIGHT_I * WEIGHT_B
    mean_load = wl.n_tokens * wl.top_k / wl.n_ranks
    g = tuple(wl.drift)
    settings = [("every_call", None), ("gate", g), ("gate_check_every_1", g[:3] + (1,) + g[4:]),
                ("gate_tol_0.03", g[:4] + (3, 100)), ("gate_cap_only", g[:4] + (0, 0))]
    rows = {}
    for name, prm in settings:
        drift = None
        if prm is not None:
            drift = (mb.DriftParams(*prm), mb.alloc_drift_state(dims, dev))
        us, reps_h, st = _time_plans(dims, ids_all, ws, bufs, speeds, repair, drift, reps, mb, torch,
                                     np)
        flags = st[..., 0]
        replanned = np.ones_like(flags, bool) if drift is None else (flags & mb.ST_REPLANNED) != 0
        guarded = (flags & mb.ST_GUARDED) != 0
        # a slot whose expert differs from the previous call's needs that
        # expert's weights copied in (an emptied slot needs nothing)
        changed = ((reps_h[:, 1:] != reps_h[:, :-1]) & (reps_h[:, 1:] >= 0)).sum(axis=2)
        ir = st[..., 2] / mean_load
        rp = replanned.ravel()
        row = {
            "params": None if prm is None else dict(zip(
                ("delta_num", "delta_den", "window", "check_every", "tol_num", "tol_den"), prm)),
            "plan_us": {"mean": round(float(us.mean()), 2), "p50": round(float(np.median(us)), 2),
                        "p99": round(float(np.percentile(us, 99)), 2),
                        "replanned_mean": round(float(us[rp].mean()), 2) if rp.any() else None,
                        "kept_mean": round(float(us[~rp].mean()), 2) if (~rp).any() else None},
            "replans": int(replanned[0].sum()),
            "guard_replans": int(guarded[0].sum()),
            "replanned_calls": [int(c) for c in np.flatnonzero(replanned[0])],
            "replica_changes": int(changed[0].sum()),
            "calls_keeping_every_slot": int((changed[0] == 0).sum()),
            "replica_weight_bytes": int(changed[0].sum()) * w_bytes,
            "ir_after_mean": round(float(ir[0].mean()), 5),
            "ir_after_max": round(float(ir[0].max()), 5),
            "unbalanced_calls": int(((flags[0] & mb.ST_UNBALANCED) != 0).sum()),
            "fatal_calls": int(((flags[0] & mb.ST_FATAL) != 0).sum()),
            "same_every_rep": bool((st == st[:1]).all() and (reps_h == reps_h[:1]).all()),
        }
        if name == "gate":
            row["changes_per_call"] = [0] + [int(v) for v in changed[0]]
            row["header"] = mb.drift_header(drift[1])
        rows[name] = row
        log(f"drift {name}: plan p50 {row['plan_us']['p50']} us, {row['replans']} replans "
            f"({row['guard_replans']} guarded), {row['replica_changes']} replica changes, "
            f"IR mean {row['ir_after_mean']}, fatal {row['fatal_calls']}")
    every = rows["every_call"]["replica_changes"]
    return {
        "calls": T, "reps": reps, "plans_timed_per_setting": reps * T,
        "weight_bytes_per_replica": w_bytes,
        "weight_model": f"W = 3*H*I*b, H={wl.hidden}, I={WEIGHT_I}, b={WEIGHT_B}",
        "replica_weight_bytes_avoided_by_gate": (every - rows["gate"]["replica_changes"]) * w_bytes,
        "settings": rows,
    }


def _speed_ratio(load, speeds, wl):
    """max_r load_r / (N*K * s_r / sum s): a rank's rows over its share in
    proportion to its speed (1 = every rank finishes together)."""
    import numpy as np

    share = wl.n_tokens * wl.top_k * speeds.astype(np.float64) / float(speeds.sum())
    return (load / share).max()


def cpu_baseline(wl, fraction: int = 2) -> dict:
    """The CPU oracle as it stands (single thread, pinned to one core) on
    1/fraction of the tokens of the same workload: plan, dispatch and combine,
    the median of five runs of each; GB/s over the same algorithmic bytes,
    plus the oracle's plan time on the full call."""
    import numpy as np

    import oracle as O
    import workload as W

    sub = wl.scaled(wl.n_tokens // fraction)
    ids, w = W.routing_for(sub)
    x, xs = W.token_rows(sub)
    # The smaller routing sample need not balance to exactly T with the same
    # slots, so its regions get room for 2 * S * K rows (same per-pair work).
    od = O.dims_for(sub, cap=2 * sub.cap)
    rows = od.n_ranks * od.cap
    # Outputs allocated and touched outside the timed region.
    buf = np.empty((rows, O.row_bytes_in(od)), np.uint8)
    buf.fill(0)
    y64 = np.empty((sub.n_tokens, od.hidden), np.float64)
    y64.fill(0.0)
    mag = np.empty_like(y64)
    mag.fill(0.0)
    speeds = W.rank_speeds(wl)
    if od.dtype_out == O.BF16 and od.dtype_in == O.BF16:
        y_exp = None  # the dispatch buffer itself (identity experts)
    elif od.dtype_out == O.F32 and od.dtype_in == O.F32:
        y_exp = None
    else:
        y_exp = W.rows_bf16(sub.seed, W.TAG_YEXP, od.hidden, n=rows)
    # One thread pinned to one host core; each stage timed five times (about
    # 10 s of oracle work at the prefill workloads) and the median kept.
    try:
        prev = os.sched_getaffinity(0)
        core = min(prev)
        os.sched_setaffinity(0, {core})
    except (AttributeError, OSError):
        prev, core = None, None
    tp, td, tc = [], [], []
    try:
        for _ in range(5):
            t0 = time.perf_counter()
            p = O.plan(od, ids, speeds=speeds)
            t1 = time.perf_counter()
            O.dispatch(od, p, x, xs, out=buf)
            t2 = time.perf_counter()
            ye = y_exp
            if ye is None:
                ye = buf.view(np.uint16 if od.dtype_out == O.BF16 else np.float32).reshape(
                    -1, od.hidden)
            t3 = time.perf_counter()
            O.combine(od, p.pos, p.status, w, ye, out=(y64, mag))
            t4 = time.perf_counter()
            tp.append(t1 - t0)
            td.append(t2 - t1)
            tc.append(t4 - t3)
        if p.flags & O.ST_FATAL:
            raise RuntimeError(f"oracle sample plan failed: status {p.status.tolist()}")
        full_ids, _ = W.routing_for(wl)
        f0 = time.perf_counter()
        O.plan(O.dims_for(wl), full_ids, speeds=speeds)
        f1 = time.perf_counter()
    finally:
        if prev is not None:
            os.sched_setaffinity(0, prev)
    med = lambda v: sorted(v)[len(v) // 2]  # noqa: E731
    t_plan, t_disp, t_comb = med(tp), med(td), med(tc)
    ab = algorithmic_bytes(sub)
    return {
        "value": round((ab["dispatch"] + ab["combine"]) / (t_disp + t_comb) / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{sub.n_tokens} of {wl.n_tokens} tokens of {wl.name} (same routing model, "
                  f"same E/K/P/R/H, regions of 2*S*K rows): plan + dispatch + combine, "
                  f"single-threaded C oracle pinned to one core, median of 5 runs per stage",
        "plan_us_sample": round(t_plan * 1e6, 1),
        "dispatch_s": round(t_disp, 3),
        "combine_s": round(t_comb, 3),
        "plan_us_full_call": round((f1 - f0) * 1e6, 1),
        "pinned_core": core,
        "host_cpu": _cpu_model(),
        "host_nproc": os.cpu_count(),
    }


CEILING_LIB = os.path.join(ROOT, "token_dispatch_mb_amd", "libmoebal_ceiling.so")


def _ceiling_lib():
    import ctypes

    if not os.path.exists(CEILING_LIB):
        raise RuntimeError(f"{CEILING_LIB} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(CEILING_LIB)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.mbc_fill.argtypes = [vp, i64, vp]
    L.mbc_copy.argtypes = [vp, vp, i64, vp]
    L.mbc_read.argtypes = [vp, i64, ctypes.POINTER(ctypes.c_uint32), vp, vp]
    L.mbc_scatter_write.argtypes = [vp, vp, i32, i32, i32, i32, vp]
    L.mbc_row_write.argtypes = [vp, vp, i32, i32, i32, i32, vp]
    L.mbc_gather_xor.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
    for f in (L.mbc_fill, L.mbc_copy, L.mbc_read, L.mbc_scatter_write, L.mbc_row_write,
              L.mbc_gather_xor):
        f.restype = ctypes.c_int
    return L


def ceiling_report(wl, dims, mb, W, torch, np, dev, reps: int) -> dict:
    """The dispatch and the combine against reference kernels of the same
    traffic on this GPU (libmoebal_ceiling): the dispatch's writes alone at
    its own rows, one KiB per wave and one row per wave; a contiguous fill of
    the same write bytes; a contiguous read of its read bytes; a contiguous
    copy; the combine's gathers and writes with an XOR for its arithmetic.
    Each kernel `reps` times, HIP events around each launch on the launch
    stream, the median kept; inputs resident and the plan made before. Every
    timed launch follows an untimed read of 512 MiB of a buffer of its own
    (torch's max reduction, so that profiles tell it from these kernels),
    which leaves nothing of the kernels' data in the 256 MB last-level cache
    (back to back, the combine measured 8 % slower: its previous launch's
    output lines were still cached)."""
    import ctypes

    L = _ceiling_lib()
    ids, _ = W.routing_for(wl)
    x, xs = W.token_rows(wl)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
    x_d = torch.from_numpy(x).view(tdt[wl.dtype_in]).to(dev)
    xs_d = torch.from_numpy(xs).to(dev) if xs is not None else None
    del x
    bufs = mb.PlanBuffers.allocate(dims, dev)
    ws = mb.alloc_workspace(dims, dev)
    mb.plan(dims, torch.from_numpy(ids).to(dev), ws, bufs, speeds=W.rank_speeds(wl))
    status = mb.plan_status(bufs)
    if status[0] & mb.ST_FATAL:
        raise RuntimeError(f"plan failed: {status.tolist()}")
    row_bytes = x_d[0].numel() * x_d.element_size()
    N, K = wl.n_tokens, wl.top_k
    buf = torch.empty((dims.rows, wl.hidden), dtype=tdt[wl.dtype_in], device=dev)
    bs = (torch.empty((dims.rows, wl.hidden // 128), dtype=torch.float32, device=dev)
          if wl.dtype_in == "fp8" else None)
    _, w = W.routing_for(wl)
    w_d = torch.from_numpy(w).to(dev)
    odt = {"f32": torch.float32, "bf16": torch.bfloat16}[wl.dtype_out]
    out_row = wl.hidden * (4 if wl.dtype_out == "f32" else 2)
    # expert outputs: the dispatch buffer itself when the row types agree
    ye = buf if wl.dtype_in == wl.dtype_out else torch.zeros((dims.rows, wl.hidden), dtype=odt,
                                                              device=dev)
    y = torch.empty((N, wl.hidden), dtype=odt, device=dev)
    write_b, read_b = N * K * row_bytes, N * row_bytes
    # fp8 rows: the dispatch also reads each scale row once and writes it K times
    scale_b = N * (1 + K) * (wl.hidden // 128) * 4 if wl.dtype_in == "fp8" else 0
    assert write_b <= buf.numel() * buf.element_size() and read_b == x_d.numel() * x_d.element_size()
    half = write_b // 32 * 16  # the copy reads and writes this many bytes
    src = torch.empty(half, dtype=torch.uint8, device=dev)
    src.fill_(0x3c)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    evict_buf = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
    key = (ctypes.c_uint32 * 4)(0xDEADBEEF, 0x0BADF00D, 0x12345678, 0x9ABCDEF1)
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def check(rc, name):
        if rc != 0:
            raise RuntimeError(f"{name} returned {rc}")

    cases = {
        "k_dispatch": (lambda: mb.dispatch(dims, bufs, x_d, buf, xs_d, bs),
                       read_b + write_b + N * K * 4 + scale_b),
        "k_scatter_write": (lambda: check(L.mbc_scatter_write(ptr(bufs.pos), ptr(buf), N, K,
                                                              row_bytes, dims.rows, sh),
                                          "mbc_scatter_write"), write_b + N * K * 4),
        "k_row_write": (lambda: check(L.mbc_row_write(ptr(bufs.pos), ptr(buf), N, K, row_bytes,
                                                      dims.rows, sh), "mbc_row_write"),
                        write_b + N * K * 4),
        "k_fill": (lambda: check(L.mbc_fill(ptr(buf), write_b, sh), "mbc_fill"), write_b),
        "k_read": (lambda: check(L.mbc_read(ptr(x_d), read_b, key, ptr(sink), sh), "mbc_read"),
                   read_b),
        "k_copy": (lambda: check(L.mbc_copy(ptr(src), ptr(buf), half, sh), "mbc_copy"), 2 * half),
        "k_combine": (lambda: mb.combine(dims, bufs, ye, w_d, y),
                      N * K * out_row + N * K * 8 + N * out_row),
        "k_gather_xor": (lambda: check(L.mbc_gather_xor(ptr(bufs.pos), ptr(ye), ptr(y), N, K, out_row,
                                                        dims.rows, sh), "mbc_gather_xor"),
                         N * K * out_row + N * K * 4 + N * out_row),
    }
    def evict():
        evict_buf.max()

    out = {}
    for name, (fn, nbytes) in cases.items():
        fn()  # warm
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for e in ev:
            evict()
            e[0].record()
            fn()
            e[1].record()
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)[reps // 2]
        gbps = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us": round(us, 2), "bytes": int(nbytes), "gbps": round(gbps, 1),
                     "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}
        log(f"ceiling {name}: {us:.1f} us, {gbps:.0f} GB/s")
    if int(sink.abs().sum()) != 0:
        raise RuntimeError("mbc_read found its key in the rows")
    d_us = out["k_dispatch"]["us"]
    best_w = min(out["k_scatter_write"]["us"], out["k_row_write"]["us"])
    return {
        "workload": wl.name, "reps": reps, "row_bytes": row_bytes,
        "kernels": out,
        "dispatch_time_over_its_writes_alone": round(d_us / best_w, 4),
        "dispatch_gbps_over_write_only_scatter_gbps": round(
            out["k_dispatch"]["gbps"] / max(out["k_scatter_write"]["gbps"],
                                            out["k_row_write"]["gbps"]), 4),
        "write_only_scatter_over_fill": round(out["k_fill"]["us"] / best_w, 4),
        "combine_gbps_over_gather_xor_gbps": round(out["k_combine"]["gbps"] /
                                                   out["k_gather_xor"]["gbps"], 4),
    }


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; a workload of several calls: five passes over "
                         "them; a drift-gated sequence: one pass)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_prefill")
    ap.add_argument("--combine-fp8", action="store_true",
                    help="fp8-row workloads: expert outputs stay fp8 with their scales and "
                         "mb_combine_fp8 dequantises while combining")
    ap.add_argument("--graph", action="store_true",
                    help="also time the steps replayed from HIP graphs captured once per "
                         "(call, buffer set): the launch cost leaves the step")
    ap.add_argument("--repair", action="store_true",
                    help="plan with the quota repair after placement (mb_plan_ex)")
    ap.add_argument("--skip-cpu-baseline", action="store_true",
                    help="leave out the CPU oracle leg (for profiler runs)")
    ap.add_argument("--no-backlog", action="store_true",
                    help="start the timed steps on an idle GPU (no queued work ahead of them)")
    ap.add_argument("--ceiling", action="store_true",
                    help="only time k_dispatch beside the reference kernels that bound it "
                         "(its writes alone, a fill, a read, a copy) and print that report")
    ap.add_argument("--reps", type=int, default=9, help="launches per kernel with --ceiling")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run torch's device copy of MIB MiB three times (the known-size "
                         "reference for the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the P logical ranks of the expert-parallel group are "
              "partitions of one GPU's memory, so there is nothing to run on more GPUs.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import token_dispatch_mb_amd as mb
    import workload as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration * 1024 * 1024
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return 0
    wl = W.get_workload(args.workload)
    dims = mb.Dims.for_workload(wl)
    log(f"workload {wl.name}: {wl.note}")
    if args.ceiling:
        print(json.dumps({"ceiling": ceiling_report(wl, dims, mb, W, torch, np, dev, args.reps)}),
              flush=True)
        return 0
    if args.steps is None:
        args.steps = 20 if wl.calls == 1 else wl.calls if wl.drift else 5 * wl.calls

    ids, w = W.routing_for(wl)
    x, xs = W.token_rows(wl)
    log("inputs generated")
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
    ids_d = torch.from_numpy(ids).to(dev)
    w_d = torch.from_numpy(w).to(dev)
    # A workload smaller than the 256 MB last-level cache would be timed
    # warm: its row buffers come in enough sets (at least 1 GiB in all,
    # at most 32) that each step touches buffers no recent step touched.
    eb = {"f32": 4, "bf16": 2, "fp8": 1}
    row_in = wl.hidden * eb[wl.dtype_in] + (wl.hidden // 128 * 4 if wl.dtype_in == "fp8" else 0)
    footprint = (wl.n_tokens + dims.rows) * row_in + (dims.rows + wl.n_tokens) * wl.hidden * \
        eb[wl.dtype_out]
    nsets = min(32, max(1, -(-(1 << 30) // footprint)))
    x_sets = [torch.from_numpy(x).view(tdt[wl.dtype_in]).to(dev) for _ in range(nsets)]
    xs_sets = [torch.from_numpy(xs).to(dev) if xs is not None else None for _ in range(nsets)]
    x_d, xs_d = x_sets[0], xs_sets[0]
    del x
    bufs = mb.PlanBuffers.allocate(dims, dev)
    ws = mb.alloc_workspace(dims, dev)
    buf_sets = [torch.empty((dims.rows, wl.hidden), dtype=tdt[wl.dtype_in], device=dev)
                for _ in range(nsets)]
    bs_sets = [torch.empty((dims.rows, wl.hidden // 128), dtype=torch.float32, device=dev)
               if wl.dtype_in == "fp8" else None for _ in range(nsets)]
    y_sets = [torch.empty((wl.n_tokens, wl.hidden), dtype=tdt[wl.dtype_out], device=dev)
              for _ in range(nsets)]
    buf, bs, y = buf_sets[0], bs_sets[0], y_sets[0]
    y_exp_sets = [torch.empty((dims.rows, wl.hidden), dtype=tdt[wl.dtype_out], device=dev)
                  for _ in range(nsets if not args.combine_fp8 else 1)]
    y_exp = y_exp_sets[0]
    # A workload of several calls (layers, or passes of one layer) steps
    # through its calls' routing decisions, one call per step.
    if wl.calls > 1:
        rw = [W.routing_for(wl, c) for c in range(wl.calls)]
        ids_all = torch.stack([torch.from_numpy(r[0]) for r in rw]).to(dev)
        w_all = torch.stack([torch.from_numpy(r[1]) for r in rw]).to(dev)
        del rw
        log(f"{wl.calls} calls of routing resident; {nsets} buffer set(s)")
    else:
        ids_all, w_all = ids_d.unsqueeze(0), w_d.unsqueeze(0)

    # Rank speeds of a workload planned against per-rank targets (None: the
    # single water level). For comparison, the equal-target plan's largest
    # ratio of load to the speed-proportional share, outside the timing.
    speeds = W.rank_speeds(wl)
    # A drift-gated workload: a drift state (zero-filled = fresh) for the layer.
    drift = None
    if wl.drift:
        drift = (mb.DriftParams(*wl.drift), mb.alloc_drift_state(dims, dev))
        log(f"drift gate {wl.drift}")

    def plan_call(i):
        mb.plan(dims, ids_all[i % wl.calls], ws, bufs, speeds=speeds, drift=drift,
                repair=args.repair)

    wir_equal = None
    if speeds is not None:
        mb.plan(dims, ids_d, ws, bufs)
        wir_equal = float(_speed_ratio(bufs.load_post.cpu().numpy(), speeds, wl))

    # Expert outputs: the dispatched rows (identity experts), or for fp8
    # rows a generated bf16 buffer (or, with --combine-fp8, the dispatched
    # fp8 rows and scales themselves).
    mb.plan(dims, ids_d, ws, bufs, speeds=speeds, repair=args.repair)
    if args.combine_fp8:
        if wl.dtype_in != "fp8":
            print("--combine-fp8 needs a workload with fp8 rows", file=sys.stderr)
            return 2
        y_exp8 = torch.empty((dims.rows, wl.hidden), dtype=torch.uint8, device=dev)
        ys8 = torch.empty((dims.rows, wl.hidden // 128), dtype=torch.float32, device=dev)
        mb.dispatch(dims, bufs, x_d, y_exp8, xs_d, ys8)
    elif wl.dtype_in == wl.dtype_out:
        for ye in y_exp_sets:
            mb.dispatch(dims, bufs, x_d, ye, xs_d, bs)
    else:
        gen = torch.from_numpy(W.rows_bf16(wl.seed, W.TAG_YEXP, wl.hidden, n=dims.rows))
        for ye in y_exp_sets:
            ye.copy_(gen.view(torch.bfloat16))
        del gen
    status = mb.plan_status(bufs)
    log(f"status {status.tolist()} (flags, T, max load, moves)")

    def step(i, ev=None):
        if ev is not None:
            ev[0].record()
        plan_call(i)
        if ev is not None:
            ev[1].record()
        k = i % nsets
        mb.dispatch(dims, bufs, x_sets[k], buf_sets[k], xs_sets[k], bs_sets[k])
        if ev is not None:
            ev[2].record()
        wi = w_all[i % wl.calls]
        if args.combine_fp8:
            mb.combine_fp8(dims, bufs, y_exp8, ys8, wi, y_sets[k])
        else:
            mb.combine(dims, bufs, y_exp_sets[k % len(y_exp_sets)], wi, y_sets[k])
        if ev is not None:
            ev[3].record()

    if wl.calls > 1:
        # One untimed pass over the calls queued without a wait: the runtime's
        # first deep queue of launches stalls the host once (34 ms at step 37
        # of decode_drift, measured), which would otherwise fall in the timed
        # steps and idle the GPU behind it.
        for i in range(wl.calls):
            step(i)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    _backlog(torch, dev, 0.0)  # its buffer and fill rate, before timing
    if drift is not None:
        drift[1].zero_()  # the timed steps run the sequence from its first call
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done; timing {args.steps} steps")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    # The timed steps queue behind about backlog_ms of unrelated GPU work
    # (fills of a scratch buffer, before the first step's event), so the host
    # starts that far ahead: a step shorter than its launches' host time
    # (decode) is then timed on the GPU, not at the host's launch rate.
    backlog_ms = 0.0 if args.no_backlog else 30.0
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    if backlog_ms:
        _backlog(torch, dev, backlog_ms)
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0

    plan_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    disp_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    comb_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    total_ms = evs[0][0].elapsed_time(evs[-1][3])
    ms_per_step = total_ms / args.steps
    ab = algorithmic_bytes(wl, combine_fp8=args.combine_fp8)
    bytes_step = ab["dispatch"] + ab["combine"]
    value = bytes_step / (ms_per_step * 1e-3) / 1e9
    d_gbps = ab["dispatch"] / (disp_ms.mean() * 1e-3) / 1e9
    c_gbps = ab["combine"] / (comb_ms.mean() * 1e-3) / 1e9
    comb_name = "k_combine_fp8" if args.combine_fp8 else "k_combine"
    # the dispatch kernel libmoebal launches for these rows: rows of whole
    # 2 KiB spans with 2 <= K <= 16 take k_dispatch_span, the rest k_dispatch
    span_rows = (row_in - (wl.hidden // 128 * 4 if wl.dtype_in == "fp8" else 0)) % 2048 == 0
    disp_name = "k_dispatch_span" if span_rows and 2 <= wl.top_k <= 16 else "k_dispatch"
    dominant = comb_name if comb_ms.mean() >= disp_ms.mean() else disp_name
    dom_bytes = ab["combine"] if dominant == comb_name else ab["dispatch"]
    dom_ms = comb_ms.mean() if dominant == comb_name else disp_ms.mean()
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9

    # Correctness spot check of the timed buffers (identity experts: the
    # combined row is sum_k w_k x_t).
    status = mb.plan_status(bufs)
    mean_load = wl.n_tokens * wl.top_k / wl.n_ranks
    # pairs served on a rank other than the one their token originates on
    src = torch.arange(wl.n_tokens, device=dev).unsqueeze(1) // wl.tokens_per_rank
    nonlocal_pairs = int((bufs.pos.view(wl.n_tokens, wl.top_k) // wl.cap != src).sum())
    if wl.dtype_in == wl.dtype_out and wl.calls == 1 and not args.combine_fp8:
        samp = torch.arange(0, wl.n_tokens, max(1, wl.n_tokens // 256), device=dev)
        y_last = y_sets[(args.steps - 1) % nsets]
        err = (y_last[samp].float() - x_d[samp].float() * w_d[samp].sum(1, keepdim=True)).abs().max()
        log(f"identity-expert check: max |y - x * sum(w)| = {float(err):.3e}")

    drift_report = None
    if drift is not None:
        drift_report = _drift_report(wl, dims, ids_all, ws, bufs, speeds, args.repair, mb, torch,
                                     np)
        drift[1].zero_()

    graph_report = None
    if args.graph:
        # One graph per distinct (call, buffer set) of the step sequence,
        # captured after the eager run and its checks; the replays take the same steps.
        graphs = {}
        torch.cuda.synchronize()
        for i in range(args.steps):
            key = (i % wl.calls, i % nsets)
            if key not in graphs:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step(i)
                graphs[key] = g
        if drift is not None:
            drift[1].zero_()
        for i in range(min(args.warmup, args.steps)):
            graphs[(i % wl.calls, i % nsets)].replay()
        if drift is not None:
            drift[1].zero_()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        g0.record()
        for i in range(args.steps):
            graphs[(i % wl.calls, i % nsets)].replay()
        g1.record()
        torch.cuda.synchronize()
        g_ms = g0.elapsed_time(g1) / args.steps
        graph_report = {"graphs": len(graphs), "ms_per_step": round(g_ms, 4)}
        log(f"graph replay: {g_ms:.4f} ms per step over {len(graphs)} graph(s)")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype_in == "bf16" else wl.dtype_in,
        "data": "synthetic",
        "config": {
            "workload": wl.name, "tokens": wl.n_tokens, "experts": wl.n_experts,
            "top_k": wl.top_k, "logical_ranks": wl.n_ranks, "replica_slots_per_rank":
                wl.slots_per_rank, "hidden": wl.hidden, "rows_in": wl.dtype_in,
            "rows_out": wl.dtype_out, "cap": wl.cap,
            "expert_outputs": "fp8+scales" if args.combine_fp8 else wl.dtype_out,
            "calls": wl.calls, "buffer_sets": nsets,
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "dispatch_combine_gbps": round(bytes_step / ((disp_ms.mean() + comb_ms.mean()) * 1e-3) / 1e9, 2),
        "plan_us": {"mean": round(plan_ms.mean() * 1e3, 2), "p50": round(float(np.median(plan_ms)) * 1e3, 2),
                    "p99": round(float(np.percentile(plan_ms, 99)) * 1e3, 2)},
        "dispatch_us": round(disp_ms.mean() * 1e3, 2),
        "combine_us": round(comb_ms.mean() * 1e3, 2),
        "dispatch_us_p50_p99": [round(float(np.median(disp_ms)) * 1e3, 2),
                                round(float(np.percentile(disp_ms, 99)) * 1e3, 2)],
        "combine_us_p50_p99": [round(float(np.median(comb_ms)) * 1e3, 2),
                               round(float(np.percentile(comb_ms, 99)) * 1e3, 2)],
        "dispatch_gbps": round(d_gbps, 2),
        "combine_gbps": round(c_gbps, 2),
        "algorithmic_bytes": {"dispatch": ab["dispatch"], "combine": ab["combine"]},
        "plan_status": {"flags": int(status[0]), "water_level": int(status[1]),
                        "max_load": int(status[2]), "moves": int(status[3]),
                        "ir_after": round(float(status[2]) / mean_load, 5),
                        "nonlocal_pairs": nonlocal_pairs, "quota_repair": bool(args.repair)},
        "speed_targets": None if speeds is None else {
            "max_load_over_share": round(float(_speed_ratio(bufs.load_post.cpu().numpy(), speeds, wl)), 5),
            "same_with_equal_targets": round(wir_equal, 5)},
        "drift_gate": drift_report,
        "graph_replay": None if graph_report is None else dict(
            graph_report, value=round((ab["dispatch"] + ab["combine"]) /
                                      (graph_report["ms_per_step"] * 1e-3) / 1e9, 2)),
        "wall_s_timed": round(t_wall, 4),
        "backlog_ms": backlog_ms,
        "roofline": {
            "kernel": dominant,
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic("k_dispatch" if dominant == disp_name else comb_name,
                                        wl.name),
        },
    }
    del buf, y_exp, y, x_d, xs_d, bs, buf_sets, y_exp_sets, y_sets, x_sets, xs_sets, bs_sets
    torch.cuda.empty_cache()
    if not args.skip_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(wl)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
