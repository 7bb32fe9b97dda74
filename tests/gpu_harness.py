"""Helpers for the GPU parity tests: run libmoebal through its C ABI on
seeded inputs and fetch results for comparison with the CPU oracle."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle as O
import token_dispatch_mb_amd as mb
import workload as W

PLAN_FIELDS = ("counts", "load_pre", "load_post", "rep_expert", "slot_quota", "cu_seqlens",
               "pos", "row_src", "status")

# Combine tolerance, relative to sum_k |w_k * y_k| per element: fp32 output
# (fp32 accumulation of K terms errs by at most ~K * 2^-24 of that sum) and
# bf16 output (one final rounding, 2^-9 of |y|).
TOL = {"f32": 1e-5, "bf16": 1e-2}


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def dev() -> torch.device:
    return torch.device("cuda:0")


class GpuPlan:
    def __init__(self, dims: mb.Dims, device=None):
        self.dims = dims
        self.device = device or dev()
        self.bufs = mb.PlanBuffers.allocate(dims, self.device)
        self.ws = mb.alloc_workspace(dims, self.device)

    def run(self, ids: np.ndarray | torch.Tensor, stream=None, speeds=None, drift=None,
            repair=False):
        ids_d = ids if isinstance(ids, torch.Tensor) else torch.from_numpy(
            np.ascontiguousarray(ids, np.int32)).to(self.device)
        mb.plan(self.dims, ids_d, self.ws, self.bufs, stream, speeds=speeds, drift=drift,
                repair=repair)
        return self

    def fetch(self) -> dict:
        torch.cuda.synchronize()
        out = {}
        for name in PLAN_FIELDS:
            out[name] = getattr(self.bufs, name).cpu().numpy()
        out["rep_expert"] = out["rep_expert"][:, : self.dims.slots_per_rank]
        return out


def assert_plan_equal(gpu: dict, ref: O.Plan, check_layout: bool = True) -> None:
    """Bit-exact comparison of every integer output the header defines: all
    of them for a usable plan; everything but pos and row_src under a fatal
    status (with bad or repeated ids the counts, loads, quotas and
    cu_seqlens are all 0 and every replica slot is empty)."""
    assert np.array_equal(gpu["status"], ref.status), (gpu["status"], ref.status)
    for name in ("counts", "load_pre", "load_post", "rep_expert", "slot_quota", "cu_seqlens"):
        g = gpu[name].reshape(getattr(ref, name).shape)
        assert np.array_equal(g, getattr(ref, name)), name
    if check_layout and not ref.status[0] & O.ST_FATAL:
        assert np.array_equal(gpu["pos"].reshape(ref.pos.shape), ref.pos), "pos"
        assert np.array_equal(gpu["row_src"], ref.row_src), "row_src"


def torch_rows(a: np.ndarray, dtype_code: int) -> torch.Tensor:
    """Host rows (float32, uint16 bf16 bits, uint8 fp8) as a device tensor of
    the matching storage type."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype_code == O.BF16:
        t = t.view(torch.bfloat16)
    return t.to(dev())


def rows_to_bytes(t: torch.Tensor) -> np.ndarray:
    """Device rows -> host uint8 [rows, row_bytes]."""
    a = t.contiguous().view(torch.uint8).cpu().numpy()
    return a.reshape(t.shape[0], -1)


def out_dtype(dims) -> torch.dtype:
    return torch.float32 if dims.dtype_out == O.F32 else torch.bfloat16


def in_dtype(dims) -> torch.dtype:
    return {O.F32: torch.float32, O.BF16: torch.bfloat16, O.FP8_E4M3: torch.uint8}[dims.dtype_in]


def y_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def assert_combine_close(y_gpu: np.ndarray, y_ref: np.ndarray, mag: np.ndarray, dtype_out: str):
    tol = TOL[dtype_out]
    err = np.abs(y_gpu - y_ref)
    bound = tol * mag + 1e-30
    bad = err > bound
    assert not bad.any(), (f"{int(bad.sum())} elements out of tolerance; worst ratio "
                           f"{float((err / bound).max()):.3g}")


def run_rows(dims: mb.Dims, gp: GpuPlan, x: np.ndarray, xs: np.ndarray | None,
             y_exp: np.ndarray, w: np.ndarray, sentinel: int = 0xA5):
    """Dispatch x and combine y_exp on the GPU with plan `gp`; returns
    (buf bytes, buf scales or None, y as float64)."""
    d = dev()
    x_d = torch_rows(x, dims.dtype_in)
    buf = torch.full((dims.rows, dims.hidden * O.ELT_BYTES[dims.dtype_in]), sentinel,
                     dtype=torch.uint8, device=d)
    buf_t = buf.view(in_dtype(dims)) if dims.dtype_in != O.FP8_E4M3 else buf
    xs_d = bs = None
    if xs is not None:
        xs_d = torch.from_numpy(np.ascontiguousarray(xs, np.float32)).to(d)
        bs = torch.zeros((dims.rows, dims.hidden // 128), dtype=torch.float32, device=d)
    mb.dispatch(dims, gp.bufs, x_d, buf_t, xs_d, bs)
    ye = torch_rows(y_exp, dims.dtype_out)
    w_d = torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(d)
    y = torch.full((dims.n_tokens, dims.hidden), float("nan"), dtype=out_dtype(dims), device=d)
    mb.combine(dims, gp.bufs, ye, w_d, y)
    torch.cuda.synchronize()
    return (buf.cpu().numpy(), None if bs is None else bs.cpu().numpy(), y_to_f64(y))
