"""CPU oracle for hot-expert replication and token dispatch/combine.

TEST INFRASTRUCTURE ONLY. The oracle (``mbref.c``, built to ``libmbref.so``)
defines the expected results the GPU library is checked against. Only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
this package; the GPU path (``token_dispatch_mb_amd``) never does, and the two
share no code.

This module only marshals numpy arrays to the C functions.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MBREF_LIB points the tests at another build of mbref.c (the mutation test
# builds deliberately broken copies to check that the pins catch them).
LIB_PATH = os.environ.get("MBREF_LIB") or os.path.join(_HERE, "libmbref.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
DTYPES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}
ELT_BYTES = {F32: 4, BF16: 2, FP8_E4M3: 1}

ST_BAD_ID, ST_DUP_ID, ST_UNBALANCED, ST_CAPACITY = 1, 2, 4, 8
ST_FATAL = ST_BAD_ID | ST_DUP_ID | ST_CAPACITY
ST_REPLANNED = 16
ST_GUARDED = 32

MOVE_FILL_HOST, MOVE_EXCESS_ONLY = 0, 1

ERR_INVALID_ARG = -1


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_tokens", "top_k", "n_experts", "n_ranks", "slots_per_rank", "hidden", "cap",
        "dtype_in", "dtype_out")]


_i32p = ctypes.POINTER(ctypes.c_int32)


class PlanOut(ctypes.Structure):
    _fields_ = [(n, _i32p) for n in (
        "counts", "load_pre", "load_post", "rep_expert", "slot_quota", "cu_seqlens", "pos",
        "row_src", "host", "status")]


class Report(ctypes.Structure):
    _fields_ = [("ir_before", ctypes.c_double), ("ir_after", ctypes.c_double),
                ("maxvio", ctypes.c_double), ("excess_removed", ctypes.c_double),
                ("water_level", ctypes.c_int64), ("n_moves", ctypes.c_int64),
                ("slots_used", ctypes.c_int64), ("excess_before", ctypes.c_int64),
                ("offhome_pairs", ctypes.c_int64), ("nonlocal_pairs", ctypes.c_int64),
                ("wir_before", ctypes.c_double), ("wir_after", ctypes.c_double)]


class DriftParams(ctypes.Structure):
    """Drift gate and load guard; tol_num = tol_den = 0 (the default) guards
    the region size only."""
    _fields_ = [(n, ctypes.c_int32) for n in ("delta_num", "delta_den", "window", "check_every",
                                             "tol_num", "tol_den")]


class _DriftStateC(ctypes.Structure):
    _fields_ = [("have_plan", ctypes.c_int32), ("countdown", ctypes.c_int32),
                ("nwin", ctypes.c_int32), ("n_moves", ctypes.c_int32),
                ("calls", ctypes.c_int64), ("replans", ctypes.c_int64),
                ("guarded", ctypes.c_int64), ("last_d", ctypes.c_double),
                ("wsum", ctypes.POINTER(ctypes.c_int64)), ("rep", _i32p), ("order", _i32p)]


class DriftState:
    """State of one layer's drift-gated planning (host memory)."""

    def __init__(self, n_experts: int, n_ranks: int, slots_per_rank: int):
        self.wsum = np.zeros(n_experts, np.int64)
        self.rep = np.full(n_ranks * slots_per_rank, -1, np.int32)
        self.order = np.full(n_ranks * slots_per_rank, -1, np.int32)
        self.c = _DriftStateC(0, 0, 0, 0, 0, 0, 0, 0.0,
                              self.wsum.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                              self.rep.ctypes.data_as(_i32p), self.order.ctypes.data_as(_i32p))

    def __getattr__(self, name):
        if name in ("have_plan", "countdown", "nwin", "n_moves", "calls", "replans", "guarded",
                    "last_d"):
            return getattr(self.c, name)
        raise AttributeError(name)


class _PlanOptionsC(ctypes.Structure):
    _fields_ = [("rank_speed", ctypes.c_void_p), ("drift", ctypes.POINTER(DriftParams)),
                ("drift_state", ctypes.POINTER(_DriftStateC)), ("quota_repair", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        L.mbref_plan.argtypes = [ctypes.POINTER(Dims), vp, ctypes.c_int32,
                                 ctypes.POINTER(PlanOut), ctypes.POINTER(Report)]
        L.mbref_plan.restype = ctypes.c_int
        L.mbref_plan_weighted.argtypes = [ctypes.POINTER(Dims), vp, vp, ctypes.c_int32,
                                          ctypes.POINTER(PlanOut), ctypes.POINTER(Report)]
        L.mbref_plan_weighted.restype = ctypes.c_int
        L.mbref_plan_drift.argtypes = [ctypes.POINTER(Dims), vp, vp, ctypes.POINTER(DriftParams),
                                       ctypes.POINTER(_DriftStateC), ctypes.POINTER(PlanOut),
                                       ctypes.POINTER(Report)]
        L.mbref_plan_drift.restype = ctypes.c_int
        L.mbref_plan_ex.argtypes = [ctypes.POINTER(Dims), vp, ctypes.POINTER(_PlanOptionsC),
                                    ctypes.POINTER(PlanOut), ctypes.POINTER(Report)]
        L.mbref_plan_ex.restype = ctypes.c_int
        L.mbref_circle_schedule.argtypes = [ctypes.c_int32, vp]
        L.mbref_circle_schedule.restype = None
        L.mbref_e4m3_value.argtypes = [ctypes.c_uint8]
        L.mbref_e4m3_value.restype = ctypes.c_double
        L.mbref_combine_fp8.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, vp, vp, ctypes.c_int32,
                                        ctypes.c_int32, vp, vp]
        L.mbref_combine_fp8.restype = ctypes.c_int
        L.mbref_dispatch.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, vp, vp, vp]
        L.mbref_dispatch.restype = ctypes.c_int
        L.mbref_dispatch_window.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, vp,
                                            ctypes.c_int64, ctypes.c_int64, vp, vp]
        L.mbref_dispatch_window.restype = ctypes.c_int
        L.mbref_combine.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, vp, ctypes.c_int32,
                                    ctypes.c_int32, vp, vp]
        L.mbref_combine.restype = ctypes.c_int
        L.mbref_version.restype = ctypes.c_int
        _lib = L
    return _lib


def make_dims(n_tokens, top_k, n_experts, n_ranks, slots_per_rank, hidden, cap=None,
              dtype_in="f32", dtype_out="f32") -> Dims:
    if cap is None:
        cap = (n_tokens // n_ranks) * top_k if n_ranks > 0 else 0
    return Dims(n_tokens, top_k, n_experts, n_ranks, slots_per_rank, hidden, cap,
                DTYPES.get(dtype_in, dtype_in) if isinstance(dtype_in, str) else dtype_in,
                DTYPES.get(dtype_out, dtype_out) if isinstance(dtype_out, str) else dtype_out)


def dims_for(wl, cap=None, n_tokens=None) -> Dims:
    n = wl.n_tokens if n_tokens is None else n_tokens
    if cap is None:
        cap = wl.cap if n_tokens is None else (n // wl.n_ranks) * wl.top_k
    return make_dims(n, wl.top_k, wl.n_experts, wl.n_ranks, wl.slots_per_rank, wl.hidden,
                     cap=cap,
                     dtype_in=wl.dtype_in, dtype_out=wl.dtype_out)


@dataclass
class Plan:
    dims: Dims
    counts: np.ndarray      # [P, E]
    load_pre: np.ndarray    # [P]
    load_post: np.ndarray   # [P]
    rep_expert: np.ndarray  # [P, R]
    slot_quota: np.ndarray  # [P, Eh+R]
    cu_seqlens: np.ndarray  # [P, Eh+R+1]
    pos: np.ndarray         # [N, K]
    row_src: np.ndarray     # [P*cap]
    host: np.ndarray        # [N, K]
    status: np.ndarray      # [4]
    report: dict

    @property
    def flags(self) -> int:
        return int(self.status[0])


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def plan(dims: Dims, ids: np.ndarray, move_rule: int = MOVE_FILL_HOST,
         speeds: np.ndarray | None = None, drift: tuple | None = None,
         repair: bool = False) -> Plan:
    """Steps O0-O4 and O7. ``speeds`` (int32 [P]) gives per-rank targets in
    proportion to rank speed in place of the single water level. ``drift`` =
    (DriftParams, DriftState) plans one call of a drift-gated sequence.
    ``repair`` runs the quota repair between placement and assignment."""
    N, K, E, P, R = dims.n_tokens, dims.top_k, dims.n_experts, dims.n_ranks, dims.slots_per_rank
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(N, K)
    eh = E // P if P > 0 else 0
    ns = eh + R
    a = {
        "counts": np.zeros((P, E), np.int32), "load_pre": np.zeros(P, np.int32),
        "load_post": np.zeros(P, np.int32), "rep_expert": np.zeros((P, R), np.int32),
        "slot_quota": np.zeros((P, ns), np.int32), "cu_seqlens": np.zeros((P, ns + 1), np.int32),
        "pos": np.zeros((N, K), np.int32), "row_src": np.zeros(max(P * dims.cap, 0), np.int32),
        "host": np.zeros((N, K), np.int32), "status": np.zeros(4, np.int32),
    }
    po = PlanOut(**{k: v.ctypes.data_as(_i32p) for k, v in a.items()})
    rep = Report()
    if repair:
        sp = None if speeds is None else np.ascontiguousarray(speeds, dtype=np.int32)
        opt = _PlanOptionsC(sp.ctypes.data if sp is not None else None,
                            ctypes.pointer(drift[0]) if drift else None,
                            ctypes.pointer(drift[1].c) if drift else None, 1)
        rc = lib().mbref_plan_ex(ctypes.byref(dims), _ptr(ids), ctypes.byref(opt),
                                 ctypes.byref(po), ctypes.byref(rep))
    elif drift is not None:
        prm, st = drift
        sp = None if speeds is None else np.ascontiguousarray(speeds, dtype=np.int32)
        rc = lib().mbref_plan_drift(ctypes.byref(dims), _ptr(ids),
                                    _ptr(sp) if sp is not None else None, ctypes.byref(prm),
                                    ctypes.byref(st.c), ctypes.byref(po), ctypes.byref(rep))
    elif speeds is None:
        rc = lib().mbref_plan(ctypes.byref(dims), _ptr(ids), move_rule, ctypes.byref(po),
                              ctypes.byref(rep))
    else:
        sp = np.ascontiguousarray(speeds, dtype=np.int32)
        assert sp.shape == (P,)
        rc = lib().mbref_plan_weighted(ctypes.byref(dims), _ptr(ids), _ptr(sp), move_rule,
                                       ctypes.byref(po), ctypes.byref(rep))
    if rc != 0:
        raise ValueError(f"mbref_plan returned {rc}")
    report = {n: getattr(rep, n) for n, _ in Report._fields_}
    return Plan(dims=dims, report=report, **a)


def plan_rc(dims: Dims, ids: np.ndarray, speeds: np.ndarray | None = None) -> int:
    """Return code of mbref_plan (or mbref_plan_weighted) alone, for invalid
    sizes and speeds."""
    N = max(dims.n_tokens, 0)
    K = max(dims.top_k, 0)
    P = max(dims.n_ranks, 1)
    E = max(dims.n_experts, 1)
    R = max(dims.slots_per_rank, 0)
    big = max(N * K, P * max(dims.cap, 1), P * E, P * (E + R + 1), 16)
    bufs = [np.zeros(big, np.int32) for _ in range(10)]
    po = PlanOut(*[b.ctypes.data_as(_i32p) for b in bufs])
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    if speeds is None:
        return lib().mbref_plan(ctypes.byref(dims), _ptr(ids), 0, ctypes.byref(po), None)
    sp = np.ascontiguousarray(speeds, dtype=np.int32)
    return lib().mbref_plan_weighted(ctypes.byref(dims), _ptr(ids), _ptr(sp), 0,
                                     ctypes.byref(po), None)


def plan_drift_rc(dims: Dims, ids: np.ndarray, params: DriftParams, state: DriftState) -> int:
    """Return code of mbref_plan_drift alone, for invalid parameters."""
    N = max(dims.n_tokens, 0)
    K = max(dims.top_k, 0)
    P = max(dims.n_ranks, 1)
    E = max(dims.n_experts, 1)
    R = max(dims.slots_per_rank, 0)
    big = max(N * K, P * max(dims.cap, 1), P * E, P * (E + R + 1), 16)
    bufs = [np.zeros(big, np.int32) for _ in range(10)]
    po = PlanOut(*[b.ctypes.data_as(_i32p) for b in bufs])
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    return lib().mbref_plan_drift(ctypes.byref(dims), _ptr(ids), None, ctypes.byref(params),
                                  ctypes.byref(state.c), ctypes.byref(po), None)


def circle_schedule(n_ranks: int) -> np.ndarray:
    """[rounds, pairs, 2] ranks met in each round of the quota repair's
    tournament (index n_ranks = the bye of an odd count)."""
    n = n_ranks + (n_ranks & 1)
    out = np.zeros((max(n - 1, 0), n // 2, 2), np.int32)
    if n >= 2:
        lib().mbref_circle_schedule(n_ranks, _ptr(out))
    return out


def row_bytes_in(dims: Dims) -> int:
    return dims.hidden * ELT_BYTES[dims.dtype_in]


def dispatch(dims: Dims, p: Plan, x: np.ndarray, x_scale: np.ndarray | None = None,
             row0: int = 0, row1: int | None = None, fill: int = 0, out: np.ndarray | None = None):
    """Rows [row0, row1) of the dispatch buffer as uint8 [rows, row_bytes]
    (rows no pair maps to hold ``fill``, or are left as they are in ``out``),
    plus the fp8 scale rows or None."""
    row1 = dims.n_ranks * dims.cap if row1 is None else row1
    rb = row_bytes_in(dims)
    if out is not None:
        assert out.dtype == np.uint8 and out.shape == (row1 - row0, rb) and out.flags.c_contiguous
        buf = out
    else:
        buf = np.full((row1 - row0, rb), fill, dtype=np.uint8)
    nsc = dims.hidden // 128 if dims.dtype_in == FP8_E4M3 else 0
    bs = np.zeros((row1 - row0, nsc), np.float32) if nsc else None
    x = np.ascontiguousarray(x)
    assert x.nbytes == dims.n_tokens * rb
    xs = np.ascontiguousarray(x_scale, dtype=np.float32) if nsc else None
    rc = lib().mbref_dispatch_window(ctypes.byref(dims), _ptr(p.pos), _ptr(p.status), _ptr(x),
                                     _ptr(xs) if xs is not None else None, row0, row1,
                                     _ptr(buf), _ptr(bs) if bs is not None else None)
    if rc < 0:
        raise ValueError(f"mbref_dispatch_window returned {rc}")
    return buf, bs, rc


def combine(dims: Dims, pos: np.ndarray, status: np.ndarray, w: np.ndarray, y_exp: np.ndarray,
            t0: int = 0, t1: int | None = None, out: tuple | None = None):
    """(y, mag) in float64 for tokens [t0, t1); y_exp is the [rows, H] expert
    output array in dims.dtype_out (float32, or uint16 bf16 bits). ``out`` may
    supply preallocated (y, mag) arrays."""
    t1 = dims.n_tokens if t1 is None else t1
    H = dims.hidden
    if out is not None:
        y, mag = out
        assert y.shape == (t1 - t0, H) and mag.shape == (t1 - t0, H)
        assert y.dtype == np.float64 and mag.dtype == np.float64
    else:
        y = np.zeros((t1 - t0, H), np.float64)
        mag = np.zeros((t1 - t0, H), np.float64)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    y_exp = np.ascontiguousarray(y_exp)
    rc = lib().mbref_combine(ctypes.byref(dims), _ptr(pos), _ptr(np.ascontiguousarray(status)),
                             _ptr(w), _ptr(y_exp), t0, t1, _ptr(y), _ptr(mag))
    if rc < 0:
        raise ValueError(f"mbref_combine returned {rc}")
    return y, mag, rc


def e4m3_value(b: int) -> float:
    return lib().mbref_e4m3_value(b)


def combine_fp8(dims: Dims, pos: np.ndarray, status: np.ndarray, w: np.ndarray,
                y_exp: np.ndarray, y_scale: np.ndarray, t0: int = 0, t1: int | None = None):
    """(y, mag) in float64 for tokens [t0, t1) from fp8 e4m3 expert outputs
    (uint8 [rows, H]) and their fp32 scales [rows, H/128]."""
    t1 = dims.n_tokens if t1 is None else t1
    H = dims.hidden
    y = np.zeros((t1 - t0, H), np.float64)
    mag = np.zeros((t1 - t0, H), np.float64)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    y_exp = np.ascontiguousarray(y_exp, dtype=np.uint8)
    y_scale = np.ascontiguousarray(y_scale, dtype=np.float32)
    rc = lib().mbref_combine_fp8(ctypes.byref(dims), _ptr(pos), _ptr(np.ascontiguousarray(status)),
                                 _ptr(w), _ptr(y_exp), _ptr(y_scale), t0, t1, _ptr(y), _ptr(mag))
    if rc < 0:
        raise ValueError(f"mbref_combine_fp8 returned {rc}")
    return y, mag, rc
