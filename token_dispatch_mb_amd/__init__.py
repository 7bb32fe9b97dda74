"""Python binding of libmoebal (include/moebal.h).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of plan / dispatch / combine runs in the HIP
kernels of ``libmoebal.so``. There is no fallback: importing this package
fails if the library is not built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoebal.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
DTYPES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}
TORCH_DTYPES = {F32: torch.float32, BF16: torch.bfloat16, FP8_E4M3: torch.uint8}
ELT_BYTES = {F32: 4, BF16: 2, FP8_E4M3: 1}

OK, ERR_INVALID_ARG, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3
ST_BAD_ID, ST_DUP_ID, ST_UNBALANCED, ST_CAPACITY = 1, 2, 4, 8
ST_FATAL = ST_BAD_ID | ST_DUP_ID | ST_CAPACITY

MAX_RANKS, MAX_EXPERTS, MAX_TOPK, MAX_SLOTS = 64, 1024, 32, 16

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; build it with `python -c 'import __graft_entry__ as g; g.build()'`"
    )
_lib = ctypes.CDLL(LIB_PATH)


class Dims(ctypes.Structure):
    """mb_dims."""

    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_tokens", "top_k", "n_experts", "n_ranks", "slots_per_rank", "hidden", "cap",
        "dtype_in", "dtype_out")]

    @classmethod
    def make(cls, n_tokens, top_k, n_experts, n_ranks, slots_per_rank, hidden, cap=None,
             dtype_in="bf16", dtype_out="bf16") -> "Dims":
        if cap is None:
            cap = (n_tokens // n_ranks) * top_k if n_ranks else 0
        di = DTYPES[dtype_in] if isinstance(dtype_in, str) else dtype_in
        do = DTYPES[dtype_out] if isinstance(dtype_out, str) else dtype_out
        return cls(n_tokens, top_k, n_experts, n_ranks, slots_per_rank, hidden, max(cap, 1), di, do)

    @classmethod
    def for_workload(cls, wl, cap=None, n_tokens=None) -> "Dims":
        n = wl.n_tokens if n_tokens is None else n_tokens
        if cap is None and n_tokens is None:
            cap = wl.cap
        return cls.make(n, wl.top_k, wl.n_experts, wl.n_ranks, wl.slots_per_rank, wl.hidden,
                        cap=cap, dtype_in=wl.dtype_in, dtype_out=wl.dtype_out)

    @property
    def eh(self) -> int:
        return self.n_experts // self.n_ranks

    @property
    def n_slots(self) -> int:
        return self.eh + self.slots_per_rank

    @property
    def rows(self) -> int:
        return self.n_ranks * self.cap


_i32p = ctypes.POINTER(ctypes.c_int32)


class _PlanBufsC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "counts", "load_pre", "load_post", "rep_expert", "slot_quota", "cu_seqlens", "pos",
        "row_src", "status")]


_vp = ctypes.c_void_p
_lib.mb_version.restype = ctypes.c_int
_lib.mb_strerror.argtypes = [ctypes.c_int]
_lib.mb_strerror.restype = ctypes.c_char_p
_lib.mb_plan_workspace_bytes.argtypes = [ctypes.POINTER(Dims)]
_lib.mb_plan_workspace_bytes.restype = ctypes.c_size_t
_lib.mb_plan.argtypes = [ctypes.POINTER(Dims), _vp, _vp, ctypes.c_size_t,
                         ctypes.POINTER(_PlanBufsC), _vp]
_lib.mb_plan.restype = ctypes.c_int
_lib.mb_plan_noalloc.argtypes = [ctypes.POINTER(Dims), _vp, ctypes.POINTER(_PlanBufsC), _vp]
_lib.mb_plan_noalloc.restype = ctypes.c_int
_lib.mb_plan_weighted.argtypes = [ctypes.POINTER(Dims), _vp, _i32p, _vp, ctypes.c_size_t,
                                  ctypes.POINTER(_PlanBufsC), _vp]
_lib.mb_plan_weighted.restype = ctypes.c_int


class DriftParams(ctypes.Structure):
    """mb_drift_params: replan when d > delta_num / delta_den, checked every
    check_every calls, reference of up to `window` calls; a kept placement
    replayed above cap or (tol_den > 0) above (1 + tol_num / tol_den) times a
    target replans in the same call. tol_num = tol_den = 0 (the default)
    guards cap only."""
    _fields_ = [(n, ctypes.c_int32) for n in ("delta_num", "delta_den", "window", "check_every",
                                             "tol_num", "tol_den")]


class _PlanOptionsC(ctypes.Structure):
    _fields_ = [("rank_speed", _i32p), ("drift", ctypes.POINTER(DriftParams)),
                ("drift_state", _vp), ("quota_repair", ctypes.c_int32)]


_lib.mb_plan_ex.argtypes = [ctypes.POINTER(Dims), _vp, ctypes.POINTER(_PlanOptionsC), _vp,
                            ctypes.c_size_t, ctypes.POINTER(_PlanBufsC), _vp]
_lib.mb_plan_ex.restype = ctypes.c_int
_lib.mb_drift_state_bytes.argtypes = [ctypes.POINTER(Dims)]
_lib.mb_drift_state_bytes.restype = ctypes.c_size_t
_lib.mb_plan_drift.argtypes = [ctypes.POINTER(Dims), _vp, _i32p, ctypes.POINTER(DriftParams), _vp,
                               _vp, ctypes.c_size_t, ctypes.POINTER(_PlanBufsC), _vp]
_lib.mb_plan_drift.restype = ctypes.c_int
_lib.mb_dispatch.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(_PlanBufsC), _vp, _vp, _vp,
                             _vp, _vp]
_lib.mb_dispatch.restype = ctypes.c_int
_lib.mb_combine.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(_PlanBufsC), _vp, _vp, _vp, _vp]
_lib.mb_combine.restype = ctypes.c_int
_lib.mb_combine_fp8.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(_PlanBufsC), _vp, _vp, _vp,
                                _vp, _vp]
_lib.mb_combine_fp8.restype = ctypes.c_int
_lib.mb_plan_status.argtypes = [ctypes.POINTER(_PlanBufsC), _vp, _i32p]
_lib.mb_plan_status.restype = ctypes.c_int

EXPORTS = ("mb_version", "mb_strerror", "mb_plan_workspace_bytes", "mb_plan",
           "mb_plan_noalloc", "mb_plan_weighted", "mb_drift_state_bytes", "mb_plan_drift", "mb_plan_ex",
           "mb_dispatch", "mb_combine", "mb_combine_fp8", "mb_plan_status")
ST_REPLANNED = 16
ST_GUARDED = 32
NOALLOC_WS_BYTES = 4 << 20
MAX_WINDOW = 4096
MAX_SPEED = 1 << 20


class MoebalError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {code} ({strerror(code)})")
        self.code = code


def version() -> int:
    return _lib.mb_version()


def strerror(code: int) -> str:
    return _lib.mb_strerror(code).decode()


def workspace_bytes(dims: Dims) -> int:
    return int(_lib.mb_plan_workspace_bytes(ctypes.byref(dims)))


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name: str, dtype=None, numel: int | None = None, nbytes: int | None = None) -> None:
    """Refuse, before any C call, what the kernels cannot take: a tensor off
    the GPU (a host pointer would fault the device), a strided view, a wrong
    dtype or too few elements / bytes."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (it is on {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (it is {t.dtype})")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {numel} needed")
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, {nbytes} needed")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _speeds(dims: "Dims", speeds):
    if len(speeds) < dims.n_ranks:
        raise ValueError(f"speeds lists {len(speeds)} ranks, {dims.n_ranks} needed")
    return (ctypes.c_int32 * dims.n_ranks)(*[int(v) for v in speeds[: dims.n_ranks]])


def _dims_key(dims: "Dims") -> tuple:
    return tuple(getattr(dims, n) for n, _ in Dims._fields_)


def _stream(stream, *tensors) -> ctypes.c_void_p:
    """The stream's HIP handle (torch's current stream by default), after
    checking that the given tensors live on the stream's GPU (a pointer into
    another GPU's memory would fault in the kernel)."""
    if stream is None:
        stream = torch.cuda.current_stream()
    dev = stream.device
    for t in tensors:
        if t is not None and t.device != dev:
            raise ValueError(f"a tensor is on {t.device}, the stream on {dev}")
    return ctypes.c_void_p(stream.cuda_stream)


@dataclass
class PlanBuffers:
    """Caller-owned device outputs of mb_plan (torch int32 tensors)."""

    counts: torch.Tensor
    load_pre: torch.Tensor
    load_post: torch.Tensor
    rep_expert: torch.Tensor
    slot_quota: torch.Tensor
    cu_seqlens: torch.Tensor
    pos: torch.Tensor
    row_src: torch.Tensor
    status: torch.Tensor
    _key: tuple | None = field(default=None, init=False, repr=False, compare=False)
    _c: _PlanBufsC | None = field(default=None, init=False, repr=False, compare=False)

    @classmethod
    def allocate(cls, dims: Dims, device) -> "PlanBuffers":
        P, E, R, N, K = dims.n_ranks, dims.n_experts, dims.slots_per_rank, dims.n_tokens, dims.top_k
        ns = dims.n_slots
        z = lambda *s: torch.empty(s, dtype=torch.int32, device=device)  # noqa: E731
        return cls(counts=z(P, E), load_pre=z(P), load_post=z(P), rep_expert=z(P, max(R, 1)),
                   slot_quota=z(P, ns), cu_seqlens=z(P, ns + 1), pos=z(N, K),
                   row_src=z(dims.rows), status=z(4))

    def check(self, dims: Dims) -> None:
        """Every buffer an int32 GPU tensor with room for its output."""
        P, E, R, N, K, ns = (dims.n_ranks, dims.n_experts, dims.slots_per_rank, dims.n_tokens,
                             dims.top_k, dims.n_slots)
        need = {"counts": P * E, "load_pre": P, "load_post": P, "rep_expert": P * R,
                "slot_quota": P * ns, "cu_seqlens": P * (ns + 1), "pos": N * K,
                "row_src": dims.rows, "status": 4}
        for name, n in need.items():
            _check(getattr(self, name), name, torch.int32, numel=n)
            if getattr(self, name).device != self.status.device:
                raise ValueError(f"{name} is on another GPU than status")

    def c_struct(self, dims: Dims | None = None) -> _PlanBufsC:
        """The mb_plan_bufs of these tensors; with `dims`, checked against
        them first (once per set of pointers and sizes)."""
        ts = [getattr(self, n) for n, _ in _PlanBufsC._fields_]
        ptrs = tuple(t.data_ptr() for t in ts)
        if dims is None:
            return self._c if self._key is not None and self._key[0] == ptrs else _PlanBufsC(*ptrs)
        # the key holds the sizes too: a smaller tensor at the same address
        # is checked again
        key = (ptrs, _dims_key(dims), tuple(t.numel() for t in ts),
               tuple(t.is_contiguous() for t in ts))
        if key != self._key:
            self.check(dims)
            self._c, self._key = _PlanBufsC(*ptrs), key
        return self._c


def alloc_workspace(dims: Dims, device) -> torch.Tensor:
    n = workspace_bytes(dims)
    if n == 0:
        raise MoebalError("mb_plan_workspace_bytes", ERR_INVALID_ARG)
    return torch.empty(n, dtype=torch.uint8, device=device)


def plan(dims: Dims, ids: torch.Tensor, ws: torch.Tensor, bufs: PlanBuffers, stream=None,
         speeds=None, drift=None, repair: bool = False) -> None:
    """mb_plan: enqueue the plan of one MoE layer call on `stream`; with
    ``speeds`` (P host ints), mb_plan_weighted; with ``drift`` =
    (DriftParams, state tensor), mb_plan_drift; with ``repair``, mb_plan_ex
    (any of the three options)."""
    _check(ids, "ids", torch.int32, numel=dims.n_tokens * dims.top_k)
    _check(ws, "ws")
    cb = bufs.c_struct(dims)
    sp = None if speeds is None else _speeds(dims, speeds)
    if drift is not None:
        prm, state = drift
        _check(state, "drift state", nbytes=int(_lib.mb_drift_state_bytes(ctypes.byref(dims))))
    st = _stream(stream, ids, ws, bufs.status, drift[1] if drift is not None else None)
    if repair:
        opt = _PlanOptionsC(ctypes.cast(sp, _i32p) if sp is not None else None,
                            ctypes.pointer(drift[0]) if drift else None,
                            _ptr(drift[1]) if drift else None, 1)
        rc = _lib.mb_plan_ex(ctypes.byref(dims), _ptr(ids), ctypes.byref(opt), _ptr(ws),
                             _nbytes(ws), ctypes.byref(cb), st)
        if rc != OK:
            raise MoebalError("mb_plan_ex", rc)
        return
    if drift is not None:
        rc = _lib.mb_plan_drift(ctypes.byref(dims), _ptr(ids), sp, ctypes.byref(prm), _ptr(state),
                                _ptr(ws), _nbytes(ws), ctypes.byref(cb), st)
        if rc != OK:
            raise MoebalError("mb_plan_drift", rc)
        return
    if sp is None:
        rc = _lib.mb_plan(ctypes.byref(dims), _ptr(ids), _ptr(ws), _nbytes(ws), ctypes.byref(cb), st)
        if rc != OK:
            raise MoebalError("mb_plan", rc)
        return
    rc = _lib.mb_plan_weighted(ctypes.byref(dims), _ptr(ids), sp, _ptr(ws), _nbytes(ws),
                               ctypes.byref(cb), st)
    if rc != OK:
        raise MoebalError("mb_plan_weighted", rc)


def plan_noalloc(dims: Dims, ids: torch.Tensor, bufs: PlanBuffers, stream=None) -> None:
    """mb_plan_noalloc: mb_plan with the library's own per-GPU workspace (no
    workspace argument; calls on one GPU must not overlap in time)."""
    _check(ids, "ids", torch.int32, numel=dims.n_tokens * dims.top_k)
    cb = bufs.c_struct(dims)
    rc = _lib.mb_plan_noalloc(ctypes.byref(dims), _ptr(ids), ctypes.byref(cb),
                              _stream(stream, ids, bufs.status))
    if rc != OK:
        raise MoebalError("mb_plan_noalloc", rc)


def dispatch(dims: Dims, bufs: PlanBuffers, x: torch.Tensor, buf: torch.Tensor,
             x_scale: torch.Tensor | None = None, buf_scale: torch.Tensor | None = None,
             stream=None) -> None:
    """mb_dispatch: buf[pos[t][k]] = x[t] (and the fp8 scale rows)."""
    row = dims.hidden * ELT_BYTES.get(dims.dtype_in, 0)
    _check(x, "x", nbytes=dims.n_tokens * row)
    _check(buf, "buf", nbytes=dims.rows * row)
    if dims.dtype_in == FP8_E4M3:
        _check(x_scale, "x_scale", torch.float32, numel=dims.n_tokens * (dims.hidden // 128))
        _check(buf_scale, "buf_scale", torch.float32, numel=dims.rows * (dims.hidden // 128))
    rc = _lib.mb_dispatch(ctypes.byref(dims), ctypes.byref(bufs.c_struct(dims)), _ptr(x),
                          _ptr(x_scale), _ptr(buf), _ptr(buf_scale),
                          _stream(stream, x, buf, x_scale, buf_scale, bufs.status))
    if rc != OK:
        raise MoebalError("mb_dispatch", rc)


def combine(dims: Dims, bufs: PlanBuffers, y_exp: torch.Tensor, w: torch.Tensor, y: torch.Tensor,
            stream=None) -> None:
    """mb_combine: y[t] = sum_k w[t][k] * y_exp[pos[t][k]] (fp32 accumulation)."""
    row = dims.hidden * ELT_BYTES.get(dims.dtype_out, 0)
    _check(y_exp, "y_exp", nbytes=dims.rows * row)
    _check(w, "w", torch.float32, numel=dims.n_tokens * dims.top_k)
    _check(y, "y", nbytes=dims.n_tokens * row)
    rc = _lib.mb_combine(ctypes.byref(dims), ctypes.byref(bufs.c_struct(dims)), _ptr(y_exp), _ptr(w),
                         _ptr(y), _stream(stream, y_exp, w, y, bufs.status))
    if rc != OK:
        raise MoebalError("mb_combine", rc)


def alloc_drift_state(dims: Dims, device) -> torch.Tensor:
    """A zero-filled (fresh) drift state buffer for one layer."""
    n = _lib.mb_drift_state_bytes(ctypes.byref(dims))
    if n == 0:
        raise MoebalError("mb_drift_state_bytes", ERR_INVALID_ARG)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def drift_header(state: torch.Tensor) -> dict:
    """The mb_drift_header fields of a state buffer (copies to the host)."""
    import numpy as np

    b = state[:64].cpu().numpy().tobytes()
    i32 = np.frombuffer(b[:16], np.int32)
    i64 = np.frombuffer(b[16:32], np.int64)
    return {"have_plan": int(i32[0]), "countdown": int(i32[1]), "nwin": int(i32[2]),
            "n_moves": int(i32[3]), "calls": int(i64[0]), "replans": int(i64[1]),
            "last_d": float(np.frombuffer(b[32:40], np.float64)[0]),
            "guarded": int(np.frombuffer(b[40:48], np.int64)[0])}


def combine_fp8(dims: Dims, bufs: PlanBuffers, y_exp: torch.Tensor, y_scale: torch.Tensor,
                w: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    """mb_combine_fp8: y[t] = sum_k w[t][k] * dequant(y_exp[pos[t][k]]) from
    fp8 e4m3 rows (uint8 [rows, H]) and fp32 scales [rows, H/128]."""
    _check(y_exp, "y_exp", torch.uint8, numel=dims.rows * dims.hidden)
    _check(y_scale, "y_scale", torch.float32, numel=dims.rows * (dims.hidden // 128))
    _check(w, "w", torch.float32, numel=dims.n_tokens * dims.top_k)
    _check(y, "y", nbytes=dims.n_tokens * dims.hidden * ELT_BYTES.get(dims.dtype_out, 0))
    rc = _lib.mb_combine_fp8(ctypes.byref(dims), ctypes.byref(bufs.c_struct(dims)), _ptr(y_exp),
                             _ptr(y_scale), _ptr(w), _ptr(y),
                             _stream(stream, y_exp, y_scale, w, y, bufs.status))
    if rc != OK:
        raise MoebalError("mb_combine_fp8", rc)


def plan_status(bufs: PlanBuffers, stream=None):
    """mb_plan_status: [flags, T, max load, moves] on the host (synchronises)."""
    import numpy as np

    _check(bufs.status, "status", torch.int32, numel=4)
    out = (ctypes.c_int32 * 4)()
    rc = _lib.mb_plan_status(ctypes.byref(bufs.c_struct()), _stream(stream, bufs.status), out)
    if rc != OK:
        raise MoebalError("mb_plan_status", rc)
    return np.array(list(out), dtype=np.int32)


def raw_call(fn: str, *args) -> int:
    """Call an exported mb_* function with raw ctypes arguments (for tests of
    the argument checks)."""
    return getattr(_lib, fn)(*args)
