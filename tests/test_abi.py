"""The C ABI of libmoebal without a GPU: every symbol include/moebal.h
declares is exported, and the host-side checks return the documented codes
before anything reaches the device."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import token_dispatch_mb_amd as mb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "moebal.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mb_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert set(names) == set(mb.EXPORTS)
    lib = ctypes.CDLL(mb.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_ceiling_library_exports_its_header():
    """libmoebal_ceiling.so (reference kernels for bench.py --ceiling)
    exports every symbol include/moebal_ceiling.h declares."""
    text = open(os.path.join(ROOT, "include", "moebal_ceiling.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(mbc_[a-z0-9_]+)\s*\(", text)))
    assert names == ["mbc_copy", "mbc_fill", "mbc_gather_xor", "mbc_read", "mbc_row_write",
                     "mbc_scatter_write"]
    lib = ctypes.CDLL(os.path.join(ROOT, "token_dispatch_mb_amd", "libmoebal_ceiling.so"))
    for n in names:
        assert hasattr(lib, n), n


def test_ceiling_library_refuses_bad_arguments_on_the_host():
    """Invalid sizes, alignments and top-K values return -1 before anything
    is launched (so this needs no GPU)."""
    lib = ctypes.CDLL(os.path.join(ROOT, "token_dispatch_mb_amd", "libmoebal_ceiling.so"))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.mbc_fill.argtypes = [vp, i64, vp]
    lib.mbc_copy.argtypes = [vp, vp, i64, vp]
    lib.mbc_read.argtypes = [vp, i64, ctypes.POINTER(ctypes.c_uint32), vp, vp]
    for f in (lib.mbc_scatter_write, lib.mbc_row_write):
        f.argtypes = [vp, vp, i32, i32, i32, i32, vp]
    lib.mbc_gather_xor.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
    a, b = vp(1 << 20), vp((1 << 20) + 8)  # 16-byte aligned / misaligned (never dereferenced)
    key = (ctypes.c_uint32 * 4)(1, 2, 3, 4)
    assert lib.mbc_fill(None, 16, None) == -1
    assert lib.mbc_fill(b, 16, None) == -1
    assert lib.mbc_fill(a, 24, None) == -1
    assert lib.mbc_fill(a, -16, None) == -1
    assert lib.mbc_copy(a, b, 16, None) == -1
    assert lib.mbc_read(a, 16, None, a, None) == -1
    assert lib.mbc_read(a, 16, key, b, None) == -1
    for K in (0, 33, -1):
        assert lib.mbc_scatter_write(a, a, 8, K, 1024, 64, None) == -1
        assert lib.mbc_gather_xor(a, a, a, 8, K, 1024, 64, None) == -1
    assert lib.mbc_row_write(a, a, 8, 17, 1024, 64, None) == -1
    for rb in (0, 8, 1000):
        assert lib.mbc_scatter_write(a, a, 8, 8, rb, 64, None) == -1
        assert lib.mbc_row_write(a, a, 8, 8, rb, 64, None) == -1
    assert lib.mbc_scatter_write(a, b, 8, 8, 1024, 64, None) == -1
    assert lib.mbc_scatter_write(a, a, -1, 8, 1024, 64, None) == -1
    assert lib.mbc_gather_xor(a, a, b, 8, 8, 1024, 64, None) == -1
    # nothing to do: no launch, success
    assert lib.mbc_fill(a, 0, None) == 0
    assert lib.mbc_scatter_write(a, a, 0, 8, 1024, 64, None) == 0


def test_version_and_strerror():
    assert mb.version() == 2
    for code in (mb.OK, mb.ERR_INVALID_ARG, mb.ERR_WORKSPACE, mb.ERR_HIP, mb.ST_BAD_ID,
                 mb.ST_DUP_ID, mb.ST_UNBALANCED, mb.ST_CAPACITY, 12345):
        assert isinstance(mb.strerror(code), str) and mb.strerror(code)


def test_workspace_bytes_host_only():
    d = mb.Dims.make(131072, 8, 256, 32, 1, 7168)
    n = mb.workspace_bytes(d)
    # per-block counts and offsets dominate: 2 * (32 sources * 16 blocks) * 256 experts * 4 B
    assert n >= 2 * 512 * 256 * 4
    assert n % 256 == 0


@pytest.mark.parametrize("args,cap", [
    ((64, 2, 16, 3, 1, 128), 32),      # N % P
    ((64, 2, 15, 4, 1, 128), 32),      # E % P
    ((64, 0, 16, 4, 1, 128), 32),      # K = 0
    ((64, 17, 16, 4, 1, 128), 32),     # K > E
    ((128, 2, 2048, 128, 1, 128), 32), # P > 64
    ((64, 2, 2048, 4, 1, 128), 32),    # E > 1024
    ((64, 2, 16, 4, 17, 128), 32),     # R > 16
    ((64, 2, 16, 4, -1, 128), 32),     # R < 0
    ((64, 2, 16, 4, 1, 128), 0),       # cap = 0
    ((64, 2, 16, 4, 1, 4), 32),        # bf16 row of 8 bytes
    ((1 << 28, 8, 16, 4, 1, 128), 32),  # N * K > INT32_MAX pairs
    # 2^23 tokens of 65536 bf16: 2^30 dispatch waves fit an int32, 2^31 combine waves do not
    ((1 << 23, 1, 4, 1, 1, 65536), 1 << 23),
])
def test_invalid_sizes_rejected_on_host(args, cap):
    d = mb.Dims.make(*args, cap=cap)
    d.cap = cap
    assert mb.workspace_bytes(d) == 0
    fake = ctypes.c_void_p(1 << 20)
    bufs = mb._PlanBufsC(*([1 << 20] * 9))
    rc = mb.raw_call("mb_plan", ctypes.byref(d), fake, fake, 1 << 30, ctypes.byref(bufs), None)
    assert rc == mb.ERR_INVALID_ARG
    rc = mb.raw_call("mb_dispatch", ctypes.byref(d), ctypes.byref(bufs), fake, None, fake, None, None)
    assert rc == mb.ERR_INVALID_ARG
    rc = mb.raw_call("mb_combine", ctypes.byref(d), ctypes.byref(bufs), fake, fake, fake, None)
    assert rc == mb.ERR_INVALID_ARG


def test_fp8_needs_h_multiple_of_128_and_scales():
    d = mb.Dims.make(64, 2, 16, 4, 1, 64, dtype_in="fp8", dtype_out="bf16")
    assert mb.workspace_bytes(d) == 0
    d = mb.Dims.make(64, 2, 16, 4, 1, 128, dtype_in="fp8", dtype_out="bf16")
    assert mb.workspace_bytes(d) > 0
    fake = ctypes.c_void_p(1 << 20)
    bufs = mb._PlanBufsC(*([1 << 20] * 9))
    rc = mb.raw_call("mb_dispatch", ctypes.byref(d), ctypes.byref(bufs), fake, None, fake, None, None)
    assert rc == mb.ERR_INVALID_ARG


def test_small_workspace_and_null_pointers_rejected():
    d = mb.Dims.make(64, 2, 16, 4, 1, 128)
    need = mb.workspace_bytes(d)
    fake = ctypes.c_void_p(1 << 20)
    bufs = mb._PlanBufsC(*([1 << 20] * 9))
    rc = mb.raw_call("mb_plan", ctypes.byref(d), fake, fake, need - 1, ctypes.byref(bufs), None)
    assert rc == mb.ERR_WORKSPACE
    rc = mb.raw_call("mb_plan", ctypes.byref(d), None, fake, need, ctypes.byref(bufs), None)
    assert rc == mb.ERR_INVALID_ARG
    nulls = mb._PlanBufsC(*([1 << 20] * 8 + [0]))
    rc = mb.raw_call("mb_plan", ctypes.byref(d), fake, fake, need, ctypes.byref(nulls), None)
    assert rc == mb.ERR_INVALID_ARG
    mis = ctypes.c_void_p((1 << 20) + 4)
    rc = mb.raw_call("mb_plan", ctypes.byref(d), fake, mis, need, ctypes.byref(bufs), None)
    assert rc == mb.ERR_INVALID_ARG
    rc = mb.raw_call("mb_dispatch", ctypes.byref(d), ctypes.byref(bufs), mis, None, fake, None, None)
    assert rc == mb.ERR_INVALID_ARG
    rc = mb.raw_call("mb_plan_status", None, None, None)
    assert rc == mb.ERR_INVALID_ARG


def test_weighted_plan_speed_checks():
    """mb_plan_weighted rejects a missing or out-of-range speed array on the
    host; valid speeds get as far as the workspace check."""
    d = mb.Dims.make(64, 2, 16, 4, 1, 128)
    need = mb.workspace_bytes(d)
    fake = ctypes.c_void_p(1 << 20)
    bufs = mb._PlanBufsC(*([1 << 20] * 9))
    I4 = ctypes.c_int32 * 4
    rc = mb.raw_call("mb_plan_weighted", ctypes.byref(d), fake, None, fake, need,
                     ctypes.byref(bufs), None)
    assert rc == mb.ERR_INVALID_ARG
    for bad in ((0, 1, 1, 1), (1, -3, 1, 1), (1, 1, 1, mb.MAX_SPEED + 1)):
        rc = mb.raw_call("mb_plan_weighted", ctypes.byref(d), fake, I4(*bad), fake, need,
                         ctypes.byref(bufs), None)
        assert rc == mb.ERR_INVALID_ARG, bad
    rc = mb.raw_call("mb_plan_weighted", ctypes.byref(d), fake, I4(3, 1, mb.MAX_SPEED, 2), fake,
                     need - 1, ctypes.byref(bufs), None)
    assert rc == mb.ERR_WORKSPACE


def test_combine_fp8_host_checks():
    """mb_combine_fp8 needs H % 128 == 0, scales, and aligned rows."""
    fake = ctypes.c_void_p(1 << 20)
    bufs = mb._PlanBufsC(*([1 << 20] * 9))
    d = mb.Dims.make(64, 2, 16, 4, 1, 64, dtype_in="fp8", dtype_out="bf16")
    rc = mb.raw_call("mb_combine_fp8", ctypes.byref(d), ctypes.byref(bufs), fake, fake, fake, fake,
                     None)
    assert rc == mb.ERR_INVALID_ARG  # H = 64
    d = mb.Dims.make(64, 2, 16, 4, 1, 128, dtype_in="fp8", dtype_out="bf16")
    rc = mb.raw_call("mb_combine_fp8", ctypes.byref(d), ctypes.byref(bufs), fake, None, fake, fake,
                     None)
    assert rc == mb.ERR_INVALID_ARG  # no scales
    rc = mb.raw_call("mb_combine_fp8", ctypes.byref(d), ctypes.byref(bufs), fake,
                     ctypes.c_void_p((1 << 20) + 2), fake, fake, None)
    assert rc == mb.ERR_INVALID_ARG  # misaligned scales
