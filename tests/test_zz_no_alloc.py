"""mb_plan_noalloc (the plan on the library's own per-GPU workspace) against
mb_plan on a caller workspace: two calls in a row, the second smaller, every
plan output bit for bit; sizes beyond the held workspace are refused."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import token_dispatch_mb_amd as mb
import workload as W

from . import gpu_harness as G

PLAN_FIELDS = ("counts", "load_pre", "load_post", "rep_expert", "slot_quota", "cu_seqlens",
               "pos", "row_src", "status")


def _outputs(bufs: mb.PlanBuffers) -> dict:
    torch.cuda.synchronize()
    return {n: getattr(bufs, n).cpu().numpy().copy() for n in PLAN_FIELDS}


def _plan_both(wl, dev):
    dims = mb.Dims.for_workload(wl)
    assert mb.workspace_bytes(dims) <= mb.NOALLOC_WS_BYTES
    ids, _ = W.routing_for(wl)
    ids_d = torch.from_numpy(ids).to(dev)
    ref = mb.PlanBuffers.allocate(dims, dev)
    mb.plan(dims, ids_d, mb.alloc_workspace(dims, dev), ref)
    got = mb.PlanBuffers.allocate(dims, dev)
    for b in (got,):
        for n in PLAN_FIELDS:
            getattr(b, n).fill_(-7)  # stale values must not survive
    mb.plan_noalloc(dims, ids_d, got)
    return _outputs(got), _outputs(ref)


@pytest.mark.gpu
def test_noalloc_matches_mb_plan_two_calls():
    dev = G.dev()
    for name in ("dsv3_prefill", "decode_drift"):  # the second call is the smaller one
        got, ref = _plan_both(W.get_workload(name), dev)
        for n in PLAN_FIELDS:
            assert np.array_equal(got[n], ref[n]), (name, n)
        assert got["status"][0] & mb.ST_FATAL == 0, got["status"]


@pytest.mark.gpu
def test_noalloc_refuses_sizes_beyond_its_workspace():
    dev = G.dev()
    dims = mb.Dims.make(1 << 20, 8, 1024, 64, 1, 128)
    assert mb.workspace_bytes(dims) > mb.NOALLOC_WS_BYTES
    ids = torch.zeros((1, 1), dtype=torch.int32, device=dev)
    bufs = mb.PlanBuffers.allocate(mb.Dims.make(64, 2, 16, 4, 1, 128), dev)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = mb.raw_call("mb_plan_noalloc", ctypes.byref(dims), ctypes.c_void_p(ids.data_ptr()),
                     ctypes.byref(bufs.c_struct()), st)
    assert rc == mb.ERR_WORKSPACE
