"""The Python binding refuses, before any C call, tensors the kernels cannot
take: host tensors (a host pointer handed to a kernel would fault the GPU),
and too few rank speeds. These checks run on the CPU; the layout, dtype and
size checks on GPU tensors are in test_gpu_binding.py."""
from __future__ import annotations

import pytest
import torch

import token_dispatch_mb_amd as mb


def _dims():
    return mb.Dims.make(64, 2, 16, 4, 1, 128, dtype_in="bf16", dtype_out="bf16")


def _host_bufs(d):
    z = lambda *s: torch.zeros(s, dtype=torch.int32)  # noqa: E731
    ns = d.n_slots
    return mb.PlanBuffers(counts=z(4, 16), load_pre=z(4), load_post=z(4), rep_expert=z(4, 1),
                          slot_quota=z(4, ns), cu_seqlens=z(4, ns + 1), pos=z(64, 2),
                          row_src=z(d.rows), status=z(4))


def test_host_ids_are_refused():
    d = _dims()
    ids = torch.zeros(64, 2, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        mb.plan(d, ids, torch.zeros(16, dtype=torch.uint8), _host_bufs(d))


def test_non_tensors_and_host_tensors_are_refused_first():
    with pytest.raises(TypeError, match="torch.Tensor"):
        mb._check([1, 2, 3], "ids")
    # the device is checked before layout and dtype
    with pytest.raises(ValueError, match="GPU tensor"):
        mb._check(torch.zeros(2, 64, dtype=torch.int64).t(), "ids", torch.int32)


def test_host_plan_buffers_are_refused():
    d = _dims()
    with pytest.raises(ValueError, match="GPU tensor"):
        _host_bufs(d).check(d)


def test_too_few_speeds_are_refused():
    d = _dims()
    with pytest.raises(ValueError, match="speeds lists 3 ranks, 4 needed"):
        mb._speeds(d, [1, 1, 1])
    sp = mb._speeds(d, [1, 2, 3, 4, 5])
    assert list(sp) == [1, 2, 3, 4]


def test_host_rows_are_refused():
    d = _dims()
    x = torch.zeros(64, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        mb.dispatch(d, _host_bufs(d), x, torch.zeros(d.rows, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU tensor"):
        mb.combine(d, _host_bufs(d), torch.zeros(d.rows, 128, dtype=torch.bfloat16),
                   torch.zeros(64, 2), x)


def test_tensors_on_another_device_than_the_stream_are_refused():
    class _Stream:  # stands in for a torch stream on GPU 1
        device = torch.device("cuda", 1)
        cuda_stream = 0

    with pytest.raises(ValueError, match="the stream on cuda:1"):
        mb._stream(_Stream(), torch.zeros(4))
    assert mb._stream(_Stream(), None).value is None
