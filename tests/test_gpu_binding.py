"""On the GPU: the binding's layout, dtype and size checks raise before launching
anything, and the plan buffers are checked once per set of pointers."""
from __future__ import annotations

import pytest
import torch

import token_dispatch_mb_amd as mb

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_required():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    yield
    torch.cuda.synchronize()


def test_short_gpu_tensors_are_refused():
    dev = torch.device("cuda:0")
    d = mb.Dims.make(64, 2, 16, 4, 1, 128, dtype_in="bf16", dtype_out="bf16")
    bufs = mb.PlanBuffers.allocate(d, dev)
    ws = mb.alloc_workspace(d, dev)
    ids = torch.zeros(64, 2, dtype=torch.int32, device=dev)
    ids[:, 1] = 1  # every token routes to experts 0 and 1
    with pytest.raises(ValueError, match="ids holds 64 elements, 128 needed"):
        mb.plan(d, ids[:32], ws, bufs)
    with pytest.raises(TypeError, match="ids must be torch.int32"):
        mb.plan(d, ids.long(), ws, bufs)
    with pytest.raises(ValueError, match="ids must be contiguous"):
        mb.plan(d, torch.zeros(2, 64, dtype=torch.int32, device=dev).t(), ws, bufs)
    x = torch.zeros(64, 128, dtype=torch.bfloat16, device=dev)
    buf = torch.zeros(d.rows, 128, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="buf holds"):
        mb.dispatch(d, bufs, x, buf[:-1])
    w = torch.zeros(64, 2, device=dev)
    with pytest.raises(ValueError, match="w holds"):
        mb.combine(d, bufs, buf, w[:10], x)
    short = mb.PlanBuffers.allocate(mb.Dims.make(32, 2, 16, 4, 1, 128), dev)
    with pytest.raises(ValueError, match="pos holds"):
        mb.plan(d, ids, ws, short)
    # the same call with sound arguments runs, and nothing ran before
    mb.plan(d, ids, ws, bufs)
    assert mb.plan_status(bufs)[0] == 0
    assert bufs._key is not None and bufs._key[1] == mb._dims_key(d)


def test_smaller_buffer_at_the_same_address_is_checked_again():
    """The checked-buffer cache keys on sizes as well as addresses: a view of
    the same storage with too few elements is refused, not taken from the
    cache."""
    dev = torch.device("cuda:0")
    d = mb.Dims.make(64, 2, 16, 4, 1, 128, dtype_in="bf16", dtype_out="bf16")
    bufs = mb.PlanBuffers.allocate(d, dev)
    bufs.c_struct(d)  # checked and cached
    bufs.pos = bufs.pos.view(-1)[:10]  # same address, 10 of 128 elements
    with pytest.raises(ValueError, match="pos holds 10 elements, 128 needed"):
        bufs.c_struct(d)
