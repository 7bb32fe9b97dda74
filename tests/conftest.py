"""Shared test setup: repository root on sys.path, the `gpu` marker, and a
one-time build of the C libraries when nothing is built yet."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")
    need = [os.path.join(ROOT, "oracle", "libmbref.so"), os.path.join(ROOT, "workload", "libmbgen.so")]
    if os.path.exists(os.path.join(ROOT, "token_dispatch_mb_amd", "csrc")):
        need.append(os.path.join(ROOT, "token_dispatch_mb_amd", "libmoebal.so"))
    if not all(os.path.exists(p) for p in need):
        import __graft_entry__

        __graft_entry__.build()


@pytest.fixture(scope="session")
def has_gpu():
    import torch

    return torch.cuda.is_available()
