import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of host work)")


def pytest_sessionstart(session):
    """A fresh checkout has no built library (it is not versioned): build it
    once before the tests that load it, where hipcc is available. The binding
    itself never builds; it refuses to run without the library."""
    lib = os.path.join(ROOT, "cross_layer_shared_amd", "libyoco.so")
    if os.path.exists(lib):
        return
    from cross_layer_shared_amd.build import _hipcc, build
    try:
        _hipcc()
    except RuntimeError:
        return   # no toolchain: the tests that need the library report it missing
    build(verbose=False)


@pytest.fixture(scope="session")
def has_gpu():
    import torch
    return torch.cuda.is_available()


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name every GPU case (flushed) before it touches the device."""
    if request.node.get_closest_marker("gpu") is not None:
        import torch
        if not torch.cuda.is_available():
            pytest.skip("needs a GPU")
        print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    yield
