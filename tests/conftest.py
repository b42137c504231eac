import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session", autouse=True)
def built_libraries():
    """Builds libattnres and the oracle only if they are missing (a stale
    build is the caller's to refresh: build() always recompiles)."""
    from kimi_k3_attention_amd import build as kbuild
    from oracle import build as obuild
    if not os.path.exists(kbuild.LIB):
        kbuild.build()
    obuild.ensure_built()


@pytest.fixture(scope="session")
def oracle_lib(built_libraries):
    from oracle import oracle as o
    return o.load_library()


@pytest.fixture(scope="module", autouse=True)
def split_wait_flag_clear_after_gpu_module(request):
    """A split-path cross-workgroup wait that gives up is reported only by a
    later synchronous attnres_device_status; every GPU test module ends by
    checking that no wait gave up while it ran."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    import torch
    if not torch.cuda.is_available():
        return
    from kimi_k3_attention_amd import attnres as A
    assert A.attnres_device_status() == A.ATTNRES_OK, \
        "a split-path cross-workgroup wait gave up during this module"
