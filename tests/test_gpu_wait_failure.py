"""The split path's bounded cross-workgroup wait, made to give up from the
host (attnres_debug_force_wait_failure: the waits look for a generation that
never comes and stop after 64 polls, so every kernel still exits).  The
device flag must then be reported once by attnres_device_status as
ATTNRES_E_DEVICE_WAIT, the workspace reset, and the next calls, with the
waits restored, must match the oracle again.  (Results of the failed calls
are not valid and are not checked.)"""
import pytest
import torch

from kimi_k3_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_harness
    return gpu_harness


def test_forced_wait_failure_is_reported_and_cleared(G):
    from kimi_k3_attention_amd import attnres as A
    case = W.Case("wait_failure", T=3, nb=8, widx=-1, seed=97)   # split path, with a norm
    inp = W.make_inputs(case)
    ref = G.oracle_full(inp)
    assert A.attnres_device_status() == A.ATTNRES_OK
    G.say(case.name, "forced failure")
    try:
        A.attnres_debug_force_wait_failure(True)
        for _ in range(2):
            d = G.upload(inp)
            G.run(d, path=A.ATTNRES_PATH_SPLIT)
        torch.cuda.synchronize()
    finally:
        A.attnres_debug_force_wait_failure(False)
    assert A.attnres_device_status() == A.CODES["ATTNRES_E_DEVICE_WAIT"]
    assert A.attnres_device_status() == A.ATTNRES_OK, "the flag was not cleared"
    G.say(case.name, "after")
    for _ in range(2):
        d = G.upload(inp)
        G.run(d, path=A.ATTNRES_PATH_SPLIT)
        G.check_full(inp, G.download(d), ref)
    assert A.attnres_device_status() == A.ATTNRES_OK
