"""The split path's two workspace frames.  Every workgroup writes its
exchange words into one frame (by default the one the set-up timing found
nearer its XCD) and reads both, so which frame a workgroup writes may change
speed but never results.  Split-path calls are made under every choice,
including the parts of one token writing different frames, and with the
choice changing from call to call (a part's generation then advances in
either frame).  Each must match the oracle and be bit-identical to the
default choice, and the library's status must stay clean."""
import numpy as np
import pytest
import torch

from kimi_k3_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

# -1: the default; masks by XCD; 256: odd parts write frame B, even ones A.
MODES = [-1, 0, 255, 0x0F, 0xF0, 256, -1, 256, 0x55, 0, -1]

CASES = [
    dict(T=1, nb=8, widx=-1),                                   # Gram product words
    dict(T=1, nb=1, widx=-1),                                   # wave-sum words
    dict(T=5, nb=4, widx=3),                                    # transposed words
    dict(T=16, nb=8, widx=7, has_delta=False),
    dict(T=2, nb=0, widx=0, cap=2),                             # one source: word 0 alone
    dict(T=3, nb=6, widx=-1, has_onorm=False),
    dict(T=1, nb=4, H=9216, widx=-1),                           # wide split, masked
]


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_harness
    return gpu_harness


def _run_modes(G, A, inp, ref):
    first = None
    try:
        for m in MODES:
            G.say(inp.case.name, "frames mode", m)
            A.attnres_debug_workspace_frames(m)
            d = G.upload(inp)
            G.run(d, path=A.ATTNRES_PATH_SPLIT)
            got = G.download(d)
            G.check_full(inp, got, ref)
            if first is None:
                first = got
            else:
                assert np.array_equal(got.out, first.out), f"{inp.case.name}: mode {m} out"
    finally:
        A.attnres_debug_workspace_frames(-1)
    assert A.attnres_device_status() == A.ATTNRES_OK


@pytest.mark.parametrize("k", range(len(CASES)))
def test_results_do_not_depend_on_the_frame_written(G, k):
    from kimi_k3_attention_amd import attnres as A
    case = W.Case(f"frames_{k}", seed=60 + k, **CASES[k])
    inp = W.make_inputs(case)
    _run_modes(G, A, inp, G.oracle_full(inp))


def test_second_exchange_under_every_frame_choice(G):
    """Sources that cancel make the split path exchange ||y||^2 directly in a
    second round (as in the parity tests' cancelling case); that round's words
    go through the two frames too."""
    from kimi_k3_attention_amd import attnres as A
    case = W.Case("frames_cancel", T=4, nb=2, cap=2, widx=-1, seed=91)
    inp = W.make_inputs(case)
    inp.res_w[:] = 0
    H, ts = case.H, case.token_stride
    for t in range(case.T):
        inp.bank[t * ts + H: t * ts + 2 * H] = inp.bank[t * ts: t * ts + H] ^ np.uint16(0x8000)
    small = (G.widen(inp.prefix) * 0.01).astype(np.float32)
    inp.prefix[:] = torch.from_numpy(small).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    _run_modes(G, A, inp, G.oracle_full(inp))


def test_rejects_unknown_modes(G):
    from kimi_k3_attention_amd import attnres as A
    for m in (-2, 257):
        with pytest.raises(A.AttnResError):
            A.attnres_debug_workspace_frames(m)
