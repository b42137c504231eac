"""attnres_fwd_noalloc, the entry point that allocates nothing (its split path
exchanges through a static per-device array), against attnres_fwd_strided,
the entry point it mirrors, through the C-ABI binding.

The bar is that of every parity test: out within atol 1e-2 + rtol 1.6e-2 of
the other entry point's output and of the fp64 oracle rounded to bf16; the
written prefix and bank rows and every untouched element bit-exact.  The two
entry points run the same kernels, so their outputs are also compared bit for
bit.  Calls come in pairs, the second with fewer tokens, so that the second
reuses the array the first left behind.
"""
import numpy as np
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


def _call(G, d, noalloc, path=None, stream=None):
    """The call through attnres_fwd_noalloc (the binding), or through the
    C function attnres_fwd_strided with the same marshalled arguments."""
    from kimi_k3_attention_amd import attnres as A
    c = d.case
    args = (d.prefix, d.delta, d.bank3, c.nb, d.res_w, d.rms_w, c.eps, d.onw, c.oeps, c.widx,
            d.out)
    if noalloc:
        A.attnres_fwd_noalloc(*args, stream=stream, path=path)
        return
    m = A._marshal(*args)
    s = stream if stream is not None else torch.cuda.current_stream()
    rc = A.lib().attnres_fwd_strided(*A._strided_args(m), s.cuda_stream,
                                     A.ATTNRES_PATH_AUTO if path is None else int(path))
    if rc != A.ATTNRES_OK:
        raise A.AttnResError(rc, "attnres_fwd_strided")


def _both(G, case, path):
    """The call through both entry points on the same inputs; each checked
    against the oracle, and the two against each other."""
    inp = W.make_inputs(case)
    ref = G.oracle_full(inp)
    got = []
    for noalloc in (False, True):
        G.say(case.name, "noalloc" if noalloc else "strided", "path", path)
        d = G.upload(inp)
        _call(G, d, noalloc, path=path)
        r = G.download(d)
        G.check_full(inp, r, ref)
        got.append(r)
    a, b = got
    G.assert_out_close(b.out, a.out, case.name + " noalloc against the allocating entry point")
    assert (a.out == b.out).all(), case.name + ": the two entry points' outputs differ in bits"
    assert (a.prefix == b.prefix).all() and (a.bank == b.bank).all()


# (first call, second call with fewer tokens), each through both entry points.
PAIRS = [
    (dict(T=40, nb=8, widx=7), dict(T=5, nb=4, widx=-1)),
    (dict(T=200, nb=6, has_onorm=False, widx=2), dict(T=1, nb=1, has_delta=False)),
    (dict(T=16, nb=0), dict(T=3, nb=8, widx=0)),
]


@pytest.mark.parametrize("first,second", PAIRS,
                         ids=[f"T{a['T']}nb{a['nb']}-T{b['T']}nb{b['nb']}" for a, b in PAIRS])
@pytest.mark.parametrize("path_name", ["split", "auto"])
def test_noalloc_matches_allocating_entry_point(G, first, second, path_name):
    from kimi_k3_attention_amd import attnres as A
    path = A.ATTNRES_PATH_SPLIT if path_name == "split" else None
    for k, kw in enumerate((first, second)):
        case = W.Case(f"noalloc_{path_name}_{k}_T{kw['T']}_nb{kw['nb']}", seed=40 + k, **kw)
        _both(G, case, path)
    assert A.attnres_device_status() == A.ATTNRES_OK


def test_noalloc_other_hidden_size_and_row_path(G):
    from kimi_k3_attention_amd import attnres as A
    for k, (kw, path) in enumerate(((dict(T=24, nb=5, H=12288, widx=4), A.ATTNRES_PATH_SPLIT),
                                    (dict(T=9, nb=3, H=2992), A.ATTNRES_PATH_SPLIT),
                                    (dict(T=300, nb=8, widx=3), A.ATTNRES_PATH_ROW),
                                    # the row kernel's small-call (range-checked) form
                                    (dict(T=100, nb=4, widx=2), A.ATTNRES_PATH_ROW),
                                    # any-H kernel with three bank rows staged in LDS
                                    (dict(T=300, nb=6, H=12288, widx=5), A.ATTNRES_PATH_ANY_H),
                                    (dict(T=800, nb=8, H=5120, widx=3), A.ATTNRES_PATH_ANY_H))):
        _both(G, W.Case(f"noalloc_misc_{k}", seed=60 + k, **kw), path)


def test_noalloc_rejects_beyond_its_array(G):
    """A split-path call of more tokens than the static array holds is refused
    before any GPU work, and touches nothing."""
    from kimi_k3_attention_amd import attnres as A
    case = W.Case("noalloc_too_many", T=A.ATTNRES_SPLIT_MAX_TOKENS + 1, nb=2, widx=1, seed=70)
    inp = W.make_inputs(case)
    d = G.upload(inp)
    with pytest.raises(A.AttnResError) as e:
        _call(G, d, True, path=A.ATTNRES_PATH_SPLIT)
    assert e.value.name == "ATTNRES_E_UNSUPPORTED"
    r = G.download(d)
    assert (r.out == inp.out_init).all() and (r.prefix == inp.prefix).all()
    assert (r.bank == inp.bank).all()


def test_noalloc_in_a_captured_graph(G):
    """Captured into a hipGraph after attnres_init (no allocation and no
    memset node in the capture): every replay, with eager work and
    synchronisations between replays, matches the eager call."""
    from kimi_k3_attention_amd import attnres as A
    A.attnres_init()
    case = W.Case("noalloc_graph", T=12, nb=8, widx=-1, seed=80)
    inp = W.make_inputs(case)
    d = G.upload(inp)
    d.delta.zero_()  # replays of the in-place call then stay a fixed point
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _call(G, d, True, path=A.ATTNRES_PATH_SPLIT, stream=s)
    torch.cuda.synchronize()
    eager = G.download(d)
    zero_delta = W.Inputs(**{**inp.__dict__, "delta": np.zeros_like(inp.delta)})
    G.check_full(zero_delta, eager, G.oracle_full(zero_delta))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(G, d, True, path=A.ATTNRES_PATH_SPLIT, stream=torch.cuda.current_stream())
    for rep in range(4):
        d.out.fill_(0x7F81)
        g.replay()
        torch.cuda.synchronize()
        _ = (d.prefix.float().sum() + 1).item()  # unrelated eager work between replays
        r = G.download(d)
        assert (r.out == eager.out).all(), f"replay {rep} differs from the eager call"
        assert (r.prefix == eager.prefix).all() and (r.bank == eager.bank).all()
    del g
    assert A.attnres_device_status() == A.ATTNRES_OK
