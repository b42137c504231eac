"""The two-kernel form (attnres_fwd_bank, then attnres_fwd_cur) against the
fp64 oracle, through the C-ABI binding, to the bar of every parity test: out
within atol 1e-2 + rtol 1.6e-2 of the oracle rounded to bf16, the written
prefix and bank rows and every untouched element bit-exact.

Also: the bank kernel on a forked branch of a captured hipGraph beside a
producer of delta (a matrix product writing delta), joined before the cur
kernel; every replay matches the one-kernel call on the same inputs.
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


def _partial(T, H):
    from kimi_k3_attention_amd import attnres as A
    n = A.attnres_partial_bytes(T, H)
    # fp32 elements, rounded up; filled with a NaN pattern so that a missing
    # write shows up in the output
    return torch.full((max(1, -(-n // 4)),), float("nan"), dtype=torch.float32, device="cuda")


def _two(G, d, partial, stream=None):
    from kimi_k3_attention_amd import attnres as A
    c = d.case
    args = (d.prefix, d.delta, d.bank3, c.nb, d.res_w, d.rms_w, c.eps, d.onw, c.oeps, c.widx, d.out)
    A.attnres_fwd_bank(*args, partial if c.nb > 0 else None, stream=stream)
    A.attnres_fwd_cur(*args, partial if c.nb > 0 else None, stream=stream)


def _check(G, case):
    inp = W.make_inputs(case)
    ref = G.oracle_full(inp)
    G.say(case.name, "two-kernel form")
    d = G.upload(inp)
    _two(G, d, _partial(case.T, case.H))
    G.check_full(inp, G.download(d), ref)


@pytest.mark.parametrize("case", W.variant_matrix(), ids=lambda c: c.name)
def test_two_kernel_variant_matrix(G, case):
    _check(G, case)


@pytest.mark.parametrize("kw", [
    dict(T=4, nb=4, seed=0),                               # the reference case's shape
    dict(T=300, nb=7, H=5120, widx=2, seed=1),
    dict(T=33, nb=3, H=2888, has_delta=False, seed=2),     # masked rows
    dict(T=20, nb=8, H=12288, widx=7, seed=3),             # four segments per lane
    dict(T=17, nb=1, H=16376, has_onorm=False, seed=4),    # masked, four segments
    dict(T=9, nb=5, recipe="soft", widx=0, seed=5),        # weights that really mix
    dict(T=64, nb=8, recipe="student_t", token_pad=64, seed=6),
    dict(T=12, nb=6, row_pad=24, widx=5, seed=7),          # strided prefix / delta / out
], ids=lambda kw: "_".join(f"{k}{v}" for k, v in kw.items()))
def test_two_kernel_other_shapes(G, kw):
    _check(G, W.Case("two_kernel_" + "_".join(f"{k}{v}" for k, v in kw.items()), **kw))


def test_two_kernel_beside_a_producer_in_a_graph(G):
    """delta is produced (an elementwise kernel: a library matrix product
    would have to be initialised outside capture first) on one branch of a
    captured graph while the bank kernel runs on another; the cur kernel runs
    after both.  Every replay (with eager work and synchronisations between
    replays) matches the one-kernel attnres_fwd after the same producer."""
    from kimi_k3_attention_amd import attnres as A
    case = W.Case("two_kernel_graph", T=16, nb=8, widx=7, seed=9)
    inp = W.make_inputs(case)
    H = case.H
    gen = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn(case.T, H, device="cuda", generator=gen)

    c = case
    d = G.upload(inp)
    prefix0 = d.prefix.clone()
    bank0 = d.bank.clone()
    partial = _partial(case.T, H)
    args = (d.prefix, d.delta, d.bank3, c.nb, d.res_w, d.rms_w, c.eps, d.onw, c.oeps, c.widx, d.out)
    side = torch.cuda.Stream()
    G.say("two-kernel graph: capture")
    g = torch.cuda.CUDAGraph()
    main = torch.cuda.Stream()
    main.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(main):
        with torch.cuda.graph(g, stream=main):
            side.wait_stream(main)
            with torch.cuda.stream(side):
                A.attnres_fwd_bank(*args, partial, stream=side)
            d.delta.copy_((x * 0.75 + 0.125).to(torch.bfloat16).view(torch.int16))
            main.wait_stream(side)
            A.attnres_fwd_cur(*args, partial, stream=main)
    torch.cuda.synchronize()
    G.say("two-kernel graph: captured")
    ref = None
    for rep in range(4):
        G.say("two-kernel graph: replay", rep)
        # the in-place rows back to their pre-call state, the output poisoned
        d.prefix.copy_(prefix0)
        d.bank.copy_(bank0)
        d.out.fill_(0x7F81)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _ = (d.prefix.float().sum() + 1).item()  # unrelated eager work between replays
        got = G.download(d)
        if ref is None:
            # The one-kernel call on the same inputs and the delta the graph produced.
            produced = got.delta.copy()
            assert np.isfinite(G.widen(produced)).all()
            ref_d = G.upload(W.Inputs(**{**inp.__dict__, "delta": produced}))
            A.attnres_fwd(ref_d.prefix, ref_d.delta, ref_d.bank3, c.nb, ref_d.res_w, ref_d.rms_w,
                          c.eps, ref_d.onw, c.oeps, c.widx, ref_d.out)
            ref = G.download(ref_d)
        assert (got.delta == ref.delta).all(), f"replay {rep}: the producer's delta changed"
        G.assert_out_close(got.out, ref.out, f"replay {rep} against the one-kernel call")
        assert (got.prefix == ref.prefix).all(), f"replay {rep}: prefix"
        assert (got.bank == ref.bank).all(), f"replay {rep}: bank"
    del g


def test_two_kernel_rejects_bad_partial_before_any_work(G):
    from kimi_k3_attention_amd import attnres as A
    case = W.Case("two_kernel_bad", T=8, nb=4, widx=1, seed=11)
    inp = W.make_inputs(case)
    d = G.upload(inp)
    c = case
    args = (d.prefix, d.delta, d.bank3, c.nb, d.res_w, d.rms_w, c.eps, d.onw, c.oeps, c.widx, d.out)
    small = torch.zeros(16, dtype=torch.float32, device="cuda")
    for fn in (A.attnres_fwd_bank, A.attnres_fwd_cur):
        with pytest.raises(A.AttnResError) as e:
            fn(*args, None)
        assert e.value.name == "ATTNRES_E_NULL"
        with pytest.raises(A.AttnResError) as e:
            fn(*args, small)
        assert e.value.name == "ATTNRES_E_SHAPE"
    # an output that lies inside the partial buffer
    big = torch.zeros(A.attnres_partial_bytes(c.T, c.H) // 4 + 64, dtype=torch.float32,
                      device="cuda")
    out_inside = big.view(torch.int16)[: c.T * c.H].view(c.T, c.H)
    with pytest.raises(A.AttnResError) as e:
        A.attnres_fwd_bank(d.prefix, d.delta, d.bank3, c.nb, d.res_w, d.rms_w, c.eps, d.onw,
                           c.oeps, c.widx, out_inside, big)
    assert e.value.name == "ATTNRES_E_ALIAS"
    got = G.download(d)
    assert (got.out == inp.out_init).all() and (got.prefix == inp.prefix).all()
    assert (got.bank == inp.bank).all()
