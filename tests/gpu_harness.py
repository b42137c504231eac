"""Moves seeded workloads to the GPU, runs the HIP path through the C-ABI
binding and compares with the oracle.  Test infrastructure."""
from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

from kimi_k3_attention_amd import attnres as A
from kimi_k3_attention_amd import workloads as W

ATOL = 1e-2
RTOL = 1.6e-2


def say(*msg):
    print("[gpu]", *msg, file=sys.stderr, flush=True)


def widen(bits: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_dev(a: Optional[np.ndarray]) -> Optional[torch.Tensor]:
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


def from_dev(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    if t is None:
        return None
    return t.contiguous().cpu().numpy().view(np.uint16)


ROW_GAP_BITS = 0x7F83   # a NaN: fills the gaps between strided rows


@dataclass
class Dev:
    case: W.Case
    prefix: torch.Tensor        # [T, H], row stride case.row_stride
    delta: Optional[torch.Tensor]
    bank: torch.Tensor          # flat
    bank3: torch.Tensor         # [T, cap, H] strided view
    res_w: torch.Tensor
    rms_w: torch.Tensor
    onw: Optional[torch.Tensor]
    out: torch.Tensor
    gaps: dict                  # name -> the full [T, row_stride] buffer of a strided matrix


def _matrix(a: Optional[np.ndarray], c: W.Case, name: str, gaps: dict):
    """A [T, H] matrix on the device: dense, or rows case.row_stride apart with
    the gaps filled by ROW_GAP_BITS."""
    if a is None:
        return None
    if c.row_pad == 0:
        return to_dev(a)
    full = torch.full((c.T, c.row_stride), ROW_GAP_BITS, dtype=torch.int16, device="cuda")
    view = full[:, :c.H]
    view.copy_(to_dev(a))
    gaps[name] = full
    return view


def upload(inp: W.Inputs) -> Dev:
    c = inp.case
    bank = to_dev(inp.bank)
    bank3 = bank.as_strided((c.T, c.cap, c.H), (c.token_stride, c.slot_stride, 1))
    gaps = {}
    return Dev(c, _matrix(inp.prefix, c, "prefix", gaps), _matrix(inp.delta, c, "delta", gaps),
               bank, bank3, to_dev(inp.res_w), to_dev(inp.rms_w), to_dev(inp.onw),
               _matrix(inp.out_init, c, "out", gaps), gaps)


def run(d: Dev, path: Optional[int] = None, stream=None) -> None:
    c = d.case
    A.attnres_fwd(d.prefix, d.delta, d.bank3, c.nb, d.res_w, d.rms_w, c.eps, d.onw, c.oeps, c.widx,
                  d.out, stream=stream, path=path)


@dataclass
class Result:
    out: np.ndarray
    prefix: np.ndarray
    bank: np.ndarray
    delta: Optional[np.ndarray]
    res_w: np.ndarray
    rms_w: np.ndarray
    onw: Optional[np.ndarray]
    gaps_untouched: dict        # name -> whether every gap element still holds ROW_GAP_BITS


def download(d: Dev) -> Result:
    torch.cuda.synchronize()
    H = d.case.H
    gaps = {name: bool((full[:, H:] == ROW_GAP_BITS).all().item()) for name, full in d.gaps.items()}
    return Result(from_dev(d.out), from_dev(d.prefix), from_dev(d.bank), from_dev(d.delta),
                  from_dev(d.res_w), from_dev(d.rms_w), from_dev(d.onw), gaps)


def oracle_full(inp: W.Inputs):
    import oracle
    c = inp.case
    return oracle.attnres_oracle(inp.prefix, inp.delta, inp.bank, c.token_stride, c.slot_stride,
                                 c.cap, c.nb, inp.res_w, inp.rms_w, c.eps, inp.onw, c.oeps, c.widx)


def oracle_full_threaded(inp: W.Inputs, threads: int = 16):
    """The oracle over every token of the call, run as contiguous token ranges
    on a pool of threads (tokens are independent; the C oracle runs without
    the GIL).  Returns out_bits, prefix_after and bank_after of the whole call,
    stitched from the ranges; the ranges' bank slices are disjoint because a
    token's rows lie within its token stride."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    c = inp.case
    T, ts = c.T, c.token_stride
    if c.cap > 1 and (c.cap - 1) * c.slot_stride + c.H > ts:
        # A token's rows do not lie within its token stride (a slot-major
        # bank): token ranges have no bank slice of their own, so run the
        # oracle over the whole call at once.
        r = oracle_full(inp)
        return FullRef(r.out_bits, r.prefix_after, r.bank_after)
    n = max(1, min(threads, T))
    bounds = [(T * k // n, T * (k + 1) // n) for k in range(n)]
    bank_after = inp.bank.copy()
    out_bits = np.empty((T, c.H), dtype=np.uint16)
    prefix_after = np.empty((T, c.H), dtype=np.uint16)

    def run(ab):
        a, b = ab
        if a == b:
            return
        r = oracle.attnres_oracle(inp.prefix[a:b], None if inp.delta is None else inp.delta[a:b],
                                  inp.bank[a * ts:b * ts], ts, c.slot_stride, c.cap, c.nb,
                                  inp.res_w, inp.rms_w, c.eps, inp.onw, c.oeps, c.widx)
        out_bits[a:b] = r.out_bits
        prefix_after[a:b] = r.prefix_after
        bank_after[a * ts:b * ts] = r.bank_after

    with ThreadPoolExecutor(max_workers=n) as pool:
        list(pool.map(run, bounds))
    return FullRef(out_bits, prefix_after, bank_after)


@dataclass
class FullRef:
    out_bits: np.ndarray
    prefix_after: np.ndarray
    bank_after: np.ndarray


def oracle_sample(inp: W.Inputs, tokens: Sequence[int]):
    import oracle
    c = inp.case
    return oracle.attnres_oracle_tokens(tokens, inp.prefix, inp.delta, inp.bank, c.token_stride,
                                        c.slot_stride, c.cap, c.nb, inp.res_w, inp.rms_w, c.eps,
                                        inp.onw, c.oeps, c.widx)


def assert_out_close(got_bits: np.ndarray, ref_bits: np.ndarray, what: str) -> None:
    """|gpu - RNE_bf16(oracle)| <= 1e-2 + 1.6e-2 * |RNE_bf16(oracle)| everywhere."""
    g = widen(got_bits)
    o = widen(ref_bits)
    assert np.isfinite(o).all(), f"{what}: oracle output not finite"
    assert np.isfinite(g).all(), f"{what}: GPU output has non-finite values (sentinel left or NaN)"
    err = np.abs(g - o)
    bound = ATOL + RTOL * np.abs(o)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; worst at {i}: "
                             f"gpu={g[i]!r} oracle={o[i]!r}")


def check_full(inp: W.Inputs, got: Result, ref) -> None:
    """Element-wise against the oracle over the whole call, bit-exact where
    exactness is required."""
    c = inp.case
    assert_out_close(got.out, ref.out_bits, c.name + " out")
    assert (got.prefix == ref.prefix_after).all(), c.name + ": prefix after the call differs"
    diff = np.nonzero(got.bank != ref.bank_after)[0]
    assert diff.size == 0, (f"{c.name}: bank differs at {diff.size} elements "
                            f"(first at flat index {diff[:4]})")
    check_inputs_untouched(inp, got)


def check_inputs_untouched(inp: W.Inputs, got: Result) -> None:
    c = inp.case
    for name, ok in got.gaps_untouched.items():
        assert ok, f"{c.name}: the gap after a {name} row was written"
    if inp.delta is not None:
        assert (got.delta == inp.delta).all(), c.name + ": delta modified"
    assert (got.res_w == inp.res_w).all() and (got.rms_w == inp.rms_w).all(), c.name + ": weights modified"
    if inp.onw is not None:
        assert (got.onw == inp.onw).all(), c.name + ": output-norm weight modified"


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    base = {0, 1, T - 2, T - 1}
    base |= set(rng.choice(T, size=min(n, T), replace=False).tolist())
    return np.array(sorted(t for t in base if 0 <= t < T))
