"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes an oracle library handle (the real one, or a copy with a
planted mistake in the mutation tests) and raises AssertionError on failure.

  * torch's float32 -> bfloat16 cast (round to nearest even) and mpmath's
    8-bit rounding pin the bf16 rounding;
  * ``torch.nn.functional.rms_norm`` in float64 pins the no-block case;
  * hand-derived closed forms (tests/golden/closed_forms.json) pin the softmax,
    the raw-row mixture and the output norm;
  * invariants: the softmax weights sum to one, permuting bank slots leaves
    the result unchanged, rescaling a source row leaves its logit unchanged;
  * mpmath brute force at hidden size 8 over nb 0..8 x delta x output norm x
    write slot, in token-major and slot-major bank layouts;
  * bit-exact written rows and untouched slots.

Definition: vllm-ascend PR #14840 "Implementation walkthrough" and the vLLM
PR #54261 digest (implementation breakdown and kernel snippet).
"""
from __future__ import annotations

import json
import os
import struct

import numpy as np
import torch

from oracle import oracle as O

from tests import mp_reference as MP

HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------------------------
# helpers (layout only; no method arithmetic)
# ----------------------------------------------------------------------------

def f2b(values) -> np.ndarray:
    """Floats that are exactly bf16 values -> bit patterns (asserted exact)."""
    out = []
    for v in values:
        u = struct.unpack("<I", struct.pack("<f", float(v)))[0]
        assert u & 0xFFFF == 0, f"{v} is not a bf16 value"
        out.append(u >> 16)
    return np.array(out, dtype=np.uint16)


def torch_bf16_bits(x: np.ndarray) -> np.ndarray:
    """torch's float32 -> bfloat16 (round to nearest even) as bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 by numpy bit placement (independent of the
    oracle's own widening)."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_bf16(rng: np.random.Generator, shape, scale=1.0) -> np.ndarray:
    return torch_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def pack_bank(rows_tic, cap: int, layout: str, pad: int = 0):
    """Logical bank [T][cap][H] of bit patterns (None = unused) -> flat buffer,
    token stride, slot stride.  Unused slots get a NaN pattern."""
    T = len(rows_tic)
    H = len(next(r for tok in rows_tic for r in tok if r is not None)) if any(
        r is not None for tok in rows_tic for r in tok) else 8
    if layout == "token":
        ss, ts = H, cap * H + pad
        size = T * ts
    else:  # slot-major
        ts, ss = H, T * H + pad
        size = cap * ss
    buf = np.full(size, 0x7FA5, dtype=np.uint16)
    for t in range(T):
        for i in range(cap):
            r = rows_tic[t][i] if i < len(rows_tic[t]) else None
            if r is not None:
                buf[t * ts + i * ss: t * ts + i * ss + H] = r
    return buf, ts, ss


def _close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max abs err {err:.3e} > {rtol:.1e} * {scale:.3e}"


# ----------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------

def pin_rne_matches_torch_cast(lib):
    """Oracle rounding == torch's float32->bf16 cast on fp32 inputs, including
    exact ties, subnormals and the overflow threshold."""
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),      # subnormal range
        (rng.standard_normal(2000) * 1e37).astype(np.float32),
    ])
    # exact ties: a bf16 value plus half its last-place step
    base = torch_bf16_bits(rng.standard_normal(3000).astype(np.float32))
    u = base.astype(np.uint32) << 16
    ties = (u | 0x8000).view(np.float32)
    extra = np.array([0.0, -0.0, 3.3895314e38, 3.3961775e38, 3.3961776e38, 1e-45, -1e-45,
                      1.1754944e-38, 9.1835e-41], dtype=np.float32)
    x = np.concatenate([x, ties, extra]).astype(np.float32)
    got = O.round_bf16_bits(x.astype(np.float64), lib=lib)
    want = torch_bf16_bits(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"rounding differs from torch at {x[bad[:5]]}: {got[bad[:5]]} vs {want[bad[:5]]}"


def pin_rne_direct_from_double(lib):
    """Doubles that are not fp32 values round directly (no detour via fp32):
    checked against mpmath's 8-bit nearest-even rounding."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal(3000) * 10.0
    # values just above / below a tie by far less than an fp32 step
    t = np.array([1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 2.0 ** -8 - 2.0 ** -40,
                  -(3.0 + 2.0 ** -7 + 2.0 ** -35), 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8])
    x = np.concatenate([x, t])
    got = O.round_bf16_bits(x, lib=lib)
    want = np.array([MP.mpf_to_bits(MP.rne8(MP.mpf(float(v)))) for v in x], dtype=np.uint16)
    assert (got == want).all(), "direct rounding of doubles differs from mpmath"
    assert list(got[-5:]) == [0x3F81, 0x3F80, 0xC041, 0x3F80, 0x3F82]


def pin_widen_exact(lib):
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    got = O.bf16_bits_to_f64(bits, lib=lib)
    want = widen(bits)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def pin_closed_forms(lib):
    """Hand-derived cases (tests/golden/closed_forms.json)."""
    with open(os.path.join(HERE, "golden", "closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        H, nb, cap = c["H"], c["nb"], c["cap"]
        bank_rows = [[f2b(r) for r in c["bank"]] + [None] * (cap - nb)]
        buf, ts, ss = pack_bank(bank_rows, cap, "token")
        pre = f2b(c["prefix"]).reshape(1, H)
        dl = None if c["delta"] is None else f2b(c["delta"]).reshape(1, H)
        onw = None if c["onw"] is None else f2b(c["onw"])
        r = O.attnres_oracle(pre, dl, buf, ts, ss, cap, nb, f2b(c["res_w"]), f2b(c["rms_w"]),
                             c["eps"], onw, c["oeps"], c["widx"], lib=lib)
        _close(r.probs[0], c["probs"], 1e-14, c["name"] + " probs")
        _close(r.out_f64[0], c["out"], 1e-14, c["name"] + " out")
        if c["widx"] >= 0:
            cur = np.array(c["prefix"]) + (0 if c["delta"] is None else np.array(c["delta"]))
            row = r.bank_after[c["widx"] * ss: c["widx"] * ss + H]
            assert (row == f2b(cur)).all(), c["name"] + " written row"


def pin_nb0_is_normalised_current_residual(lib):
    """nb = 0: out = RNE(cur) without output norm (bit-exact), and torch's
    float64 rms_norm of cur with it."""
    rng = np.random.default_rng(13)
    H, T = 7168, 3
    pre = rand_bf16(rng, (T, H))
    dl = rand_bf16(rng, (T, H))
    w = torch_bf16_bits(1.0 + 0.1 * rng.standard_normal(H).astype(np.float32))
    rw = torch_bf16_bits(1.0 + 0.1 * rng.standard_normal(H).astype(np.float32))
    cur_bits = torch_bf16_bits(widen(pre).astype(np.float32)
                               + widen(dl).astype(np.float32))
    for use_delta in (False, True):
        cur = cur_bits if use_delta else pre
        d = dl if use_delta else None
        r = O.attnres_oracle(pre, d, None, 0, 0, 0, 0, rw, rw, 1e-6, None, 1e-6, -1, lib=lib)
        assert (r.out_bits == cur).all(), "nb=0 without output norm must return cur"
        assert np.all(r.probs == 1.0)
        r = O.attnres_oracle(pre, d, None, 0, 0, 0, 0, rw, rw, 1e-6, w, 1e-5, -1, lib=lib)
        ref = torch.nn.functional.rms_norm(
            torch.from_numpy(widen(cur)), (H,),
            torch.from_numpy(widen(w)), eps=1e-5).numpy()
        _close(r.out_f64, ref, 1e-13, "nb=0 with output norm vs torch rms_norm")
    # A single source keeps weight 1 when its logit is 0/0 (eps = 0, an
    # all-zero row): the output is that row, zero, and not a NaN.
    zero = np.zeros((T, H), dtype=np.uint16)
    r = O.attnres_oracle(zero, None, None, 0, 0, 0, 0, rw, rw, 0.0, None, 1e-6, -1, lib=lib)
    assert np.all(r.probs == 1.0), "nb=0: weight 1 even for a 0/0 logit"
    assert (r.out_bits == 0).all(), "nb=0, zero row, eps = 0: out is the zero row"
    r = O.attnres_oracle(zero, None, None, 0, 0, 0, 0, rw, rw, 0.0, w, 1e-6, -1, lib=lib)
    assert (widen(r.out_bits) == 0).all(), "nb=0 with output norm: a zero row stays zero"


def _random_case(rng, T, H, nb, cap, scale_rows=True):
    pre = rand_bf16(rng, (T, H))
    dl = rand_bf16(rng, (T, H))
    rows = [[rand_bf16(rng, H, float(rng.uniform(0.2, 5.0)) if scale_rows else 1.0)
             for _ in range(nb)] + [None] * (cap - nb) for _ in range(T)]
    res_w = torch_bf16_bits(1.0 + 0.3 * rng.standard_normal(H).astype(np.float32))
    rms_w = torch_bf16_bits(1.0 + 0.3 * rng.standard_normal(H).astype(np.float32))
    onw = torch_bf16_bits(1.0 + 0.3 * rng.standard_normal(H).astype(np.float32))
    return pre, dl, rows, res_w, rms_w, onw


def pin_softmax_sums_to_one(lib):
    rng = np.random.default_rng(14)
    for nb in (0, 1, 3, 8):
        pre, dl, rows, res_w, rms_w, onw = _random_case(rng, 4, 64, nb, 8)
        buf, ts, ss = pack_bank(rows, 8, "token")
        r = O.attnres_oracle(pre, dl, buf, ts, ss, 8, nb, res_w, rms_w, 1e-6, onw, 1e-6, -1, lib=lib)
        assert np.all(r.probs >= 0)
        assert np.max(np.abs(r.probs.sum(axis=1) - 1.0)) <= 1e-15 * (nb + 1)
        # the probabilities are the softmax of the reported logits
        e = np.exp(r.logits - r.logits.max(axis=1, keepdims=True))
        _close(r.probs, e / e.sum(axis=1, keepdims=True), 1e-14, "probs vs logits")


def pin_permutation_invariance(lib):
    """Permuting bank slots 0..nb-1 (and the write slot with them) leaves the
    output, and the written row, unchanged."""
    rng = np.random.default_rng(15)
    H, T, nb, cap = 96, 3, 6, 8
    pre, dl, rows, res_w, rms_w, onw = _random_case(rng, T, H, nb, cap)
    widx = 2
    buf, ts, ss = pack_bank(rows, cap, "token")
    base = O.attnres_oracle(pre, dl, buf, ts, ss, cap, nb, res_w, rms_w, 1e-6, onw, 1e-6, widx, lib=lib)
    for _ in range(4):
        perm = rng.permutation(nb)            # new slot k holds old slot perm[k]
        rows2 = [[tok[perm[k]] for k in range(nb)] + [None] * (cap - nb) for tok in rows]
        widx2 = int(np.nonzero(perm == widx)[0][0])
        buf2, _, _ = pack_bank(rows2, cap, "token")
        r = O.attnres_oracle(pre, dl, buf2, ts, ss, cap, nb, res_w, rms_w, 1e-6, onw, 1e-6, widx2, lib=lib)
        _close(r.out_f64, base.out_f64, 1e-13, "permuted output")
        _close(r.logits[:, :nb], base.logits[:, perm], 1e-13, "permuted logits")
        for t in range(T):
            a = r.bank_after[t * ts + widx2 * ss: t * ts + widx2 * ss + H]
            b = base.bank_after[t * ts + widx * ss: t * ts + widx * ss + H]
            assert (a == b).all(), "permuted written row"


def pin_logit_scale_invariance(lib):
    """Scaling a source row by c > 0 leaves its logit unchanged when eps = 0,
    and changes it by at most |l| * eps/(2 ms) * |1/c^2 - 1| otherwise.
    Scaling by powers of two keeps the row exactly representable."""
    rng = np.random.default_rng(16)
    H, nb, cap = 128, 4, 4
    pre, dl, rows, res_w, rms_w, onw = _random_case(rng, 1, H, nb, cap, scale_rows=False)
    for eps in (0.0, 1e-3):
        buf, ts, ss = pack_bank(rows, cap, "token")
        base = O.attnres_oracle(pre, None, buf, ts, ss, cap, nb, res_w, rms_w, eps, None, 0.0, -1, lib=lib)
        for j, c in ((0, 4.0), (2, 0.25), (3, 64.0)):
            x = widen(rows[0][j]) * c
            rows2 = [list(rows[0])]
            rows2[0][j] = torch_bf16_bits(x.astype(np.float32))
            assert (widen(rows2[0][j]) == x).all()
            buf2, _, _ = pack_bank(rows2, cap, "token")
            r = O.attnres_oracle(pre, None, buf2, ts, ss, cap, nb, res_w, rms_w, eps, None, 0.0, -1, lib=lib)
            l0, l1 = base.logits[0, j], r.logits[0, j]
            ms = float(np.mean(widen(rows[0][j]) ** 2))
            bound = abs(l0) * (eps / (2 * ms)) * abs(1 / c ** 2 - 1) + 1e-12 * abs(l0)
            assert abs(l1 - l0) <= bound, (eps, j, l0, l1)
            others = [k for k in range(nb + 1) if k != j]
            _close(r.logits[0, others], base.logits[0, others], 1e-15, "other logits")


def pin_brute_force_mp(lib):
    """mpmath at 50 digits over nb 0..8 x delta x onorm x write slot in
    {-1, nb-1, nb}, two tokens each, both bank layouts (104 draws)."""
    rng = np.random.default_rng(17)
    H, T, cap = 8, 2, 9
    k = 0
    for nb in range(0, 9):
        for use_delta in (False, True):
            for use_onorm in (False, True):
                for widx in sorted({-1, nb - 1, nb}):
                    if widx < -1:
                        continue
                    layout = "token" if k % 2 == 0 else "slot"
                    k += 1
                    pre, dl, rows, res_w, rms_w, onw = _random_case(rng, T, H, nb, cap)
                    buf, ts, ss = pack_bank(rows, cap, layout, pad=8 if layout == "token" else 0)
                    d = dl if use_delta else None
                    w = onw if use_onorm else None
                    r = O.attnres_oracle(pre, d, buf, ts, ss, cap, nb, res_w, rms_w, 1e-6, w,
                                         1e-6, widx, lib=lib)
                    for t in range(T):
                        y, p, lg, cur = MP.attnres_token(
                            rows[t][:nb], pre[t], None if d is None else d[t], res_w, rms_w,
                            w, 1e-6, 1e-6)
                        tag = f"nb={nb} delta={use_delta} onorm={use_onorm} widx={widx} {layout} t={t}"
                        _close(r.out_f64[t], [float(v) for v in y], 1e-12, tag + " out")
                        _close(r.probs[t], [float(v) for v in p], 1e-12, tag + " probs")
                        _close(r.logits[t], [float(v) for v in lg], 1e-12, tag + " logits")
                        want_pre = np.array(cur if d is not None else pre[t], dtype=np.uint16)
                        assert (r.prefix_after[t] == want_pre).all(), tag + " prefix"
                        for i in range(cap):
                            got = r.bank_after[t * ts + i * ss: t * ts + i * ss + H]
                            if i == widx:
                                assert (got == np.array(cur, dtype=np.uint16)).all(), tag + " written"
                            else:
                                old = buf[t * ts + i * ss: t * ts + i * ss + H]
                                assert (got == old).all(), tag + f" slot {i} touched"
    assert k >= 100


def pin_written_rows_and_untouched(lib):
    """prefix' = RNE(prefix + delta) (torch fp32 add + bf16 cast, which is the
    correctly rounded sum of two bf16 values), the same row lands in the
    write slot; every other bank element, the padding and delta stay put."""
    rng = np.random.default_rng(18)
    H, T, nb, cap = 7168, 2, 5, 8
    pre, dl, rows, res_w, rms_w, onw = _random_case(rng, T, H, nb, cap)
    buf, ts, ss = pack_bank(rows, cap, "token", pad=64)
    dl_copy = dl.copy()
    want = torch_bf16_bits(widen(pre).astype(np.float32)
                           + widen(dl).astype(np.float32))
    for widx in (-1, 1, 6):
        r = O.attnres_oracle(pre, dl, buf, ts, ss, cap, nb, res_w, rms_w, 1e-6, onw, 1e-6, widx, lib=lib)
        assert (r.prefix_after == want).all()
        changed = np.nonzero(r.bank_after != buf)[0]
        if widx >= 0:
            expect = np.concatenate([np.arange(t * ts + widx * ss, t * ts + widx * ss + H)
                                     for t in range(T)])
            for t in range(T):
                assert (r.bank_after[t * ts + widx * ss: t * ts + widx * ss + H] == want[t]).all()
            assert set(changed.tolist()) <= set(expect.tolist())
        else:
            assert changed.size == 0
        assert (dl == dl_copy).all()
    r = O.attnres_oracle(pre, None, buf, ts, ss, cap, nb, res_w, rms_w, 1e-6, onw, 1e-6, -1, lib=lib)
    assert (r.prefix_after == pre).all(), "prefix must stay untouched without delta"


def pin_unused_slots_never_read(lib):
    """NaN in every unused slot and in the padding: the output stays finite
    and equals the output with those elements zeroed."""
    rng = np.random.default_rng(19)
    H, T, nb, cap = 256, 3, 3, 8
    pre, dl, rows, res_w, rms_w, onw = _random_case(rng, T, H, nb, cap)
    buf, ts, ss = pack_bank(rows, cap, "token", pad=16)   # NaN pattern in unused slots
    a = O.attnres_oracle(pre, dl, buf, ts, ss, cap, nb, res_w, rms_w, 1e-6, onw, 1e-6, -1, lib=lib)
    assert np.isfinite(a.out_f64).all()
    buf0 = buf.copy()
    buf0[np.isnan(widen(buf0))] = 0
    b = O.attnres_oracle(pre, dl, buf0, ts, ss, cap, nb, res_w, rms_w, 1e-6, onw, 1e-6, -1, lib=lib)
    assert (a.out_bits == b.out_bits).all()


def pin_token_independence(lib):
    """Running tokens one at a time equals running them together (checks the
    token stride as well as the per-token state reset)."""
    rng = np.random.default_rng(20)
    H, T, nb, cap = 64, 5, 4, 6
    pre, dl, rows, res_w, rms_w, onw = _random_case(rng, T, H, nb, cap)
    buf, ts, ss = pack_bank(rows, cap, "token", pad=8)
    whole = O.attnres_oracle(pre, dl, buf, ts, ss, cap, nb, res_w, rms_w, 1e-6, onw, 1e-6, 2, lib=lib)
    part = O.attnres_oracle_tokens(range(T), pre, dl, buf, ts, ss, cap, nb, res_w, rms_w, 1e-6,
                                   onw, 1e-6, 2, lib=lib)
    assert (whole.out_bits == part.out_bits).all()
    assert (whole.prefix_after == part.prefix_after).all()


ALL_PINS = [pin_rne_matches_torch_cast, pin_rne_direct_from_double, pin_widen_exact,
            pin_closed_forms, pin_nb0_is_normalised_current_residual, pin_softmax_sums_to_one,
            pin_permutation_invariance, pin_logit_scale_invariance, pin_brute_force_mp,
            pin_written_rows_and_untouched, pin_unused_slots_never_read, pin_token_independence]
