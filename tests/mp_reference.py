"""Brute-force evaluation of the attention-residual forward in mpmath at 50
significant digits, for tiny hidden sizes.

Independent of the C oracle: it receives the sources as nested Python lists
(never the strided bank), rounds with mpmath's own round-to-nearest-even at 8
significant bits, uses the un-shifted softmax exp(l_j) / sum_k exp(l_k) and the
factored logit (q . x) / sqrt(mean(x^2) + eps).

Definition: Kimi K3 attention-residual walkthrough (vllm-ascend PR #14840,
"Implementation walkthrough"), with the in-place semantics of the vLLM
PR #54261 digest's kernel snippet; softmax over raw rows, cur = RNE(prefix +
delta).
"""
from __future__ import annotations

import struct
from typing import List, Optional, Sequence

from mpmath import mp, mpf

mp.dps = 50


def b2m(bits: int) -> mpf:
    """bf16 bit pattern -> exact mpf."""
    return mpf(struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0])


def rne8(x: mpf) -> mpf:
    """Round to 8 significant bits, nearest, ties to even (mpmath rounding;
    no exponent limits, so only for values well inside bf16's range)."""
    with mp.workprec(8):
        r = +x
    return mpf(r)


def mpf_to_bits(x: mpf) -> int:
    """An mpf that is exactly a bf16 value -> its bit pattern."""
    f = float(x)
    u = struct.unpack("<I", struct.pack("<f", f))[0]
    assert u & 0xFFFF == 0, "value is not a bf16 number"
    return u >> 16


def attnres_token(bank_rows: Sequence[Sequence[int]], prefix: Sequence[int],
                  delta: Optional[Sequence[int]], res_w: Sequence[int],
                  rms_w: Sequence[int], onw: Optional[Sequence[int]],
                  eps: float, oeps: float):
    """One token.  bank_rows are the nb valid source rows as bit patterns.
    Returns (y as mpf list, probs, logits, cur bit patterns)."""
    H = len(prefix)
    P = [b2m(v) for v in prefix]
    if delta is not None:
        cur = [rne8(P[h] + b2m(delta[h])) for h in range(H)]
    else:
        cur = P
    sources: List[List[mpf]] = [[b2m(v) for v in row] for row in bank_rows] + [cur]
    q = [b2m(rms_w[h]) * b2m(res_w[h]) for h in range(H)]
    e = mpf(eps)
    logits = []
    for x in sources:
        ms = mp.fsum(v * v for v in x) / H
        logits.append(mp.fdot(q, x) / mp.sqrt(ms + e))
    ex = [mp.exp(l) for l in logits]
    Z = mp.fsum(ex)
    p = [v / Z for v in ex]
    y = [mp.fsum(p[j] * sources[j][h] for j in range(len(sources))) for h in range(H)]
    if onw is not None:
        r = mp.sqrt(mp.fsum(v * v for v in y) / H + mpf(oeps))
        y = [y[h] / r * b2m(onw[h]) for h in range(H)]
    return y, p, logits, [mpf_to_bits(v) for v in cur]
