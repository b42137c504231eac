"""Seeded synthetic inputs for the attention-residual forward.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so the GPU tests, the oracle tests and the benchmark can
all use it without sharing any computation.  Everything is generated on the
CPU from a ``torch.Generator`` in fp32 and rounded once to bf16 by torch's
round-to-nearest-even cast.

Workload shapes follow the pages: hidden size 7168, at most 8 block residuals
per token, single-token decode up to long prefill (vLLM PR #54261 digest,
"Motivation" and "Risks and impact").  The pages benchmark on random inputs
only, so no dataset is involved.  Other hidden sizes use the same recipes.

Layout conventions used everywhere:
  * prefix, delta, out: [T, H] bf16 values, held densely here; on the device
    their rows may be placed ``row_pad`` elements apart beyond H (the gap
    filled with a sentinel).
  * bank: one flat bf16 buffer; element (t, i, h) sits at
    ``t*token_stride + i*slot_stride + h``.  Token-major by default
    (slot_stride = H, token_stride = cap*H + token_pad); slot-major on request.
  * unused bank slots, token padding and the output buffer are pre-filled with
    a NaN sentinel that depends on position, so a stray read poisons the
    output and a stray write breaks bit-exactness.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np
import torch

HIDDEN = 7168
MAX_BLOCKS = 8


@dataclass(frozen=True)
class Case:
    name: str
    T: int
    nb: int
    cap: int = MAX_BLOCKS
    H: int = HIDDEN
    has_delta: bool = True
    has_onorm: bool = True
    widx: int = -1
    token_pad: int = 0          # extra elements per token after the cap slots
    row_pad: int = 0            # extra elements after each prefix/delta/out row on the device
    slot_major: bool = False    # bank laid out [cap, T, H] instead of [T, cap, H]
    recipe: str = "normal"      # normal | decode | student_t | soft
    seed: int = 0
    eps: float = 1e-6
    oeps: float = 1e-6

    @property
    def row_stride(self) -> int:
        return self.H + self.row_pad

    @property
    def slot_stride(self) -> int:
        return self.T * self.H if self.slot_major else self.H

    @property
    def token_stride(self) -> int:
        return self.H if self.slot_major else self.cap * self.H + self.token_pad

    @property
    def bank_elems(self) -> int:
        if self.slot_major:
            return self.cap * self.T * self.H
        return self.T * self.token_stride

    def algorithmic_bytes(self) -> int:
        """Bytes a call must move at minimum: rows read + rows written per
        token, plus the weight rows once."""
        rows_read = self.nb + 1 + int(self.has_delta)
        rows_written = 1 + int(self.has_delta) + int(self.widx >= 0)
        weight_rows = 2 + int(self.has_onorm)
        return 2 * self.H * (self.T * (rows_read + rows_written) + weight_rows)


def sentinel_bits(t: np.ndarray, i: np.ndarray, h: np.ndarray) -> np.ndarray:
    """A position-dependent bf16 NaN pattern: exponent all ones, mantissa in
    1..127, sign clear."""
    return (0x7F80 | (1 + (t * 31 + i * 7 + h) % 127)).astype(np.uint16)


def _sentinel_block(t_col: np.ndarray, base_mod: np.ndarray) -> np.ndarray:
    """sentinel_bits for a block of rows: t_col [n, 1] token indices and
    base_mod [m] = (i*7 + h) mod 127 of each column, without int64 modulo
    over the whole block."""
    tm = ((t_col * 31) % 127).astype(np.uint16)
    r = base_mod.astype(np.uint16)[None, :] + tm
    r -= np.uint16(127) * (r >= 127)
    return np.uint16(0x7F80) | (r + np.uint16(1))


def _bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def _bits(x: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (a view-copy, no rounding)."""
    return x.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class Inputs:
    case: Case
    prefix: np.ndarray                    # [T, H] uint16
    delta: Optional[np.ndarray]           # [T, H] uint16 or None
    bank: np.ndarray                      # flat uint16, bank_elems long
    res_w: np.ndarray                     # [H] uint16
    rms_w: np.ndarray                     # [H] uint16
    onw: Optional[np.ndarray]             # [H] uint16 or None
    out_init: np.ndarray                  # [T, H] uint16 sentinel
    meta: Dict[str, float] = field(default_factory=dict)


def _rows(gen: torch.Generator, n: int, H: int, recipe: str,
          slot: Optional[int]) -> torch.Tensor:
    """n fp32 rows of the value recipe."""
    z = torch.randn(n, H, generator=gen)
    if recipe in ("normal", "soft"):
        return z
    if recipe == "decode":
        # bank slot i has standard deviation i+1; prefix/delta stay N(0,1)
        return z if slot is None else z * float(slot + 1)
    if recipe == "student_t":
        # Student-t with 4 degrees of freedom: Z / sqrt(V/4), V ~ chi^2_4,
        # where chi^2_4 = -2 ln(U1) - 2 ln(U2).  Each row is then rescaled to a
        # root-mean-square drawn uniformly from [1, 50].
        u1 = torch.rand(n, H, generator=gen).clamp_min_(1e-30)
        u2 = torch.rand(n, H, generator=gen).clamp_min_(1e-30)
        v = -2.0 * (torch.log(u1) + torch.log(u2))
        x = z / torch.sqrt(v / 4.0)
        target = 1.0 + 49.0 * torch.rand(n, 1, generator=gen)
        cur_rms = torch.sqrt(torch.mean(x.double() * x.double(), dim=1, keepdim=True)).float()
        return x * (target / cur_rms)
    raise ValueError(f"unknown recipe {recipe!r}")


def make_inputs(case: Case, chunk_tokens: int = 512) -> Inputs:
    """All inputs of one call, as bf16 bit patterns on the CPU."""
    gen = torch.Generator().manual_seed(case.seed)
    T, H, cap, nb = case.T, case.H, case.cap, case.nb

    w_res = 1.0 + 0.1 * torch.randn(H, generator=gen)
    if case.recipe == "soft":
        # soft-logit variant: sqrt(sum q^2) ~ 1 so the softmax is not one-hot
        w_res = (0.0118 * (HIDDEN / H) ** 0.5) * torch.randn(H, generator=gen)
    res_w = _bits(_bf16(w_res))
    rms_w = _bits(_bf16(1.0 + 0.1 * torch.randn(H, generator=gen)))
    onw = _bits(_bf16(1.0 + 0.1 * torch.randn(H, generator=gen))) if case.has_onorm else None

    prefix = np.empty((T, H), dtype=np.uint16)
    delta = np.empty((T, H), dtype=np.uint16) if case.has_delta else None
    bank = np.empty(case.bank_elems, dtype=np.uint16)
    if case.slot_major:
        view = bank.reshape(cap, T, H)
    else:
        view = bank.reshape(T, case.token_stride)

    # Position of every element of one token's bank span: slot i and element h
    # (token padding lands at i == cap).
    if not case.slot_major:
        off = np.arange(case.token_stride, dtype=np.int64)
        i_of, h_of = np.divmod(off, H)
        base_mod = (i_of * 7 + h_of) % 127

    for t0 in range(0, T, chunk_tokens):
        n = min(chunk_tokens, T - t0)
        t_col = np.arange(t0, t0 + n, dtype=np.int64)[:, None]
        # sentinel in the unused slots and the token padding
        if case.slot_major:
            h_row = np.arange(H, dtype=np.int64)
            for i in range(nb, cap):
                view[i, t0:t0 + n] = _sentinel_block(t_col, (i * 7 + h_row) % 127)
        elif nb * H < case.token_stride:
            view[t0:t0 + n, nb * H:] = _sentinel_block(t_col, base_mod[nb * H:])

        prefix[t0:t0 + n] = _bits(_bf16(_rows(gen, n, H, case.recipe, None)))
        if delta is not None:
            delta[t0:t0 + n] = _bits(_bf16(_rows(gen, n, H, case.recipe, None)))
        for i in range(nb):
            rows = _bits(_bf16(_rows(gen, n, H, case.recipe, i)))
            if case.slot_major:
                view[i, t0:t0 + n] = rows
            else:
                view[t0:t0 + n, i * H:(i + 1) * H] = rows

    out_init = _sentinel_block(np.arange(T, dtype=np.int64)[:, None],
                               (9 * 7 + np.arange(H, dtype=np.int64)) % 127)
    return Inputs(case, prefix, delta, bank, res_w, rms_w, onw, out_init)


# ---------------------------------------------------------------------------
# The named workloads.
# ---------------------------------------------------------------------------

def pr1_ref() -> Case:
    """Small reference case: 4 tokens, 4 blocks, delta and output norm on."""
    return Case("pr1_ref_T4_nb4", T=4, nb=4, seed=0)


def decode_sweep(nbs=(0, 1, 4, 8)) -> List[Case]:
    """Single-token decode: slot i drawn with standard deviation i+1."""
    return [Case(f"decode_T1_nb{nb}", T=1, nb=nb, recipe="decode", seed=1) for nb in nbs]


def mid_prefill() -> Case:
    """1024 tokens, 8 blocks, delta and output norm on, write into slot 3
    (a slot that is also a source)."""
    return Case("mid_prefill_T1024_nb8_w3", T=1024, nb=8, widx=3, seed=2)


def long_prefill(T: int = 8192) -> Case:
    """Long prefill: heavy-tailed rows, token stride padded by 64 elements,
    no delta, no output norm, no write."""
    return Case(f"long_prefill_T{T}_nb8", T=T, nb=8, has_delta=False, has_onorm=False,
                token_pad=64, recipe="student_t", seed=3 if T == 8192 else 4)


def variant_matrix(Ts=(1, 16, 256, 2048)) -> List[Case]:
    """T x nb in {0,4,8} x delta x output norm x write in {-1, nb-1}: 80 cases
    for the default T list (nb = 0 folds the two write choices)."""
    cases = []
    k = 0
    for T in Ts:
        for nb in (0, 4, 8):
            for d in (False, True):
                for o in (False, True):
                    for w in sorted({-1, nb - 1}):
                        cases.append(Case(f"var_T{T}_nb{nb}_d{int(d)}_o{int(o)}_w{w}",
                                          T=T, nb=nb, has_delta=d, has_onorm=o, widx=w,
                                          seed=5 + k))
                        k += 1
    return cases


def soft_logits(T: int = 64, nb: int = 8) -> Case:
    """Not one of the named workloads: scoring weights scaled so logits are
    O(1) and the mixture really mixes."""
    return Case(f"soft_T{T}_nb{nb}", T=T, nb=nb, widx=nb - 1, recipe="soft", seed=77)


def other_hidden(H: int, T: int = 40, nb: int = 6, **kw) -> Case:
    """Not one of the named workloads: the same recipe at another hidden
    size (delta, output norm and a write into a source slot by default)."""
    kw.setdefault("widx", nb - 1 if nb > 0 else -1)
    kw.setdefault("seed", 1000 + H + T + nb)
    return Case(f"hidden{H}_T{T}_nb{nb}", T=T, nb=nb, H=H, **kw)


def with_(case: Case, **kw) -> Case:
    return replace(case, **kw)
