"""ctypes glue around the fp64 C oracle (``attnres_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Arguments are numpy arrays of bf16 *bit patterns*
(``uint16``) so that no bf16 conversion happens outside the C oracle.  The
oracle never mutates its inputs: it works on copies of ``prefix`` and of the
block bank and returns their post-call state.

Definition followed: the Kimi K3 attention-residual walkthrough of the
vllm-ascend PR #14840 page, with the in-place prefix and bank semantics of the
vLLM PR #54261 digest (kernel snippet, "Key source snippets").  The readings
taken where the pages are silent are listed in the C file's header.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from . import build as _build

_libs = {}


def load_library(path: Optional[str] = None):
    """ctypes handle of the oracle library (the built one by default; the
    mutation tests pass the path of a deliberately broken copy)."""
    if path is None:
        path = _build.ensure_built()
    lib = _libs.get(path)
    if lib is None:
        lib = ctypes.CDLL(path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f64p = ctypes.POINTER(ctypes.c_double)
        lib.oracle_attnres_fwd.restype = ctypes.c_int
        lib.oracle_attnres_fwd.argtypes = [
            ctypes.c_int64, ctypes.c_int64, u16p, u16p, u16p, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int, ctypes.c_int, u16p, u16p,
            ctypes.c_double, u16p, ctypes.c_double, ctypes.c_int, f64p, u16p,
            f64p, f64p]
        lib.oracle_round_bf16.restype = None
        lib.oracle_round_bf16.argtypes = [f64p, u16p, ctypes.c_int64]
        lib.oracle_bf16_to_double.restype = None
        lib.oracle_bf16_to_double.argtypes = [u16p, f64p, ctypes.c_int64]
        _libs[path] = lib
    return lib


def _load(lib=None):
    return lib if lib is not None else load_library()


def _u16(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.uint16 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def _f64(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def round_bf16_bits(x: np.ndarray, lib=None) -> np.ndarray:
    """bf16 bit patterns of round-to-nearest-even(x), x given in float64."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load(lib).oracle_round_bf16(_f64(x), _u16(out), x.size)
    return out


def bf16_bits_to_f64(b: np.ndarray, lib=None) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    _load(lib).oracle_bf16_to_double(_u16(b), _f64(out), b.size)
    return out


@dataclass
class OracleResult:
    out_f64: np.ndarray          # [T, H] float64, before the final rounding
    out_bits: np.ndarray         # [T, H] uint16, RNE_bf16 of out_f64
    prefix_after: np.ndarray     # [T, H] uint16, prefix after the call
    bank_after: Optional[np.ndarray]  # flat uint16, bank after the call
    logits: np.ndarray           # [T, nb+1] float64
    probs: np.ndarray            # [T, nb+1] float64


def attnres_oracle(prefix: np.ndarray, delta: Optional[np.ndarray],
                   bank: Optional[np.ndarray], token_stride: int,
                   slot_stride: int, cap: int, num_blocks: int,
                   res_w: np.ndarray, rms_w: np.ndarray, rms_eps: float,
                   output_norm_weight: Optional[np.ndarray],
                   output_norm_eps: float, block_write_idx: int, lib=None
                   ) -> OracleResult:
    """Runs the oracle over every token.

    prefix/delta are [T, H] uint16; bank is the flat uint16 buffer in which
    element (t, i, h) sits at ``t*token_stride + i*slot_stride + h``.
    """
    prefix = np.ascontiguousarray(prefix, dtype=np.uint16)
    T, H = prefix.shape
    nsrc = num_blocks + 1
    if T > 0 and (num_blocks > 0 or block_write_idx >= 0):
        # The C code trusts the strides: refuse a bank buffer they overrun.
        need = (T - 1) * int(token_stride) + (int(cap) - 1) * int(slot_stride) + H
        if bank is None or np.asarray(bank).size < need:
            raise ValueError(f"bank holds {0 if bank is None else np.asarray(bank).size} "
                             f"elements; the strides address {need}")
    pre = prefix.copy()
    bnk = None if bank is None else np.array(bank, dtype=np.uint16, copy=True)
    dlt = None if delta is None else np.ascontiguousarray(delta, dtype=np.uint16)
    out_f64 = np.empty((T, H), dtype=np.float64)
    out_bits = np.empty((T, H), dtype=np.uint16)
    logits = np.empty((T, nsrc), dtype=np.float64)
    probs = np.empty((T, nsrc), dtype=np.float64)
    onw = (None if output_norm_weight is None
           else np.ascontiguousarray(output_norm_weight, dtype=np.uint16))
    rc = _load(lib).oracle_attnres_fwd(
        T, H, _u16(pre), _u16(dlt), _u16(bnk), int(token_stride),
        int(slot_stride), int(cap), int(num_blocks),
        _u16(np.ascontiguousarray(res_w, dtype=np.uint16)),
        _u16(np.ascontiguousarray(rms_w, dtype=np.uint16)), float(rms_eps),
        _u16(onw), float(output_norm_eps), int(block_write_idx),
        _f64(out_f64), _u16(out_bits), _f64(logits), _f64(probs))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (rc={rc})")
    return OracleResult(out_f64, out_bits, pre, bnk, logits, probs)


@dataclass
class OracleTokens:
    tokens: np.ndarray           # the sampled token indices
    out_f64: np.ndarray          # [n, H]
    out_bits: np.ndarray         # [n, H]
    prefix_after: np.ndarray     # [n, H]
    written_row: Optional[np.ndarray]  # [n, H] bank row block_write_idx after the call
    probs: np.ndarray            # [n, nb+1]


def attnres_oracle_tokens(tokens: Sequence[int], prefix: np.ndarray,
                          delta: Optional[np.ndarray], bank: Optional[np.ndarray],
                          token_stride: int, slot_stride: int, cap: int,
                          num_blocks: int, res_w: np.ndarray, rms_w: np.ndarray,
                          rms_eps: float, output_norm_weight: Optional[np.ndarray],
                          output_norm_eps: float, block_write_idx: int, lib=None
                          ) -> OracleTokens:
    """Runs the oracle on selected tokens only (tokens are independent in the
    definition), for sampled checks of workloads too large to run whole."""
    H = prefix.shape[1]
    window = (cap - 1) * slot_stride + H
    outs_f, outs_b, pres, rows, probs = [], [], [], [], []
    for t in tokens:
        b = None
        if bank is not None:
            b = np.ascontiguousarray(bank[t * token_stride: t * token_stride + window])
        r = attnres_oracle(prefix[t:t + 1], None if delta is None else delta[t:t + 1],
                           b, token_stride, slot_stride, cap, num_blocks, res_w,
                           rms_w, rms_eps, output_norm_weight, output_norm_eps,
                           block_write_idx, lib=lib)
        outs_f.append(r.out_f64[0])
        outs_b.append(r.out_bits[0])
        pres.append(r.prefix_after[0])
        probs.append(r.probs[0])
        if block_write_idx >= 0:
            s = block_write_idx * slot_stride
            rows.append(r.bank_after[s:s + H].copy())
    return OracleTokens(np.asarray(tokens), np.stack(outs_f), np.stack(outs_b),
                        np.stack(pres), np.stack(rows) if rows else None,
                        np.stack(probs))
