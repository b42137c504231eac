"""Thin Python binding of libattnres (C ABI in include/attnres.h).

Argument marshalling only: tensors are turned into device pointers, bank
strides and the current HIP stream; every step of the computation runs in the
HIP kernels.  There is no CPU fallback: if the library is missing this module
fails to import, and every call that the library rejects raises.

PyTorch supplies device memory and streams; tensors are bf16 (or int16 /
uint16 views of bf16 bit patterns).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattnres.so")

ATTNRES_OK = 0
ATTNRES_PATH_AUTO = 0
ATTNRES_PATH_ROW = 1
ATTNRES_PATH_SPLIT = 2
ATTNRES_SPLIT_MAX_TOKENS = 256

STATUS = {
    0: "ATTNRES_OK", -1: "ATTNRES_E_NULL", -2: "ATTNRES_E_SHAPE", -3: "ATTNRES_E_UNSUPPORTED",
    -4: "ATTNRES_E_NUM_BLOCKS", -5: "ATTNRES_E_WRITE_IDX", -6: "ATTNRES_E_ALIGN",
    -7: "ATTNRES_E_STRIDE", -8: "ATTNRES_E_ALIAS", -9: "ATTNRES_E_EPS", -10: "ATTNRES_E_NOT_INIT",
    -11: "ATTNRES_E_HIP", -12: "ATTNRES_E_PATH", -13: "ATTNRES_E_DEVICE_WAIT",
}
CODES = {v: k for k, v in STATUS.items()}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m kimi_k3_attention_amd.build` "
        "(there is no CPU fallback)")

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_f32 = ctypes.c_float
_FWD_ARGS = [_vp, _vp, _vp, _i64, _i64, _int, _int, _vp, _vp, _f32, _vp, _f32, _int, _vp,
             _i64, _i64]

_lib = ctypes.CDLL(LIB_PATH)
_lib.attnres_fwd.argtypes = _FWD_ARGS + [_vp]
_lib.attnres_fwd.restype = _int
_lib.attnres_fwd_path.argtypes = _FWD_ARGS + [_vp, _int]
_lib.attnres_fwd_path.restype = _int
_lib.attnres_validate.argtypes = list(_FWD_ARGS)
_lib.attnres_validate.restype = _int
_lib.attnres_init.argtypes = [_int]
_lib.attnres_init.restype = _int
_lib.attnres_shutdown.argtypes = []
_lib.attnres_shutdown.restype = None
_lib.attnres_device_status.argtypes = [_int]
_lib.attnres_device_status.restype = _int
_lib.attnres_strerror.argtypes = [_int]
_lib.attnres_strerror.restype = ctypes.c_char_p
_lib.attnres_last_hip_error.argtypes = []
_lib.attnres_last_hip_error.restype = _int


def lib() -> ctypes.CDLL:
    """The ctypes handle, argument types set (for raw-pointer calls)."""
    return _lib


class AttnResError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        self.name = STATUS.get(code, str(code))
        msg = _lib.attnres_strerror(code).decode()
        if code == CODES["ATTNRES_E_HIP"]:
            msg += f" (hipError {_lib.attnres_last_hip_error()})"
        super().__init__(f"{where}: {self.name}: {msg}")


_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _rows(name: str, t: Optional[torch.Tensor], T: int, H: int, required: bool):
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if t.dtype not in _BF16_LIKE:
        raise TypeError(f"{name} must be bf16 (got {t.dtype})")
    if t.dim() != 2 or t.shape[0] != T or t.shape[1] != H:
        raise ValueError(f"{name} must be [{T}, {H}] with row stride {H}")
    if T > 0 and (t.stride(1) != 1 or (T > 1 and t.stride(0) != H)):
        raise ValueError(f"{name} must be [{T}, {H}] with row stride {H}")


def _marshal(prefix, delta, blocks, num_blocks, res_w, rms_w, rms_eps, output_norm_weight,
             output_norm_eps, block_write_idx, out):
    if prefix.dim() != 2:
        raise ValueError("prefix must be [T, H]")
    T, H = prefix.shape
    _rows("prefix", prefix, T, H, True)
    _rows("delta", delta, T, H, False)
    _rows("out", out, T, H, True)
    for name, w in (("res_w", res_w), ("rms_w", rms_w), ("output_norm_weight", output_norm_weight)):
        if w is None:
            if name != "output_norm_weight":
                raise ValueError(f"{name} is required")
            continue
        if w.dtype not in _BF16_LIKE or w.dim() != 1 or w.shape[0] != H or \
                (H > 0 and w.stride(0) != 1):
            raise ValueError(f"{name} must be a contiguous bf16 [{H}] vector")
    if blocks is None:
        ts = ss = cap = 0
    else:
        if blocks.dtype not in _BF16_LIKE:
            raise TypeError("blocks must be bf16")
        if blocks.dim() != 3 or blocks.shape[0] != T or blocks.shape[2] != H or \
                (blocks.numel() > 0 and blocks.stride(2) != 1):
            raise ValueError(f"blocks must be [{T}, capacity, {H}] with unit element stride")
        ts, ss, cap = blocks.stride(0), blocks.stride(1), blocks.shape[1]
    return (_ptr(prefix), _ptr(delta), _ptr(blocks), ts, ss, cap, int(num_blocks), _ptr(res_w),
            _ptr(rms_w), float(rms_eps), _ptr(output_norm_weight), float(output_norm_eps),
            int(block_write_idx), _ptr(out), T, H)


def attnres_fwd(prefix: torch.Tensor, delta: Optional[torch.Tensor],
                blocks: Optional[torch.Tensor], num_blocks: int, res_w: torch.Tensor,
                rms_w: torch.Tensor, rms_eps: float,
                output_norm_weight: Optional[torch.Tensor], output_norm_eps: float,
                block_write_idx: int, out: torch.Tensor,
                stream: Optional[torch.cuda.Stream] = None, path: Optional[int] = None) -> None:
    """Enqueues the AttnRes forward on `stream` (default: the current stream).

    prefix, delta, out: [T, H]; blocks: [T, capacity, H] (any token/slot
    strides); weights: [H].  prefix (with a delta) and blocks[:, block_write_idx]
    are updated in place.  `path` forces ATTNRES_PATH_ROW / ATTNRES_PATH_SPLIT.
    """
    args = _marshal(prefix, delta, blocks, num_blocks, res_w, rms_w, rms_eps, output_norm_weight,
                    output_norm_eps, block_write_idx, out)
    dev = prefix.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    with torch.cuda.device(dev):
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        if path is None:
            rc = _lib.attnres_fwd(*args, s.cuda_stream)
        else:
            rc = _lib.attnres_fwd_path(*args, s.cuda_stream, int(path))
    if rc != ATTNRES_OK:
        raise AttnResError(rc, "attnres_fwd")


def attnres_fwd_path(*args, path: int, **kw) -> None:
    """attnres_fwd with an explicit path selector."""
    attnres_fwd(*args, path=path, **kw)


def attnres_validate(prefix, delta, blocks, num_blocks, res_w, rms_w, rms_eps,
                     output_norm_weight, output_norm_eps, block_write_idx, out) -> int:
    """The library's host-side checks alone; returns the status code."""
    return _lib.attnres_validate(*_marshal(prefix, delta, blocks, num_blocks, res_w, rms_w,
                                           rms_eps, output_norm_weight, output_norm_eps,
                                           block_write_idx, out))


def attnres_init(device: Optional[int] = None) -> None:
    d = torch.cuda.current_device() if device is None else int(device)
    rc = _lib.attnres_init(d)
    if rc != ATTNRES_OK:
        raise AttnResError(rc, "attnres_init")


def attnres_shutdown() -> None:
    _lib.attnres_shutdown()


def attnres_device_status(device: Optional[int] = None) -> int:
    d = torch.cuda.current_device() if device is None else int(device)
    return _lib.attnres_device_status(d)


def attnres_strerror(status: int) -> str:
    return _lib.attnres_strerror(int(status)).decode()


def attnres_last_hip_error() -> int:
    return _lib.attnres_last_hip_error()
