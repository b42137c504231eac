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
ATTNRES_PATH_ANY_H = 3
ATTNRES_SPLIT_MAX_TOKENS = 256
ATTNRES_MAX_HIDDEN = 16384

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
# prefix, prefix_stride, delta, delta_stride, blocks, ts, ss, cap, nb, res_w, rms_w, eps,
# onw, oeps, widx, out, out_stride, T, H
_STRIDED_ARGS = [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _int, _int, _vp, _vp, _f32, _vp, _f32,
                 _int, _vp, _i64, _i64, _i64]
_lib.attnres_fwd_strided.argtypes = _STRIDED_ARGS + [_vp, _int]
_lib.attnres_fwd_strided.restype = _int
_lib.attnres_fwd_noalloc.argtypes = _STRIDED_ARGS + [_vp, _int]
_lib.attnres_fwd_noalloc.restype = _int
_lib.attnres_partial_bytes.argtypes = [_i64, _i64]
_lib.attnres_partial_bytes.restype = _i64
_lib.attnres_fwd_bank.argtypes = _STRIDED_ARGS + [_vp, _i64, _vp]
_lib.attnres_fwd_bank.restype = _int
_lib.attnres_fwd_cur.argtypes = _STRIDED_ARGS + [_vp, _i64, _vp]
_lib.attnres_fwd_cur.restype = _int
_lib.attnres_validate_strided.argtypes = list(_STRIDED_ARGS)
_lib.attnres_validate_strided.restype = _int
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
_lib.attnres_auto_path.argtypes = [_i64, _i64, _int]
_lib.attnres_auto_path.restype = _int
_lib.attnres_debug_force_wait_failure.argtypes = [_int]
_lib.attnres_debug_force_wait_failure.restype = _int
_lib.attnres_debug_workspace_frames.argtypes = [_int]
_lib.attnres_debug_workspace_frames.restype = _int


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


def _rows(name: str, t: Optional[torch.Tensor], T: int, H: int, required: bool) -> int:
    """Checks a [T, H] matrix argument; returns its row stride in elements
    (H when T <= 1, where the library ignores it)."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return H
    if t.dtype not in _BF16_LIKE:
        raise TypeError(f"{name} must be bf16 (got {t.dtype})")
    if t.dim() != 2 or t.shape[0] != T or t.shape[1] != H:
        raise ValueError(f"{name} must be [{T}, {H}] with unit element stride")
    if T > 0 and H > 0 and t.stride(1) != 1:
        raise ValueError(f"{name} must be [{T}, {H}] with unit element stride")
    return t.stride(0) if T > 1 else H


def _marshal(prefix, delta, blocks, num_blocks, res_w, rms_w, rms_eps, output_norm_weight,
             output_norm_eps, block_write_idx, out):
    if prefix.dim() != 2:
        raise ValueError("prefix must be [T, H]")
    T, H = prefix.shape
    ps = _rows("prefix", prefix, T, H, True)
    ds = _rows("delta", delta, T, H, False)
    os_ = _rows("out", out, T, H, True)
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
    return dict(prefix=_ptr(prefix), ps=ps, delta=_ptr(delta), ds=ds, blocks=_ptr(blocks), ts=ts,
                ss=ss, cap=cap, nb=int(num_blocks), res_w=_ptr(res_w), rms_w=_ptr(rms_w),
                eps=float(rms_eps), onw=_ptr(output_norm_weight), oeps=float(output_norm_eps),
                widx=int(block_write_idx), out=_ptr(out), os=os_, T=T, H=H)


def _dense_args(m):
    return (m["prefix"], m["delta"], m["blocks"], m["ts"], m["ss"], m["cap"], m["nb"], m["res_w"],
            m["rms_w"], m["eps"], m["onw"], m["oeps"], m["widx"], m["out"], m["T"], m["H"])


def _strided_args(m):
    return (m["prefix"], m["ps"], m["delta"], m["ds"], m["blocks"], m["ts"], m["ss"], m["cap"],
            m["nb"], m["res_w"], m["rms_w"], m["eps"], m["onw"], m["oeps"], m["widx"], m["out"],
            m["os"], m["T"], m["H"])


def _dense(m) -> bool:
    return m["ps"] == m["H"] and m["ds"] == m["H"] and m["os"] == m["H"]


def _device_of(prefix: torch.Tensor, **others: Optional[torch.Tensor]) -> torch.device:
    """prefix's GPU, once every other tensor argument is on it too: the kernels
    dereference every pointer on that device, so a host tensor or one on
    another GPU would fault there and is refused here."""
    dev = prefix.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    for name, t in others.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, prefix on {dev}: all tensors must be "
                             "on the same GPU")
    return dev


def attnres_fwd(prefix: torch.Tensor, delta: Optional[torch.Tensor],
                blocks: Optional[torch.Tensor], num_blocks: int, res_w: torch.Tensor,
                rms_w: torch.Tensor, rms_eps: float,
                output_norm_weight: Optional[torch.Tensor], output_norm_eps: float,
                block_write_idx: int, out: torch.Tensor,
                stream: Optional[torch.cuda.Stream] = None, path: Optional[int] = None) -> None:
    """Enqueues the AttnRes forward on `stream` (default: the current stream).

    prefix, delta, out: [T, H] with unit element stride and any row stride
    (dense rows go through attnres_fwd / attnres_fwd_path, others through
    attnres_fwd_strided); blocks: [T, capacity, H] (any token/slot strides);
    weights: [H].  prefix (with a delta) and blocks[:, block_write_idx] are
    updated in place.  `path` forces one of the ATTNRES_PATH_* kernels.
    """
    m = _marshal(prefix, delta, blocks, num_blocks, res_w, rms_w, rms_eps, output_norm_weight,
                 output_norm_eps, block_write_idx, out)
    dev = _device_of(prefix, delta=delta, blocks=blocks, res_w=res_w, rms_w=rms_w,
                     output_norm_weight=output_norm_weight, out=out)
    with torch.cuda.device(dev):
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        if not _dense(m):
            rc = _lib.attnres_fwd_strided(*_strided_args(m), s.cuda_stream,
                                          ATTNRES_PATH_AUTO if path is None else int(path))
            where = "attnres_fwd_strided"
        elif path is None:
            rc = _lib.attnres_fwd(*_dense_args(m), s.cuda_stream)
            where = "attnres_fwd"
        else:
            rc = _lib.attnres_fwd_path(*_dense_args(m), s.cuda_stream, int(path))
            where = "attnres_fwd_path"
    if rc != ATTNRES_OK:
        raise AttnResError(rc, where)


def attnres_fwd_noalloc(prefix: torch.Tensor, delta: Optional[torch.Tensor],
                        blocks: Optional[torch.Tensor], num_blocks: int, res_w: torch.Tensor,
                        rms_w: torch.Tensor, rms_eps: float,
                        output_norm_weight: Optional[torch.Tensor], output_norm_eps: float,
                        block_write_idx: int, out: torch.Tensor,
                        stream: Optional[torch.cuda.Stream] = None,
                        path: Optional[int] = None) -> None:
    """attnres_fwd through the library's entry point that allocates nothing
    (the split path then exchanges through a static per-device array; calls
    that overlap on one GPU race).  Same arguments as attnres_fwd."""
    m = _marshal(prefix, delta, blocks, num_blocks, res_w, rms_w, rms_eps, output_norm_weight,
                 output_norm_eps, block_write_idx, out)
    dev = _device_of(prefix, delta=delta, blocks=blocks, res_w=res_w, rms_w=rms_w,
                     output_norm_weight=output_norm_weight, out=out)
    with torch.cuda.device(dev):
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        rc = _lib.attnres_fwd_noalloc(*_strided_args(m), s.cuda_stream,
                                      ATTNRES_PATH_AUTO if path is None else int(path))
    if rc != ATTNRES_OK:
        raise AttnResError(rc, "attnres_fwd_noalloc")


def attnres_partial_bytes(T: int, H: int) -> int:
    """Bytes of the partial-state buffer of the two-kernel form."""
    n = _lib.attnres_partial_bytes(int(T), int(H))
    if n < 0:
        raise AttnResError(int(n), "attnres_partial_bytes")
    return n


def _two_part(fn_name, prefix, delta, blocks, num_blocks, res_w, rms_w, rms_eps,
              output_norm_weight, output_norm_eps, block_write_idx, out, partial, stream):
    m = _marshal(prefix, delta, blocks, num_blocks, res_w, rms_w, rms_eps, output_norm_weight,
                 output_norm_eps, block_write_idx, out)
    dev = _device_of(prefix, delta=delta, blocks=blocks, res_w=res_w, rms_w=rms_w,
                     output_norm_weight=output_norm_weight, out=out, partial=partial)
    nbytes = 0 if partial is None else partial.numel() * partial.element_size()
    if partial is not None and not partial.is_contiguous():
        raise ValueError("partial must be contiguous")
    with torch.cuda.device(dev):
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        rc = getattr(_lib, fn_name)(*_strided_args(m), _ptr(partial), nbytes, s.cuda_stream)
    if rc != ATTNRES_OK:
        raise AttnResError(rc, fn_name)


def attnres_fwd_bank(prefix, delta, blocks, num_blocks, res_w, rms_w, rms_eps,
                     output_norm_weight, output_norm_eps, block_write_idx, out,
                     partial: Optional[torch.Tensor],
                     stream: Optional[torch.cuda.Stream] = None) -> None:
    """First kernel of the two-kernel form (the bank rows only; see
    include/attnres.h): writes the partial state into `partial`, a contiguous
    device tensor of at least attnres_partial_bytes(T, H) bytes."""
    _two_part("attnres_fwd_bank", prefix, delta, blocks, num_blocks, res_w, rms_w, rms_eps,
              output_norm_weight, output_norm_eps, block_write_idx, out, partial, stream)


def attnres_fwd_cur(prefix, delta, blocks, num_blocks, res_w, rms_w, rms_eps,
                    output_norm_weight, output_norm_eps, block_write_idx, out,
                    partial: Optional[torch.Tensor],
                    stream: Optional[torch.cuda.Stream] = None) -> None:
    """Second kernel of the two-kernel form: cur, the merge with the bank
    part's state, the output norm and every store of attnres_fwd."""
    _two_part("attnres_fwd_cur", prefix, delta, blocks, num_blocks, res_w, rms_w, rms_eps,
              output_norm_weight, output_norm_eps, block_write_idx, out, partial, stream)


def attnres_fwd_path(*args, path: int, **kw) -> None:
    """attnres_fwd with an explicit path selector."""
    attnres_fwd(*args, path=path, **kw)


def attnres_validate(prefix, delta, blocks, num_blocks, res_w, rms_w, rms_eps,
                     output_norm_weight, output_norm_eps, block_write_idx, out) -> int:
    """The library's host-side checks alone; returns the status code."""
    m = _marshal(prefix, delta, blocks, num_blocks, res_w, rms_w, rms_eps, output_norm_weight,
                 output_norm_eps, block_write_idx, out)
    if _dense(m):
        return _lib.attnres_validate(*_dense_args(m))
    return _lib.attnres_validate_strided(*_strided_args(m))


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


def attnres_auto_path(T: int, H: int, num_blocks: int) -> int:
    """The ATTNRES_PATH_* kernel that attnres_fwd runs for these sizes
    (host only); raises AttnResError for sizes it rejects."""
    rc = _lib.attnres_auto_path(int(T), int(H), int(num_blocks))
    if rc < 0:
        raise AttnResError(rc, "attnres_auto_path")
    return rc


def attnres_debug_force_wait_failure(enable: bool) -> None:
    """Tests of the failure path only: while enabled, split-path calls give
    up their cross-workgroup waits (see include/attnres.h)."""
    _lib.attnres_debug_force_wait_failure(1 if enable else 0)


def attnres_debug_workspace_frames(mode: int) -> None:
    """Tests only: which of the split path's two workspace frames each
    workgroup writes (-1 default, 0..255 a mask by XCD, 256 by part parity;
    see include/attnres.h)."""
    rc = _lib.attnres_debug_workspace_frames(int(mode))
    if rc != ATTNRES_OK:
        raise AttnResError(rc, "attnres_debug_workspace_frames")
