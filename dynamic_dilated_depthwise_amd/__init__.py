"""MI355X (gfx950) library for the Dynamic Dilated Pyramid Module (DDPM) of HDFNet.

This module is the thin Python binding over the C ABI in ``include/ddpm.h``
(``libddpm.so``, hand-written HIP kernels).  Each function has the name of the C
entry point it calls and does argument marshalling only: it checks that the torch
tensors are contiguous device tensors of the right shapes and dtype, passes their
device pointers and the current HIP stream, and raises ``DDPMError`` when the
library returns an error.  Every step of the computation runs in the library's
kernels; there is no CPU or PyTorch fallback, and a missing library is an error.

Tensor layouts (NCHW, contiguous):
  x, y, grad_x, grad_y  [N, C, H, W]
  weight [3*C*K*K, C], bias [3*C*K*K]   (generator row o = (b*C + c)*K*K + t)
  taps   [N, 3*C*K*K, H, W]
  out, grad_out [N, 4*C, H, W]          (channel blocks x, d1, d3, d5)
  dweight_partials [S, 3*C*K*K, C], dbias_partials [S, 3*C*K*K]  float32
"""
import ctypes
import os

import torch

__all__ = [
    "DDPMError",
    "ddpm_filter_fwd",
    "ddpm_filter_bwd",
    "ddpm_fused_fwd",
    "ddpm_fused_bwd",
    "ddpm_fused_bwd_noalloc",
    "ddpm_reduce_partials",
    "ddpm_status_string",
    "num_partials_for",
    "library_path",
    "MAX_PARTIALS",
    "NOALLOC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libddpm.so")
MAX_PARTIALS = 16
NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024  # the library's fixed partials buffer (DDPM_NOALLOC_SCRATCH_BYTES)
_CUS = 256  # compute units of the chip (MI355X)
_DTYPES = {torch.float32: 0, torch.bfloat16: 1}

_lib = None


class DDPMError(RuntimeError):
    """A DDPM library call returned a non-zero status."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {ddpm_status_string(status)} ({status})")


def library_path():
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"DDPM HIP library not found at {_LIB_PATH}; build it with "
            "`python -m dynamic_dilated_depthwise_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.ddpm_filter_fwd.argtypes = [P, P, P, I64, I64, I64, I64, I, I, P]
    lib.ddpm_filter_bwd.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I, I, P]
    lib.ddpm_fused_fwd.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I, I, P]
    lib.ddpm_fused_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I64, I64, I64, I64, I, I, P]
    lib.ddpm_reduce_partials.argtypes = [P, P, I, P, P, I64, I, I, P]
    lib.ddpm_fused_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I, I64, I64, I64, I64, I, I, P]
    for f in ("ddpm_filter_fwd", "ddpm_filter_bwd", "ddpm_fused_fwd", "ddpm_fused_bwd", "ddpm_reduce_partials",
              "ddpm_fused_bwd_noalloc"):
        getattr(lib, f).restype = I
    lib.ddpm_status_string.argtypes = [I]
    lib.ddpm_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def raw_library():
    """The loaded ctypes library (for callers that pass raw device pointers)."""
    return _load()


def ddpm_status_string(status):
    return _load().ddpm_status_string(int(status)).decode()


def num_partials_for(N, C, H, W, K):
    """Split count S for the weight-gradient partials of an [N, C, H, W] input.

    At most one split per 1024 tokens and at most 16.  Among those counts, the one
    whose launch puts the least work on the busiest compute unit: the partial
    kernel runs 3K * ceil(C/16) * ceil(C/64) workgroups per split (one kernel row of
    one branch x 16 depthwise channels x up to 64 input channels), dealt over the
    chip's 256 CUs, so the busiest CU holds ceil(S * tiles / 256) of them, each over
    1/S of the tokens.  Ties go to the larger S.  At B=1, C=64, K=3 this gives 14
    (504 workgroups, at most two per CU) rather than 16 (576: a quarter of the CUs
    with three), which the kernel runs 15-20 % faster.
    """
    from fractions import Fraction
    tokens = int(N) * int(H) * int(W)
    smax = max(1, min(MAX_PARTIALS, -(-tokens // 1024)))
    tiles = 3 * int(K) * (-(-int(C) // 16)) * (-(-int(C) // 64))
    return min(range(1, smax + 1), key=lambda S: (Fraction(-(-S * tiles // _CUS), S), -S))


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DTYPES[t.dtype]


def _check(fn, status):
    if status != 0:
        raise DDPMError(fn, status)


def ddpm_filter_fwd(x, taps, out, K, stream=None):
    """out = [x, d1, d3, d5] from materialised taps (see include/ddpm.h)."""
    N, C, H, W = x.shape
    R = 3 * C * K * K
    dt = x.dtype
    args = (_dev(x, "x", dt), _dev(taps, "taps", dt, (N, R, H, W)), _dev(out, "out", dt, (N, 4 * C, H, W)))
    _check("ddpm_filter_fwd", _load().ddpm_filter_fwd(*args, N, C, H, W, K, _dtype_code(x), _stream(stream)))


def ddpm_filter_bwd(x, taps, grad_out, grad_x, grad_taps, K, stream=None):
    """grad_x and / or grad_taps of the materialised filter (see include/ddpm.h);
    either output may be None to skip it."""
    N, C, H, W = x.shape
    R = 3 * C * K * K
    dt = x.dtype
    null = ctypes.c_void_p(None)
    args = (_dev(x, "x", dt), _dev(taps, "taps", dt, (N, R, H, W)),
            _dev(grad_out, "grad_out", dt, (N, 4 * C, H, W)),
            null if grad_x is None else _dev(grad_x, "grad_x", dt, (N, C, H, W)),
            null if grad_taps is None else _dev(grad_taps, "grad_taps", dt, (N, R, H, W)))
    _check("ddpm_filter_bwd", _load().ddpm_filter_bwd(*args, N, C, H, W, K, _dtype_code(x), _stream(stream)))


def ddpm_fused_fwd(x, y, weight, bias, out, K, stream=None):
    """out = [x, d1, d3, d5] with the 1x1 generator fused in (see include/ddpm.h)."""
    N, C, H, W = x.shape
    R = 3 * C * K * K
    dt = x.dtype
    args = (_dev(x, "x", dt), _dev(y, "y", dt, (N, C, H, W)), _dev(weight, "weight", dt, (R, C)),
            _dev(bias, "bias", dt, (R,)), _dev(out, "out", dt, (N, 4 * C, H, W)))
    _check("ddpm_fused_fwd", _load().ddpm_fused_fwd(*args, N, C, H, W, K, _dtype_code(x), _stream(stream)))


def ddpm_fused_bwd(x, y, weight, bias, grad_out, grad_x, grad_y, dweight_partials, dbias_partials, K,
                   stream=None):
    """grad_x, grad_y and the float32 weight/bias partials (see include/ddpm.h).

    grad_x, grad_y, or both partial tensors may be None to skip that part."""
    N, C, H, W = x.shape
    R = 3 * C * K * K
    dt = x.dtype
    if (dweight_partials is None) != (dbias_partials is None):
        raise ValueError("dweight_partials and dbias_partials must both be given or both be None")
    S = dweight_partials.shape[0] if dweight_partials is not None else 0
    null = ctypes.c_void_p(None)
    args = (_dev(x, "x", dt), _dev(y, "y", dt, (N, C, H, W)), _dev(weight, "weight", dt, (R, C)),
            _dev(bias, "bias", dt, (R,)), _dev(grad_out, "grad_out", dt, (N, 4 * C, H, W)),
            null if grad_x is None else _dev(grad_x, "grad_x", dt, (N, C, H, W)),
            null if grad_y is None else _dev(grad_y, "grad_y", dt, (N, C, H, W)),
            null if dweight_partials is None else
            _dev(dweight_partials, "dweight_partials", torch.float32, (S, R, C)),
            null if dbias_partials is None else _dev(dbias_partials, "dbias_partials", torch.float32, (S, R)))
    _check("ddpm_fused_bwd",
           _load().ddpm_fused_bwd(*args, S, N, C, H, W, K, _dtype_code(x), _stream(stream)))


def ddpm_reduce_partials(dweight_partials, dbias_partials, grad_weight, grad_bias, K, stream=None):
    """grad_weight, grad_bias = fixed-order float32 sums of the partials, in the parameter dtype."""
    S, R, C = dweight_partials.shape
    if R != 3 * C * K * K:
        raise ValueError(f"dweight_partials rows {R} != 3*C*K*K = {3 * C * K * K}")
    dt = grad_weight.dtype
    args = (_dev(dweight_partials, "dweight_partials", torch.float32),
            _dev(dbias_partials, "dbias_partials", torch.float32, (S, R)))
    outs = (_dev(grad_weight, "grad_weight", dt, (R, C)), _dev(grad_bias, "grad_bias", dt, (R,)))
    _check("ddpm_reduce_partials",
           _load().ddpm_reduce_partials(*args, S, *outs, C, K, _dtype_code(grad_weight), _stream(stream)))


def ddpm_fused_bwd_noalloc(x, y, weight, bias, grad_out, grad_x, grad_y, grad_weight, grad_bias, K,
                           num_partials=None, stream=None):
    """grad_x, grad_y, grad_weight and grad_bias with the float32 partials kept in the
    library's fixed device buffer: no workspace, nothing allocated (see include/ddpm.h).

    grad_x or grad_y may be None; grad_weight and grad_bias are both given or both
    None.  num_partials defaults to num_partials_for(N, C, H, W, K)."""
    N, C, H, W = x.shape
    R = 3 * C * K * K
    dt = x.dtype
    if (grad_weight is None) != (grad_bias is None):
        raise ValueError("grad_weight and grad_bias must both be given or both be None")
    S = num_partials_for(N, C, H, W, K) if num_partials is None else int(num_partials)
    null = ctypes.c_void_p(None)
    args = (_dev(x, "x", dt), _dev(y, "y", dt, (N, C, H, W)), _dev(weight, "weight", dt, (R, C)),
            _dev(bias, "bias", dt, (R,)), _dev(grad_out, "grad_out", dt, (N, 4 * C, H, W)),
            null if grad_x is None else _dev(grad_x, "grad_x", dt, (N, C, H, W)),
            null if grad_y is None else _dev(grad_y, "grad_y", dt, (N, C, H, W)),
            null if grad_weight is None else _dev(grad_weight, "grad_weight", dt, (R, C)),
            null if grad_bias is None else _dev(grad_bias, "grad_bias", dt, (R,)))
    _check("ddpm_fused_bwd_noalloc",
           _load().ddpm_fused_bwd_noalloc(*args, S, N, C, H, W, K, _dtype_code(x), _stream(stream)))
