"""fp64 CPU oracle for the Dynamic Dilated Pyramid Module (DDPM).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the ``smoke()`` check of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import this
package.  The HIP library never imports, links or calls it, and it shares no code
with the HIP library.

The arithmetic lives in ``ddpm_oracle.c`` (plain C loops, double accumulation);
this module only marshals numpy arrays into it.  What is computed follows the page
"lartpang/DynamicConvolutionOperator" (DDPM from HDFNet, ECCV 2020): the unfold
definition named there as the mathematical reference ("Dynamic Convolution
Operator" intro, "问题与目标"), the dilation set (1, 3, 5) and the output order
[x, d1, d3, d5] and the filter's dX / dK backward ("CUDA 动态过滤"), the 1x1 generator ("CUDA 融合生成器推理") and the
training adjoints ("CUDA Flash 式融合训练").

Every function takes and returns float64 arrays in NCHW layout:
  x, y [N,C,H,W]; Wg [3*C*K*K, C]; bg [3*C*K*K]; taps [N,3*C*K*K,H,W];
  out and grad_out [N,4*C,H,W].
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ddpm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Plain, portable flags: no -ffast-math, no -march=native (the library is built on
# one host and may run on another).
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared"]


def build(src=_SRC, out=_LIB, extra_flags=()):
    """Compile the oracle C source into a shared library with gcc."""
    cmd = ["gcc", *CFLAGS, *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


def load(path=_LIB):
    """Load an oracle shared library (built from ddpm_oracle.c or a test variant)."""
    if path == _LIB and not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    lib.ddpm_oracle_generator.argtypes = [_D, _D, _D, _D, _I64, _I64, _I64, _I64, ctypes.c_int]
    lib.ddpm_oracle_filter_fwd.argtypes = [_D, _D, _D, _I64, _I64, _I64, _I64, ctypes.c_int]
    lib.ddpm_oracle_fused_fwd.argtypes = [_D, _D, _D, _D, _D, _I64, _I64, _I64, _I64, ctypes.c_int]
    lib.ddpm_oracle_fused_bwd.argtypes = [_D] * 9 + [_I64, _I64, _I64, _I64, ctypes.c_int]
    lib.ddpm_oracle_sum_partials.argtypes = [_D, _D, _I64, _I64]
    lib.ddpm_oracle_filter_bwd.argtypes = [_D] * 5 + [_I64, _I64, _I64, _I64, ctypes.c_int]
    for f in ("ddpm_oracle_generator", "ddpm_oracle_filter_fwd", "ddpm_oracle_fused_fwd",
              "ddpm_oracle_fused_bwd", "ddpm_oracle_sum_partials", "ddpm_oracle_filter_bwd"):
        getattr(lib, f).restype = None
    return lib


_lib = None


def _default():
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


def _arr(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    return a


def _p(a):
    return a.ctypes.data_as(_D)


class Oracle:
    """numpy-level wrappers over one loaded oracle library."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else _default()

    def generator(self, y, Wg, bg, K):
        y, Wg, bg = _arr(y), _arr(Wg), _arr(bg)
        N, C, H, W = y.shape
        R = 3 * C * K * K
        assert Wg.shape == (R, C) and bg.shape == (R,)
        taps = np.empty((N, R, H, W), dtype=np.float64)
        self.lib.ddpm_oracle_generator(_p(y), _p(Wg), _p(bg), _p(taps), N, C, H, W, K)
        return taps

    def filter_fwd(self, x, taps, K):
        x, taps = _arr(x), _arr(taps)
        N, C, H, W = x.shape
        assert taps.shape == (N, 3 * C * K * K, H, W)
        out = np.empty((N, 4 * C, H, W), dtype=np.float64)
        self.lib.ddpm_oracle_filter_fwd(_p(x), _p(taps), _p(out), N, C, H, W, K)
        return out

    def fused_fwd(self, x, y, Wg, bg, K):
        x, y, Wg, bg = _arr(x), _arr(y), _arr(Wg), _arr(bg)
        N, C, H, W = x.shape
        R = 3 * C * K * K
        assert y.shape == x.shape and Wg.shape == (R, C) and bg.shape == (R,)
        out = np.empty((N, 4 * C, H, W), dtype=np.float64)
        self.lib.ddpm_oracle_fused_fwd(_p(x), _p(y), _p(Wg), _p(bg), _p(out), N, C, H, W, K)
        return out

    def fused_bwd(self, x, y, Wg, bg, G, K):
        """Returns (dx, dy, dWg, dbg) for L = <G, fused_fwd(x, y, Wg, bg)>."""
        x, y, Wg, bg, G = _arr(x), _arr(y), _arr(Wg), _arr(bg), _arr(G)
        N, C, H, W = x.shape
        R = 3 * C * K * K
        assert G.shape == (N, 4 * C, H, W)
        dx = np.empty_like(x)
        dy = np.empty_like(y)
        dWg = np.empty((R, C), dtype=np.float64)
        dbg = np.empty((R,), dtype=np.float64)
        self.lib.ddpm_oracle_fused_bwd(_p(x), _p(y), _p(Wg), _p(bg), _p(G), _p(dx), _p(dy),
                                       _p(dWg), _p(dbg), N, C, H, W, K)
        return dx, dy, dWg, dbg

    def filter_bwd(self, x, taps, G, K):
        """Returns (dx, dtaps) for L = <G, filter_fwd(x, taps)>."""
        x, taps, G = _arr(x), _arr(taps), _arr(G)
        N, C, H, W = x.shape
        assert taps.shape == (N, 3 * C * K * K, H, W) and G.shape == (N, 4 * C, H, W)
        dx = np.empty_like(x)
        dtaps = np.empty_like(taps)
        self.lib.ddpm_oracle_filter_bwd(_p(x), _p(taps), _p(G), _p(dx), _p(dtaps), N, C, H, W, K)
        return dx, dtaps

    def sum_partials(self, partials):
        partials = _arr(partials)
        S = partials.shape[0]
        M = int(np.prod(partials.shape[1:]))
        out = np.empty(partials.shape[1:], dtype=np.float64)
        self.lib.ddpm_oracle_sum_partials(_p(partials), _p(out), S, M)
        return out


def default():
    return Oracle()
