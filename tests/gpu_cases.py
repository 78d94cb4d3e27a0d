"""Helpers for the GPU parity tests: run the HIP path through the binding and the
fp64 oracle on the same seeded inputs, and compare.

Tolerances (error = max|gpu - oracle| / max|oracle|, per tensor):
  float32   outputs 2e-4, gradients 1e-3
  bfloat16  outputs and gradients 2e-2
The x block of every forward output must equal x bit for bit, and so must every
element of the materialised-filter tap gradient (one product of two inputs, exact
in fp64 and rounded once on either side).
"""
import sys

import numpy as np
import torch

import dynamic_dilated_depthwise_amd as ddpm
import oracle
from dynamic_dilated_depthwise_amd import synth

TOL = {
    torch.float32: {"out": 2e-4, "grad": 1e-3},
    torch.bfloat16: {"out": 2e-2, "grad": 2e-2},
}


def announce(*parts):
    print("[gpu case]", *parts, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = max(float(np.abs(ref).max()), 1e-30)
    return float(np.abs(got - ref).max()) / scale


def assert_close(got, ref, tol, what):
    err = rel_err(got, ref)
    assert err <= tol, f"{what}: rel err {err:.3e} > {tol:.1e}"
    return err


_orc = None


def orc():
    global _orc
    if _orc is None:
        _orc = oracle.default()
    return _orc


def inputs(shape, block, dtype, **kw):
    return synth.make_inputs(shape, block, dtype, **kw)


def dev(d):
    return {k: v.to("cuda").contiguous() for k, v in d.items()}


def gpu_filter(d, K):
    x, taps = d["x"], d["taps"]
    N, C, H, W = x.shape
    out = torch.empty((N, 4 * C, H, W), device="cuda", dtype=x.dtype)
    ddpm.ddpm_filter_fwd(x, taps, out, K)
    torch.cuda.synchronize()
    return out


def gpu_fused(d, K):
    x = d["x"]
    N, C, H, W = x.shape
    out = torch.empty((N, 4 * C, H, W), device="cuda", dtype=x.dtype)
    ddpm.ddpm_fused_fwd(x, d["y"], d["weight"], d["bias"], out, K)
    torch.cuda.synchronize()
    return out


def gpu_bwd(d, K, S=None):
    x = d["x"]
    N, C, H, W = x.shape
    R = 3 * C * K * K
    S = ddpm.num_partials_for(N, C, H, W, K) if S is None else S
    gx = torch.empty_like(x)
    gy = torch.empty_like(x)
    pw = torch.empty((S, R, C), device="cuda", dtype=torch.float32)
    pb = torch.empty((S, R), device="cuda", dtype=torch.float32)
    ddpm.ddpm_fused_bwd(x, d["y"], d["weight"], d["bias"], d["grad_out"], gx, gy, pw, pb, K)
    gw = torch.empty((R, C), device="cuda", dtype=x.dtype)
    gb = torch.empty((R,), device="cuda", dtype=x.dtype)
    ddpm.ddpm_reduce_partials(pw, pb, gw, gb, K)
    torch.cuda.synchronize()
    return gx, gy, gw, gb, pw, pb


def gpu_filter_bwd(d, K, want_dx=True, want_dk=True):
    x, taps = d["x"], d["taps"]
    gx = torch.empty_like(x) if want_dx else None
    gk = torch.empty_like(taps) if want_dk else None
    ddpm.ddpm_filter_bwd(x, taps, d["grad_out"], gx, gk, K)
    torch.cuda.synchronize()
    return gx, gk
