"""GPU parity of the DDPM module (both paths) against an fp64 composition.

Expected values: the oracle's fused forward / backward (fp64, CPU) for
[x, d1, d3, d5], composed with a float64 CPU torch convolution for the 3x3 fuse
layer and its adjoint.  The module runs the library's kernels (fused or
materialised path) plus torch's GPU convolutions, so this checks the autograd
wiring, the dispatch and the weight layout (generator row o = (b*C + c)*K^2 + t
as a [3CK^2, C, 1, 1] conv weight) end to end.
"""
import pytest
import torch
import torch.nn.functional as F

from dynamic_dilated_depthwise_amd import synth
from dynamic_dilated_depthwise_amd.module import DDPM
from gpu_cases import TOL, announce, assert_close, f64, orc

pytestmark = pytest.mark.gpu
S_ = synth.Shape

SHAPES = [("nonaligned", S_(2, 24, 15, 17, 3), 401), ("c64_32x40", S_(1, 64, 32, 40, 3), 402),
          ("k5", S_(1, 16, 12, 13, 5), 403), ("k1", S_(1, 8, 9, 10, 1), 404)]
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _module(shape, dtype, seed, **kw):
    torch.manual_seed(seed)
    m = DDPM(dim=shape.C, kernel_size=shape.K, **kw)
    return m.to(device="cuda", dtype=dtype)


def _reference(m, x, y, gout, K):
    """fp64 module forward and gradients (x, y, generator weight/bias, fuse weight/bias)."""
    R = 3 * m.dim * K * K
    W = f64(m.generator.weight).reshape(R, m.dim)
    b = f64(m.generator.bias)
    xs, ys = f64(x), f64(y)
    feats = orc().fused_fwd(xs, ys, W, b, K)
    fw = m.fuse.weight.detach().cpu().double().requires_grad_(True)
    fb = m.fuse.bias.detach().cpu().double().requires_grad_(True)
    ft = torch.from_numpy(feats).requires_grad_(True)
    out = F.conv2d(ft, fw, fb, padding=1)
    if gout is None:
        return out.detach().numpy(), None
    out.backward(torch.from_numpy(f64(gout)))
    G = ft.grad.numpy()
    dx, dy, dW, db = orc().fused_bwd(xs, ys, W, b, G, K)
    grads = {"x": dx, "y": dy, "gen_w": dW.reshape(R, m.dim, 1, 1), "gen_b": db,
             "fuse_w": fw.grad.numpy(), "fuse_b": fb.grad.numpy()}
    return out.detach().numpy(), grads


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("name,shape,seed", SHAPES, ids=[s[0] for s in SHAPES])
def test_inference(name, shape, seed, dt):
    dtype = DT[dt]
    m = _module(shape, dtype, seed, fused_generator_inference=True)
    h = synth.make_inputs(shape, seed, dtype)
    x, y = h["x"].cuda(), h["y"].cuda()
    announce("module inference", name, dt, shape)
    with torch.no_grad():
        out = m(x, y)
    assert m.last_path == "fused"
    ref, _ = _reference(m, x, y, None, shape.K)
    assert_close(f64(out), ref, TOL[dtype]["out"], f"module out {name} {dt}")


@pytest.mark.parametrize("path", ["fused", "materialised"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("name,shape,seed", SHAPES, ids=[s[0] for s in SHAPES])
def test_training(name, shape, seed, dt, path):
    dtype = DT[dt]
    m = _module(shape, dtype, seed, fused_generator_training=(path == "fused"))
    h = synth.make_inputs(shape, seed, dtype)
    x = h["x"].cuda().requires_grad_(True)
    y = h["y"].cuda().requires_grad_(True)
    gout = torch.randn((shape.N, shape.C, shape.H, shape.W), generator=torch.Generator().manual_seed(seed)).to(
        dtype).cuda()
    announce("module training", path, name, dt, shape)
    out = m(x, y)
    assert m.last_path == path
    out.backward(gout)
    ref, grads = _reference(m, x, y, gout, shape.K)
    tol = TOL[dtype]
    assert_close(f64(out), ref, tol["out"], f"module out {path} {name} {dt}")
    got = {"x": x.grad, "y": y.grad, "gen_w": m.generator.weight.grad, "gen_b": m.generator.bias.grad,
           "fuse_w": m.fuse.weight.grad, "fuse_b": m.fuse.bias.grad}
    for k, g in got.items():
        assert_close(f64(g), grads[k], tol["grad"], f"d{k} {path} {name} {dt}")


def test_auto_and_mismatch_paths():
    """Automatic mode follows the measured thresholds (K=3 trains fused at every
    size, fp32 K=5 below 96^2 materialised); a dtype mismatch takes the
    materialised path and computes in the generator's dtype."""
    shape, seed = S_(1, 16, 10, 12, 5), 405
    sb = S_(1, 16, 32, 40, 3)  # 1280 tokens
    mb = _module(sb, torch.bfloat16, seed)
    hb = synth.make_inputs(sb, seed, torch.bfloat16)
    announce("module auto/mismatch", shape, sb)
    mb(hb["x"].cuda().requires_grad_(True), hb["y"].cuda())
    assert mb.last_path == "fused"
    m = _module(shape, torch.float32, seed)
    h = synth.make_inputs(shape, seed, torch.float32)
    x = h["x"].cuda().requires_grad_(True)
    y = h["y"].cuda()
    out = m(x, y)
    assert m.last_path == "materialised"
    ref, _ = _reference(m, x, y, None, shape.K)
    assert_close(f64(out), ref, TOL[torch.float32]["out"], "auto materialised")
    xb = x.detach().to(torch.bfloat16)
    with torch.no_grad():
        out_b = m(xb, y)
    assert m.last_path == "materialised" and out_b.dtype == torch.float32
    ref_b, _ = _reference(m, xb.float(), y, None, shape.K)
    assert_close(f64(out_b), ref_b, TOL[torch.float32]["out"], "mismatch materialised")


def test_autocast_bf16():
    """Under autocast the generator runs in bfloat16 (torch) and the library filters
    in bfloat16; the result stays within the bfloat16 tolerance of fp64."""
    shape, seed = S_(1, 16, 10, 12, 3), 406
    m = _module(shape, torch.float32, seed)
    h = synth.make_inputs(shape, seed, torch.float32)
    x = h["x"].cuda().requires_grad_(True)
    y = h["y"].cuda().requires_grad_(True)
    announce("module autocast", shape)
    with torch.autocast("cuda", dtype=torch.bfloat16):
        out = m(x, y)
    assert m.last_path == "materialised"
    out.float().sum().backward()
    ref, _ = _reference(m, x, y, None, shape.K)
    assert_close(f64(out), ref, TOL[torch.bfloat16]["out"], "autocast out")
    assert x.grad is not None and y.grad is not None and m.generator.weight.grad is not None


def test_autocast_fp16():
    """Under torch's default CUDA autocast (float16) the generator makes float16
    taps; the library takes float32 and bfloat16, so the materialised path widens
    the taps and x to float32 (exactly) and filters in float32.  Forward and the
    backward into every input run, within the bfloat16 bound of fp64 (float16
    taps carry 2^-11 relative rounding)."""
    shape, seed = S_(1, 16, 10, 12, 3), 407
    m = _module(shape, torch.float32, seed)
    h = synth.make_inputs(shape, seed, torch.float32)
    x = h["x"].cuda().requires_grad_(True)
    y = h["y"].cuda().requires_grad_(True)
    announce("module autocast fp16", shape)
    with torch.autocast("cuda"):
        out = m(x, y)
        feats = m.dynamic_filter(x, y)
    assert m.last_path == "materialised" and feats.dtype == torch.float32
    out.float().sum().backward()
    ref, _ = _reference(m, x, y, None, shape.K)
    assert_close(f64(out), ref, TOL[torch.bfloat16]["out"], "autocast fp16 out")
    assert x.grad is not None and y.grad is not None and m.generator.weight.grad is not None
    assert torch.isfinite(x.grad).all() and torch.isfinite(m.generator.weight.grad).all()
