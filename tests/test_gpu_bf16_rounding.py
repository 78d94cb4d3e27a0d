"""bf16 tap quantisation, checked bit for bit on the GPU.

The page quantises the taps to bfloat16 before they are used ("CUDA Flash 式融合训练",
precision paragraph); the reading taken here rounds each tap once, round to nearest
even, after the fp32 generator sum plus bias, and rounds every bf16 output once.
With K = 1 and one channel every step is either exact in fp32 (a product of two
bf16 values) or one fp32 addition in a fixed order, so a few lines of numpy with an
explicit bf16 rounding predict the kernels' outputs exactly:
  fused forward   out_b = rne(rne(W_b y + b_b) x)
  fused dX        dX = rne(((0 + q_0 G_0) + q_1 G_1) + q_2 G_2 + G_x),  q_b = rne(W_b y + b_b)
  fused dY        dY = rne(sum_b W_b rne(G_b x))   (dK rounded as the MFMA operand)
The same model without the tap rounding must differ somewhere, so the test tells the
two readings apart.
"""
import numpy as np
import pytest
import torch

import dynamic_dilated_depthwise_amd as ddpm

pytestmark = pytest.mark.gpu


def _rne_bits(a):
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bits_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def _rne(a):
    return _bits_f32(_rne_bits(a))


def _draw(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


def _case(seed):
    H, W = 9, 70
    x = _draw((1, 1, H, W), seed)
    y = _draw((1, 1, H, W), seed + 1)
    w = _draw((3, 1), seed + 2)
    b = _draw((3,), seed + 3, 0.3)
    gout = _draw((1, 4, H, W), seed + 4)
    f = lambda t: t.float().numpy()
    return x, y, w, b, gout, f(x)[0, 0], f(y)[0, 0], f(w)[:, 0], f(b), f(gout)[0]


def _taps(yv, wv, bv, quantise):
    T = [np.float32(wv[k]) * yv + np.float32(bv[k]) for k in range(3)]  # product exact, one rounding
    T = [t.astype(np.float32) for t in T]
    return [_rne(t) for t in T] if quantise else T


@pytest.mark.parametrize("seed", [11, 12])
def test_fused_forward_rounds_taps(seed):
    x, y, w, b, _, xv, yv, wv, bv, _ = _case(seed)
    out = torch.empty((1, 4, *x.shape[2:]), device="cuda", dtype=torch.bfloat16)
    ddpm.ddpm_fused_fwd(x.cuda(), y.cuda(), w.cuda(), b.cuda(), out, 1)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    want = [_rne_bits((q * xv).astype(np.float32)) for q in _taps(yv, wv, bv, True)]
    plain = [_rne_bits((t * xv).astype(np.float32)) for t in _taps(yv, wv, bv, False)]
    for k in range(3):
        assert np.array_equal(got[0, 1 + k], want[k]), f"branch {k}: not rne(rne(T) x)"
    assert any(not np.array_equal(want[k], plain[k]) for k in range(3)), "case does not separate the readings"


@pytest.mark.parametrize("seed", [21, 22])
def test_fused_dx_rounds_taps(seed):
    x, y, w, b, gout, xv, yv, wv, bv, gv = _case(seed)
    gx = torch.empty_like(x, device="cuda")
    ddpm.ddpm_fused_bwd(x.cuda(), y.cuda(), w.cuda(), b.cuda(), gout.cuda(), gx, None, None, None, 1)
    torch.cuda.synchronize()
    got = gx.cpu().view(torch.int16).numpy().view(np.uint16)[0, 0]

    def model(quantise):
        q = _taps(yv, wv, bv, quantise)
        acc = np.zeros_like(xv, dtype=np.float32)
        for k in range(3):
            acc = (acc + (q[k] * gv[1 + k]).astype(np.float32)).astype(np.float32)
        return _rne_bits((acc + gv[0]).astype(np.float32))

    assert np.array_equal(got, model(True)), "dX is not the sum of rounded taps times G"
    assert not np.array_equal(model(True), model(False)), "case does not separate the readings"


def _grid_values(shape, seed):
    """bf16 values 1 + k/128, k in 0..3: products and sums of a few dozen of them are
    exact in fp32 whatever the summation order."""
    g = torch.Generator().manual_seed(seed)
    k = torch.randint(0, 4, shape, generator=g).float()
    return (1.0 + k / 128.0).to(torch.bfloat16)


@pytest.mark.parametrize("seed", [31, 32])
def test_weight_gradient_rounds_dk_bias_gradient_does_not(seed):
    """dW sums rne(dK) * y (dK is a bf16 MFMA operand), db sums the fp32 dK unrounded;
    with K = 1, dK_b = G_b * x at the same pixel."""
    H, W = 4, 6
    x = _grid_values((1, 1, H, W), seed)
    y = _grid_values((1, 1, H, W), seed + 1)
    gout = _grid_values((1, 4, H, W), seed + 2)
    w = _draw((3, 1), seed + 3)
    b = _draw((3,), seed + 4, 0.3)
    pw = torch.empty((1, 3, 1), device="cuda", dtype=torch.float32)
    pb = torch.empty((1, 3), device="cuda", dtype=torch.float32)
    ddpm.ddpm_fused_bwd(x.cuda(), y.cuda(), w.cuda(), b.cuda(), gout.cuda(), None, None, pw, pb, 1)
    torch.cuda.synchronize()
    xv, yv, gv = x.float().numpy()[0, 0], y.float().numpy()[0, 0], gout.float().numpy()[0]
    for k in range(3):
        dk = (gv[1 + k] * xv).astype(np.float32)  # exact
        want_w = np.float32(np.sum(_rne(dk).astype(np.float64) * yv))  # every partial sum exact
        want_b = np.float32(np.sum(dk.astype(np.float64)))
        other_w = np.float32(np.sum(dk.astype(np.float64) * yv))
        other_b = np.float32(np.sum(_rne(dk).astype(np.float64)))
        assert pw[0, k, 0].item() == want_w, f"dW row {k}: {pw[0, k, 0].item()!r} != {want_w!r}"
        assert pb[0, k].item() == want_b, f"db row {k}: {pb[0, k].item()!r} != {want_b!r}"
        assert want_w != other_w and want_b != other_b, "case does not separate the readings"


@pytest.mark.parametrize("seed", [33, 34])
def test_weight_gradient_rounding_c64(seed):
    """The same two readings at C = 64 (the segment-staged partial kernel): with
    K = 1, dW[(b, c), c'] = sum_p rne(G_b[c, p] x[c, p]) y[c', p] and
    db[(b, c)] = sum_p G_b[c, p] x[c, p], over 2 x 16 pixels.  The grid values keep
    every product and partial sum exact in float32 whatever the summation order."""
    C, H, W = 64, 2, 16
    x = _grid_values((1, C, H, W), seed)
    y = _grid_values((1, C, H, W), seed + 1)
    gout = _grid_values((1, 4 * C, H, W), seed + 2)
    w = _draw((3 * C, C), seed + 3, 0.1)
    b = _draw((3 * C,), seed + 4, 0.3)
    pw = torch.empty((1, 3 * C, C), device="cuda", dtype=torch.float32)
    pb = torch.empty((1, 3 * C), device="cuda", dtype=torch.float32)
    ddpm.ddpm_fused_bwd(x.cuda(), y.cuda(), w.cuda(), b.cuda(), gout.cuda(), None, None, pw, pb, 1)
    torch.cuda.synchronize()
    xv = x.float().numpy()[0].reshape(C, -1)
    yv = y.float().numpy()[0].reshape(C, -1).astype(np.float64)
    gv = gout.float().numpy()[0].reshape(4 * C, -1)
    got_w, got_b = pw[0].cpu().numpy(), pb[0].cpu().numpy()
    separated_w = separated_b = False
    for k in range(3):
        dk = (gv[(1 + k) * C:(2 + k) * C] * xv).astype(np.float32)  # exact, [c, p]
        want_w = (_rne(dk).astype(np.float64) @ yv.T).astype(np.float32)  # [c, c']
        want_b = dk.astype(np.float64).sum(1).astype(np.float32)
        other_w = (dk.astype(np.float64) @ yv.T).astype(np.float32)
        other_b = _rne(dk).astype(np.float64).sum(1).astype(np.float32)
        bad_w = int((got_w[k * C:(k + 1) * C] != want_w).sum())
        bad_b = int((got_b[k * C:(k + 1) * C] != want_b).sum())
        assert bad_w == 0, f"branch {k}: {bad_w} dW elements differ from sum rne(dK) y"
        assert bad_b == 0, f"branch {k}: {bad_b} db elements differ from sum dK"
        separated_w = separated_w or bool((want_w != other_w).any())
        separated_b = separated_b or bool((want_b != other_b).any())
    assert separated_w and separated_b, "case does not separate the readings"


@pytest.mark.parametrize("seed", [41, 42])
def test_fused_dy_rounds_dk(seed):
    """dY = W^T rne(dK): with K = 1 and one channel, dY = rne(sum_b W_b rne(G_b x)).
    W = (1, -1, 0) and G_1 one bfloat16 step above G_0 make the two branch terms
    nearly cancel: the exact dK difference G_0 x - G_1 x is then far below one
    bfloat16 step of dK, so rounding dK first or not gives different outputs.
    Every sum is exact in float32 (differences of nearly equal values whose
    mantissas hold at most 16 bits), so the order of the MFMA sums does not matter."""
    H, W = 9, 70
    x = _draw((1, 1, H, W), seed)
    g0 = _draw((1, 1, H, W), seed + 1)
    g0_bits = g0.view(torch.int16)
    g1 = (g0_bits + 1).view(torch.bfloat16)  # next bfloat16 value away from zero
    g2 = _draw((1, 1, H, W), seed + 2)
    gx_blk = _draw((1, 1, H, W), seed + 3)
    gout = torch.cat([gx_blk, g0, g1, g2], dim=1).contiguous()
    w = torch.tensor([[1.0], [-1.0], [0.0]]).to(torch.bfloat16)
    y = _draw((1, 1, H, W), seed + 4)
    b = _draw((3,), seed + 5, 0.3)
    gy = torch.empty_like(x, device="cuda")
    ddpm.ddpm_fused_bwd(x.cuda(), y.cuda(), w.cuda(), b.cuda(), gout.cuda(), None, gy, None, None, 1)
    torch.cuda.synchronize()
    got = gy.cpu().view(torch.int16).numpy().view(np.uint16)[0, 0]
    xv = x.float().numpy()[0, 0]
    gv = gout.float().numpy()[0]
    wv = w.float().numpy()[:, 0]

    def model(round_dk):
        acc = np.zeros_like(xv, dtype=np.float64)
        for k in range(3):
            dk = (gv[1 + k] * xv).astype(np.float32)  # exact product of two bf16 values
            q = _rne(dk) if round_dk else dk
            acc += np.float64(wv[k]) * q.astype(np.float64)
        assert np.array_equal(acc.astype(np.float32).astype(np.float64), acc), "sum not exact in float32"
        return _rne_bits(acc.astype(np.float32))

    assert np.array_equal(got, model(True)), "dY is not W^T rne(dK)"
    assert not np.array_equal(model(True), model(False)), "case does not separate the readings"
