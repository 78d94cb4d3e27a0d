"""Pins for the fp64 oracle: checks against facts fixed by the page and by mathematics.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises ``AssertionError``
when the oracle disagrees with something other than itself:

* an independent numpy brute force (explicit zero padding, einsum generator,
  slicing) -- a different index convention from the oracle's bounds tests;
* the page's own reference construction, three ``Unfold`` patch tensors times the
  generator output ("Dynamic Convolution Operator" intro and "问题与目标"), built
  from torch's ``F.unfold`` / ``F.conv2d`` in float64;
* special cases that reduce to textbook operators: a zero generator weight gives
  an ordinary dilated depthwise convolution (torch ``conv2d`` with groups=C); a
  one-hot centre tap reproduces x; K=1 reduces to x * (Wg y + bg);
* the closed-form count of in-image neighbours when x, the taps and the bias are
  all ones;
* invariants: linearity in x, affinity in y, the x block equal to x;
* gradients: central finite differences, which are exact here because the loss
  <G, out> is affine in each of x, y, Wg and bg taken alone; the adjoint
  (dot-product) identity for dX; and torch autograd through the unfold
  construction in float64.

The same functions run against deliberately broken copies of the oracle in
``test_oracle_mutants.py`` to show that each plausible mistake is caught.
"""
import numpy as np
import torch
import torch.nn.functional as F

DILATIONS = (1, 3, 5)


def _rand_case(rng, N, C, H, W, K, w_scale=None, b_scale=0.1):
    R = 3 * C * K * K
    w_scale = (1.0 / np.sqrt(C)) if w_scale is None else w_scale
    x = rng.standard_normal((N, C, H, W))
    y = rng.standard_normal((N, C, H, W))
    Wg = rng.standard_normal((R, C)) * w_scale
    bg = rng.standard_normal(R) * b_scale
    return x, y, Wg, bg


def _close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(np.abs(b).max(), 1e-300)
    err = np.abs(a - b).max() / scale
    assert err <= rtol, f"{what}: rel err {err:.3e} > {rtol:.1e}"


# ----------------------------------------------------------------------------- references
def numpy_brute_fwd(x, y, Wg, bg, K):
    """Zero-pad x by the largest reach, materialise the generator, slice per tap."""
    N, C, H, W = x.shape
    r = (K - 1) // 2
    P = 5 * r
    xp = np.zeros((N, C, H + 2 * P, W + 2 * P))
    xp[:, :, P:P + H, P:P + W] = x
    T = np.einsum("oc,nchw->nohw", Wg, y) + bg[None, :, None, None]
    T = T.reshape(N, 3, C, K, K, H, W)
    out = np.zeros((N, 4, C, H, W))
    out[:, 0] = x
    for bi, D in enumerate(DILATIONS):
        for ki in range(K):
            for kj in range(K):
                dh, dw = (ki - r) * D, (kj - r) * D
                out[:, 1 + bi] += T[:, bi, :, ki, kj] * xp[:, :, P + dh:P + dh + H, P + dw:P + dw + W]
    return out.reshape(N, 4 * C, H, W)


def numpy_brute_filter(x, taps, K):
    N, C, H, W = x.shape
    r = (K - 1) // 2
    P = 5 * r
    xp = np.zeros((N, C, H + 2 * P, W + 2 * P))
    xp[:, :, P:P + H, P:P + W] = x
    T = taps.reshape(N, 3, C, K, K, H, W)
    out = np.zeros((N, 4, C, H, W))
    out[:, 0] = x
    for bi, D in enumerate(DILATIONS):
        for ki in range(K):
            for kj in range(K):
                dh, dw = (ki - r) * D, (kj - r) * D
                out[:, 1 + bi] += T[:, bi, :, ki, kj] * xp[:, :, P + dh:P + dh + H, P + dw:P + dw + W]
    return out.reshape(N, 4 * C, H, W)


def torch_unfold_fwd(x, y, Wg, bg, K):
    """The page's reference construction: 1x1 generator conv, three Unfold(x), multiply-sum."""
    N, C, H, W = x.shape
    R = 3 * C * K * K
    r = (K - 1) // 2
    T = F.conv2d(y, Wg.reshape(R, C, 1, 1), bg).reshape(N, 3, C, K * K, H, W)
    outs = [x]
    for bi, D in enumerate(DILATIONS):
        U = F.unfold(x, K, dilation=D, padding=D * r).reshape(N, C, K * K, H, W)
        outs.append((U * T[:, bi]).sum(2))
    return torch.cat(outs, 1)


# ----------------------------------------------------------------------------- pins
def pin_brute_force(o):
    rng = np.random.default_rng(11)
    for (N, C, H, W, K) in [(1, 8, 16, 16, 3), (2, 5, 15, 17, 3), (1, 3, 9, 7, 5), (2, 4, 6, 5, 1),
                            (1, 2, 1, 1, 3), (1, 2, 2, 13, 5)]:
        x, y, Wg, bg = _rand_case(rng, N, C, H, W, K)
        ref = numpy_brute_fwd(x, y, Wg, bg, K)
        _close(o.fused_fwd(x, y, Wg, bg, K), ref, 1e-13, f"fused_fwd brute {N,C,H,W,K}")
        taps = rng.standard_normal((N, 3 * C * K * K, H, W))
        _close(o.filter_fwd(x, taps, K), numpy_brute_filter(x, taps, K), 1e-13,
               f"filter_fwd brute {N,C,H,W,K}")


def pin_generator_einsum(o):
    rng = np.random.default_rng(12)
    for (N, C, H, W, K) in [(2, 6, 5, 7, 3), (1, 4, 3, 3, 5)]:
        x, y, Wg, bg = _rand_case(rng, N, C, H, W, K)
        ref = np.einsum("oc,nchw->nohw", Wg, y) + bg[None, :, None, None]
        _close(o.generator(y, Wg, bg, K), ref, 1e-13, "generator")


def pin_unfold_reference(o):
    rng = np.random.default_rng(13)
    for (N, C, H, W, K) in [(1, 8, 16, 16, 3), (2, 6, 15, 17, 3), (1, 3, 12, 11, 5)]:
        x, y, Wg, bg = _rand_case(rng, N, C, H, W, K)
        ref = torch_unfold_fwd(*(torch.from_numpy(a) for a in (x, y, Wg, bg)), K).numpy()
        _close(o.fused_fwd(x, y, Wg, bg, K), ref, 1e-12, f"unfold {N,C,H,W,K}")
        taps = o.generator(y, Wg, bg, K)
        _close(o.filter_fwd(x, taps, K), ref, 1e-12, f"filter(unfold) {N,C,H,W,K}")


def pin_zero_weight_is_dilated_depthwise_conv(o):
    rng = np.random.default_rng(14)
    for (N, C, H, W, K) in [(2, 5, 15, 17, 3), (1, 3, 13, 12, 5)]:
        x, y, Wg, bg = _rand_case(rng, N, C, H, W, K)
        Wg[:] = 0.0
        out = o.fused_fwd(x, y, Wg, bg, K)
        r = (K - 1) // 2
        xt = torch.from_numpy(x)
        for bi, D in enumerate(DILATIONS):
            w = torch.from_numpy(bg[bi * C * K * K:(bi + 1) * C * K * K].reshape(C, 1, K, K).copy())
            ref = F.conv2d(xt, w, dilation=D, padding=D * r, groups=C).numpy()
            _close(out[:, (1 + bi) * C:(2 + bi) * C], ref, 1e-13, f"depthwise conv d={D}")


def pin_one_hot_centre_tap(o):
    rng = np.random.default_rng(15)
    for (N, C, H, W, K) in [(1, 8, 16, 16, 3), (2, 3, 7, 9, 5), (1, 4, 5, 5, 1)]:
        x, y, Wg, bg = _rand_case(rng, N, C, H, W, K)
        Wg[:] = 0.0
        bg = np.zeros_like(bg)
        centre = (K * K - 1) // 2
        bg.reshape(3, C, K * K)[:, :, centre] = 1.0
        out = o.fused_fwd(x, y, Wg, bg, K)
        for b in range(4):
            _close(out[:, b * C:(b + 1) * C], x, 0.0, f"one-hot block {b}")


def pin_k1_is_x_times_generator(o):
    rng = np.random.default_rng(16)
    N, C, H, W, K = 2, 6, 5, 7, 1
    x, y, Wg, bg = _rand_case(rng, N, C, H, W, K)
    out = o.fused_fwd(x, y, Wg, bg, K)
    for bi in range(3):
        gen = np.einsum("oc,nchw->nohw", Wg[bi * C:(bi + 1) * C], y) + bg[bi * C:(bi + 1) * C, None, None]
        _close(out[:, (1 + bi) * C:(2 + bi) * C], x * gen, 1e-13, f"K=1 branch {bi}")


def _count_in_image(n_pos, K, D):
    r = (K - 1) // 2
    return np.array([sum(1 for k in range(K) if 0 <= i + (k - r) * D < n_pos) for i in range(n_pos)],
                    dtype=np.float64)


def pin_all_ones_border_count(o):
    for (N, C, H, W, K) in [(1, 2, 15, 17, 3), (1, 1, 16, 16, 5), (1, 2, 1, 1, 3), (1, 1, 4, 23, 5)]:
        R = 3 * C * K * K
        x = np.ones((N, C, H, W))
        y = np.zeros((N, C, H, W))
        Wg = np.zeros((R, C))
        bg = np.ones(R)
        out = o.fused_fwd(x, y, Wg, bg, K)
        for bi, D in enumerate(DILATIONS):
            ref = np.outer(_count_in_image(H, K, D), _count_in_image(W, K, D))
            for n in range(N):
                for c in range(C):
                    _close(out[n, (1 + bi) * C + c], ref, 0.0, f"count d={D} {H}x{W} K={K}")


def pin_linear_in_x_affine_in_y(o):
    rng = np.random.default_rng(17)
    N, C, H, W, K = 2, 5, 9, 11, 3
    x1, y1, Wg, bg = _rand_case(rng, N, C, H, W, K)
    x2, y2, _, _ = _rand_case(rng, N, C, H, W, K)
    a, b = 0.75, -1.25
    lhs = o.fused_fwd(a * x1 + b * x2, y1, Wg, bg, K)
    rhs = a * o.fused_fwd(x1, y1, Wg, bg, K) + b * o.fused_fwd(x2, y1, Wg, bg, K)
    _close(lhs, rhs, 1e-13, "linear in x")
    t = 0.3
    lhs = o.fused_fwd(x1, t * y1 + (1 - t) * y2, Wg, bg, K)
    rhs = t * o.fused_fwd(x1, y1, Wg, bg, K) + (1 - t) * o.fused_fwd(x1, y2, Wg, bg, K)
    _close(lhs, rhs, 1e-13, "affine in y")
    _close(lhs[:, :C], x1, 0.0, "x block")


def pin_finite_differences(o):
    rng = np.random.default_rng(18)
    for (N, C, H, W, K) in [(2, 4, 7, 9, 3), (1, 3, 12, 11, 5), (1, 3, 4, 5, 1)]:
        x, y, Wg, bg = _rand_case(rng, N, C, H, W, K)
        G = rng.standard_normal((N, 4 * C, H, W))
        grads = dict(zip(("x", "y", "Wg", "bg"), o.fused_bwd(x, y, Wg, bg, G, K)))
        args = dict(x=x, y=y, Wg=Wg, bg=bg)

        def loss(**kw):
            a = dict(args, **kw)
            return float((o.fused_fwd(a["x"], a["y"], a["Wg"], a["bg"], K) * G).sum())

        for name, val in args.items():
            v = rng.standard_normal(val.shape)
            h = 0.5
            fd = (loss(**{name: val + h * v}) - loss(**{name: val - h * v})) / (2 * h)
            an = float((grads[name] * v).sum())
            assert abs(fd - an) <= 1e-9 * max(abs(fd), 1.0), f"FD {name} {N,C,H,W,K}: {fd} vs {an}"


def pin_adjoint_dx(o):
    rng = np.random.default_rng(19)
    N, C, H, W, K = 2, 4, 10, 13, 3
    x, y, Wg, bg = _rand_case(rng, N, C, H, W, K)
    G = rng.standard_normal((N, 4 * C, H, W))
    dx, _, _, _ = o.fused_bwd(x, y, Wg, bg, G, K)
    v = rng.standard_normal(x.shape)
    lhs = float(((dx - G[:, :C]) * v).sum())
    rhs = float((G[:, C:] * o.fused_fwd(v, y, Wg, bg, K)[:, C:]).sum())
    assert abs(lhs - rhs) <= 1e-11 * max(abs(rhs), 1.0), f"adjoint {lhs} vs {rhs}"


def pin_autograd_unfold(o):
    rng = np.random.default_rng(20)
    for (N, C, H, W, K) in [(2, 6, 15, 17, 3), (1, 3, 9, 8, 5), (1, 8, 16, 16, 3)]:
        x, y, Wg, bg = _rand_case(rng, N, C, H, W, K)
        G = rng.standard_normal((N, 4 * C, H, W))
        ts = [torch.from_numpy(a.copy()).requires_grad_(True) for a in (x, y, Wg, bg)]
        out = torch_unfold_fwd(*ts, K)
        (out * torch.from_numpy(G)).sum().backward()
        got = o.fused_bwd(x, y, Wg, bg, G, K)
        for name, t, g in zip(("dx", "dy", "dWg", "dbg"), ts, got):
            _close(g, t.grad.numpy(), 1e-12, f"autograd {name} {N,C,H,W,K}")


def torch_unfold_filter(x, taps, K):
    """The page's construction with materialised taps: three Unfold(x) times the taps."""
    N, C, H, W = x.shape
    r = (K - 1) // 2
    T = taps.reshape(N, 3, C, K * K, H, W)
    outs = [x]
    for bi, D in enumerate(DILATIONS):
        U = F.unfold(x, K, dilation=D, padding=D * r).reshape(N, C, K * K, H, W)
        outs.append((U * T[:, bi]).sum(2))
    return torch.cat(outs, 1)


def numpy_brute_dtaps(x, G, K):
    """dK[o, p] = G_b[c, p] * x[c, p + delta] by zero padding and slicing."""
    N, C, H, W = x.shape
    r = (K - 1) // 2
    P = 5 * r
    xp = np.zeros((N, C, H + 2 * P, W + 2 * P))
    xp[:, :, P:P + H, P:P + W] = x
    out = np.zeros((N, 3, C, K, K, H, W))
    for bi, D in enumerate(DILATIONS):
        Gb = G[:, (1 + bi) * C:(2 + bi) * C]
        for ki in range(K):
            for kj in range(K):
                dh, dw = (ki - r) * D, (kj - r) * D
                out[:, bi, :, ki, kj] = Gb * xp[:, :, P + dh:P + dh + H, P + dw:P + dw + W]
    return out.reshape(N, 3 * C * K * K, H, W)


def pin_filter_bwd_brute_and_autograd(o):
    rng = np.random.default_rng(22)
    for (N, C, H, W, K) in [(2, 5, 15, 17, 3), (1, 3, 9, 8, 5), (1, 4, 6, 7, 1), (1, 2, 1, 1, 3)]:
        x = rng.standard_normal((N, C, H, W))
        taps = rng.standard_normal((N, 3 * C * K * K, H, W))
        G = rng.standard_normal((N, 4 * C, H, W))
        dx, dtaps = o.filter_bwd(x, taps, G, K)
        _close(dtaps, numpy_brute_dtaps(x, G, K), 1e-14, f"dtaps brute {N,C,H,W,K}")
        xt = torch.from_numpy(x.copy()).requires_grad_(True)
        tt = torch.from_numpy(taps.copy()).requires_grad_(True)
        (torch_unfold_filter(xt, tt, K) * torch.from_numpy(G)).sum().backward()
        _close(dx, xt.grad.numpy(), 1e-12, f"filter dx autograd {N,C,H,W,K}")
        _close(dtaps, tt.grad.numpy(), 1e-12, f"filter dtaps autograd {N,C,H,W,K}")


def pin_filter_bwd_finite_differences_and_adjoint(o):
    rng = np.random.default_rng(23)
    N, C, H, W, K = 2, 4, 10, 13, 3
    x = rng.standard_normal((N, C, H, W))
    taps = rng.standard_normal((N, 3 * C * K * K, H, W))
    G = rng.standard_normal((N, 4 * C, H, W))
    dx, dtaps = o.filter_bwd(x, taps, G, K)
    # L = <G, out> is linear in x alone and in taps alone: central differences are exact
    for name, val, grad in (("x", x, dx), ("taps", taps, dtaps)):
        v = rng.standard_normal(val.shape)
        def loss(a):
            return float((o.filter_fwd(a if name == "x" else x, a if name == "taps" else taps, K) * G).sum())
        fd = (loss(val + 0.5 * v) - loss(val - 0.5 * v)) / 1.0
        an = float((grad * v).sum())
        assert abs(fd - an) <= 1e-9 * max(abs(fd), 1.0), f"filter FD {name}: {fd} vs {an}"
    v = rng.standard_normal(x.shape)
    lhs = float(((dx - G[:, :C]) * v).sum())
    rhs = float((G[:, C:] * o.filter_fwd(v, taps, K)[:, C:]).sum())
    assert abs(lhs - rhs) <= 1e-11 * max(abs(rhs), 1.0), f"filter adjoint {lhs} vs {rhs}"


def pin_filter_bwd_matches_fused_bwd(o):
    """With taps = generator(y), the filter's dX equals the fused backward's dX."""
    rng = np.random.default_rng(24)
    N, C, H, W, K = 1, 3, 11, 9, 3
    x, y, Wg, bg = _rand_case(rng, N, C, H, W, K)
    G = rng.standard_normal((N, 4 * C, H, W))
    dx_f, _ = o.filter_bwd(x, o.generator(y, Wg, bg, K), G, K)
    dx_u, _, _, _ = o.fused_bwd(x, y, Wg, bg, G, K)
    _close(dx_f, dx_u, 1e-12, "filter dx vs fused dx")


def pin_sum_partials(o):
    rng = np.random.default_rng(21)
    p = rng.standard_normal((16, 27, 8))
    _close(o.sum_partials(p), p.sum(0), 1e-14, "sum partials")
    _close(o.sum_partials(p[:1]), p[0], 0.0, "single partial")


ALL_PINS = [
    pin_brute_force,
    pin_generator_einsum,
    pin_unfold_reference,
    pin_zero_weight_is_dilated_depthwise_conv,
    pin_one_hot_centre_tap,
    pin_k1_is_x_times_generator,
    pin_all_ones_border_count,
    pin_linear_in_x_affine_in_y,
    pin_finite_differences,
    pin_adjoint_dx,
    pin_autograd_unfold,
    pin_filter_bwd_brute_and_autograd,
    pin_filter_bwd_finite_differences_and_adjoint,
    pin_filter_bwd_matches_fused_bwd,
    pin_sum_partials,
]
