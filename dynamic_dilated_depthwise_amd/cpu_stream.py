"""CPU path of the DDPM dynamic filter, with token streaming for large inputs.

Page "lartpang/DynamicConvolutionOperator", section "CPU 与超大输入" (CPU and very
large inputs), with the constructor arguments of "使用" (usage):

* while the generated taps, N * 3CK^2 * H * W elements, fit ``max_generated_bytes``
  (256 MiB by default) the generator stays one 1x1 convolution over the whole
  input (a oneDNN GEMM) and the filter reads x through a zero-padded copy and
  shifted views of it (no unfold); training differentiates these torch ops, which
  keep the tap tensor for the backward;
* beyond that budget the taps are generated and consumed one spatial tile of at
  most ``spatial_tile_size`` tokens per image (4096 by default) at a time, so the
  temporary tap tensor is O(N * T * 3CK^2) instead of O(N * H * W * 3CK^2);
  training then keeps only x, y and the generator, and the backward recomputes
  each tile's taps (``recompute=True``; with ``recompute=False`` the tiles are
  differentiated as they are, keeping every tile's taps).

What is computed is the module's dynamic filter, ``[x, d1, d3, d5]``:
  T[n, o, p] = bias[o] + sum_c' weight[o, c'] y[n, c', p],  o = (b*C + c)*K*K + t,
  O_b[n, c, h, w] = sum_t T[n, o, h, w] x[n, c, h + (ki - r) D_b, w + (kj - r) D_b]
with D = (1, 3, 5), r = (K-1)/2, t = ki*K + kj and x zero outside the image.
Precision: the generator runs in the input dtype (bfloat16 taps are rounded once,
as torch's bfloat16 convolution gives them); every product and sum of the filter
and of the streamed backward is float32, and results are rounded once to the
input dtype.

This is a CPU execution path for CPU tensors; device tensors always take the HIP
library (the package's C ABI), never this module.
"""
import torch
import torch.nn.functional as F

__all__ = ["ddpm_cpu", "generated_bytes", "tile_shape", "DEFAULT_TILE_TOKENS", "DEFAULT_MAX_GENERATED_BYTES"]

DEFAULT_TILE_TOKENS = 4096
DEFAULT_MAX_GENERATED_BYTES = 256 * 1024 ** 2
_DILATIONS = (1, 3, 5)


def generated_bytes(N, C, H, W, K, dtype):
    """Bytes of the whole generated tap tensor [N, 3CK^2, H, W] in `dtype`."""
    return N * 3 * C * K * K * H * W * torch.empty((), dtype=dtype).element_size()


def tile_shape(H, W, tokens):
    """(rows, cols) of a spatial tile of at most `tokens` pixels: whole rows when a
    row fits, else a run of one row."""
    tw = min(W, max(1, tokens))
    th = max(1, min(H, tokens // tw))
    return th, tw


def _offsets(K):
    """(b, t, dy, dx) of every (dilation, tap): the source pixel of output (h, w) is
    (h + dy, w + dx)."""
    r = (K - 1) // 2
    return [(b, ki * K + kj, (ki - r) * D, (kj - r) * D)
            for b, D in enumerate(_DILATIONS) for ki in range(K) for kj in range(K)]


def _gen(y, weight, bias):
    """1x1 generator: [N, C, h, w] -> [N, R, h, w] (one GEMM over the tokens)."""
    return F.conv2d(y, weight[:, :, None, None], bias)


def _filter_tile(xp, T, K, P, h0, w0, th, tw):
    """Branch outputs [N, 3, C, th, tw] (float32) of the tile at (h0, w0) from the padded
    x `xp` (pad P on every side) and the tile's taps T [N, R, th, tw]."""
    N, C = xp.shape[0], xp.shape[1]
    KK = K * K
    Tv = T.view(N, 3, C, KK, th, tw)
    acc = torch.zeros((N, 3, C, th, tw), dtype=torch.float32)
    for b, t, dy, dx in _offsets(K):
        src = xp[:, :, P + h0 + dy:P + h0 + dy + th, P + w0 + dx:P + w0 + dx + tw]
        acc[:, b].addcmul_(Tv[:, b, :, t].float(), src.float())
    return acc


def _direct(x, y, weight, bias, K):
    """Whole-input path, differentiable by autograd: one generator GEMM, padded x and
    shifted views."""
    N, C, H, W = x.shape
    KK = K * K
    P = 5 * ((K - 1) // 2)
    T = _gen(y, weight, bias).view(N, 3, C, KK, H, W)
    xp = F.pad(x, (P, P, P, P))
    blocks = []
    for b in range(3):
        acc = None
        for bb, t, dy, dx in _offsets(K):
            if bb != b:
                continue
            term = T[:, b, :, t].float() * xp[:, :, P + dy:P + dy + H, P + dx:P + dx + W].float()
            acc = term if acc is None else acc + term
        blocks.append(acc.to(x.dtype))
    return torch.cat([x] + blocks, dim=1)


def _tiles(H, W, tile_tokens):
    th, tw = tile_shape(H, W, tile_tokens)
    for h0 in range(0, H, th):
        for w0 in range(0, W, tw):
            yield h0, w0, min(th, H - h0), min(tw, W - w0)


def _streamed_forward(x, y, weight, bias, K, tile_tokens):
    N, C, H, W = x.shape
    P = 5 * ((K - 1) // 2)
    xp = F.pad(x, (P, P, P, P))
    out = torch.empty((N, 4 * C, H, W), dtype=x.dtype)
    out[:, :C] = x
    ov = out.view(N, 4, C, H, W)
    for h0, w0, th, tw in _tiles(H, W, tile_tokens):
        T = _gen(y[:, :, h0:h0 + th, w0:w0 + tw], weight, bias)
        ov[:, 1:, :, h0:h0 + th, w0:w0 + tw] = _filter_tile(xp, T, K, P, h0, w0, th, tw).to(x.dtype)
    return out


class _StreamedRecompute(torch.autograd.Function):
    """Streamed forward; the backward regenerates each tile's taps (nothing but x, y
    and the generator is kept between the passes)."""

    @staticmethod
    def forward(ctx, x, y, weight, bias, K, tile_tokens):
        ctx.save_for_backward(x, y, weight, bias)
        ctx.K, ctx.tile_tokens = K, tile_tokens
        with torch.no_grad():
            return _streamed_forward(x, y, weight, bias, K, tile_tokens)

    @staticmethod
    def backward(ctx, grad_out):
        x, y, weight, bias = ctx.saved_tensors
        K, tile_tokens = ctx.K, ctx.tile_tokens
        N, C, H, W = x.shape
        R = weight.shape[0]
        KK = K * K
        P = 5 * ((K - 1) // 2)
        g = grad_out.contiguous().view(N, 4, C, H, W)
        xp = F.pad(x, (P, P, P, P))
        wf = weight.float()
        # gradients of the padded x, of y, of the generator (float32 sums)
        dxp = torch.zeros((N, C, H + 2 * P, W + 2 * P), dtype=torch.float32)
        dy = torch.empty((N, C, H, W), dtype=torch.float32)
        dw = torch.zeros((R, C), dtype=torch.float32)
        db = torch.zeros((R,), dtype=torch.float32)
        for h0, w0, th, tw in _tiles(H, W, tile_tokens):
            yt = y[:, :, h0:h0 + th, w0:w0 + tw]
            Tv = _gen(yt, weight, bias).view(N, 3, C, KK, th, tw)
            gb = g[:, 1:, :, h0:h0 + th, w0:w0 + tw].float()           # [N, 3, C, th, tw]
            dT = torch.empty((N, 3, C, KK, th, tw), dtype=torch.float32)  # gradient of the tile's taps
            for b, t, dyo, dxo in _offsets(K):
                hs, ws = P + h0 + dyo, P + w0 + dxo
                dT[:, b, :, t] = gb[:, b] * xp[:, :, hs:hs + th, ws:ws + tw].float()
                # each tap reached x at its source pixel: send its share back there
                dxp[:, :, hs:hs + th, ws:ws + tw].addcmul_(Tv[:, b, :, t].float(), gb[:, b])
            dTm = dT.view(N, R, th * tw)
            ytm = yt.float().reshape(N, C, th * tw)
            dw += torch.einsum("nrp,ncp->rc", dTm, ytm)
            db += dTm.sum(dim=(0, 2))
            dy[:, :, h0:h0 + th, w0:w0 + tw] = torch.matmul(wf.t(), dTm).view(N, C, th, tw)
        dx = dxp[:, :, P:P + H, P:P + W] + g[:, 0].float()
        return (dx.to(x.dtype), dy.to(y.dtype), dw.to(weight.dtype), db.to(bias.dtype), None, None)


def ddpm_cpu(x, y, weight, bias, K, spatial_tile_size=DEFAULT_TILE_TOKENS,
             max_generated_bytes=DEFAULT_MAX_GENERATED_BYTES, recompute=True):
    """[x, d1, d3, d5] of CPU tensors x, y [N, C, H, W] with the generator weight
    [3CK^2, C] and bias [3CK^2]; differentiable.  Returns (output, path) with path
    "cpu_direct" (the taps fit the budget) or "cpu_streamed"."""
    for name, t in (("x", x), ("y", y), ("weight", weight), ("bias", bias)):
        if t.device.type != "cpu":
            raise ValueError(f"ddpm_cpu takes CPU tensors ({name} is on {t.device})")
    if K not in (1, 3, 5):
        raise ValueError("K must be 1, 3 or 5")
    if spatial_tile_size < 1:
        raise ValueError("spatial_tile_size must be positive")
    N, C, H, W = x.shape
    if tuple(y.shape) != (N, C, H, W) or tuple(weight.shape) != (3 * C * K * K, C) or \
            tuple(bias.shape) != (3 * C * K * K,):
        raise ValueError("shapes: x, y [N, C, H, W], weight [3CK^2, C], bias [3CK^2]")
    x, y, weight, bias = x.contiguous(), y.contiguous(), weight.contiguous(), bias.contiguous()
    if generated_bytes(N, C, H, W, K, y.dtype) <= max_generated_bytes:
        return _direct(x, y, weight, bias, K), "cpu_direct"
    needs_grad = torch.is_grad_enabled() and any(t.requires_grad for t in (x, y, weight, bias))
    if not needs_grad:
        with torch.no_grad():
            return _streamed_forward(x, y, weight, bias, K, spatial_tile_size), "cpu_streamed"
    if recompute:
        return _StreamedRecompute.apply(x, y, weight, bias, K, spatial_tile_size), "cpu_streamed"
    # no recompute: differentiate each tile as it is (its taps stay alive for the backward)
    P = 5 * ((K - 1) // 2)
    xp = F.pad(x, (P, P, P, P))
    rows = []
    th, tw = tile_shape(H, W, spatial_tile_size)
    for h0 in range(0, H, th):
        cols = []
        for w0 in range(0, W, tw):
            h1, w1 = min(H, h0 + th), min(W, w0 + tw)
            T = _gen(y[:, :, h0:h1, w0:w1], weight, bias)
            cols.append(_filter_tile(xp, T, K, P, h0, w0, h1 - h0, w1 - w0).to(x.dtype))
        rows.append(torch.cat(cols, dim=-1))
    blocks = torch.cat(rows, dim=-2).reshape(N, 3 * C, H, W)
    return torch.cat([x, blocks], dim=1), "cpu_streamed"
