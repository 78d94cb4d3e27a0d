"""PyTorch-facing DDPM: autograd functions over the library and the ``DDPM`` module.

Page "lartpang/DynamicConvolutionOperator", section "使用" (usage): the module is
built as ``DDPM(dim, kernel_size)`` and called as ``module(x, y)``; a 1x1
generator over the guidance features y makes the per-pixel K x K taps of the three
dilations, the dynamic filter applies them to x, and the concatenation
``[x, d1, d3, d5]`` goes through a final 3x3 fuse convolution, which the page
leaves to the vendor convolution library ("CUDA 融合生成器推理").

Two execution paths, both through the HIP library (torch supplies memory,
streams, the 1x1 generator of the materialised path and the 3x3 fuse conv):

* **fused** ("CUDA 融合生成器推理", "CUDA Flash 式融合训练"): ``ddpm_fused_fwd``
  generates and consumes the taps on chip; training saves only x, y and the
  generator parameters and runs ``ddpm_fused_bwd`` + ``ddpm_reduce_partials``;
* **materialised**: torch's 1x1 convolution writes the tap tensor, then
  ``ddpm_filter_fwd`` / ``ddpm_filter_bwd`` ("CUDA 动态过滤"); torch's convolution
  backward carries the tap gradient into the generator.

Dispatch follows the page's rules ("CUDA Flash 式融合训练", automatic mode): the
fused path needs x, y and the generator in one dtype and autocast off; ``True``
forces it (for training; an error if it is not eligible), ``False`` forces the
materialised path, ``None`` (the default) picks the fused path when it is eligible
and the token count N*H*W reaches the threshold for (mode, dtype, K) in
``AUTO_MIN_TOKENS``.  The page's thresholds were tuned on its own GPU; these come
from timing both paths on MI355X (``bench_module.py``, B=1, C=64, 16^2 .. 256^2):
training is fused at every size with K = 3 and in bfloat16, from 96^2 = 9216
tokens with K = 5 in fp32, and inference is fused at every size.  The fused path also needs about a tenth of the
temporary memory (the tap tensor and its gradient are never stored).

CPU tensors take the CPU path of ``cpu_stream`` (section "CPU 与超大输入": one
generator GEMM while the taps fit ``max_generated_bytes``, token tiles of
``spatial_tile_size`` beyond it, with per-tile recompute in training when
``recompute`` is set); device tensors never do.  Under autocast in float16 the
materialised path filters in float32 (the library takes float32 and bfloat16).
"""
import torch
import torch.nn as nn

from . import (ddpm_filter_bwd, ddpm_filter_fwd, ddpm_fused_bwd, ddpm_fused_fwd, ddpm_reduce_partials,
               num_partials_for)
from .cpu_stream import DEFAULT_MAX_GENERATED_BYTES, DEFAULT_TILE_TOKENS, ddpm_cpu

__all__ = ["DDPMFused", "DDPMFilter", "ddpm_fused", "ddpm_filter", "choose_path", "auto_min_tokens", "DDPM",
           "AUTO_MIN_TOKENS"]

# Smallest N*H*W at which automatic mode takes the fused path, per (mode, dtype, K);
# None: never (MI355X timings of bench_module.py; K = 1 follows K = 3).
_F32, _BF16 = torch.float32, torch.bfloat16
AUTO_MIN_TOKENS = {
    ("train", _F32, 3): 1, ("train", _F32, 5): 9216,
    ("train", _BF16, 3): 1, ("train", _BF16, 5): 1,
    ("infer", _F32, 3): 1, ("infer", _F32, 5): 1,
    ("infer", _BF16, 3): 1, ("infer", _BF16, 5): 1,
}


def auto_min_tokens(training, dtype, K):
    return AUTO_MIN_TOKENS[("train" if training else "infer", dtype, 3 if K == 1 else K)]

_SUPPORTED = (torch.float32, torch.bfloat16)


def _autocast():
    return torch.is_autocast_enabled("cuda")


def _check_gpu(*ts):
    for t in ts:
        if not t.is_cuda:
            raise RuntimeError("the HIP library takes device tensors; CPU tensors go through "
                               "DDPM's CPU path (cpu_stream.ddpm_cpu)")
        if t.dtype not in _SUPPORTED:
            raise TypeError(f"DDPM supports float32 and bfloat16 tensors, got {t.dtype}")


class DDPMFused(torch.autograd.Function):
    """[x, d1, d3, d5] from x, y and the generator (weight [3CK^2, C], bias
    [3CK^2]) with the taps made and consumed on chip; the backward recomputes
    them (dX gather, dY = W^T dK, dW/db over <= 16 fp32 token partials)."""

    @staticmethod
    def forward(ctx, x, y, weight, bias, K):
        N, C, H, W = x.shape
        out = torch.empty((N, 4 * C, H, W), device=x.device, dtype=x.dtype)
        ddpm_fused_fwd(x, y, weight, bias, out, K)
        ctx.save_for_backward(x, y, weight, bias)
        ctx.K = K
        return out

    @staticmethod
    def backward(ctx, grad_out):
        x, y, weight, bias = ctx.saved_tensors
        K = ctx.K
        N, C, H, W = x.shape
        R = 3 * C * K * K
        need_x, need_y, need_w, need_b = ctx.needs_input_grad[:4]
        g = grad_out.contiguous()
        gx = torch.empty_like(x) if need_x else None
        gy = torch.empty_like(y) if need_y else None
        gw = gb = None
        pw = pb = None
        if need_w or need_b:
            S = num_partials_for(N, C, H, W, K)
            pw = torch.empty((S, R, C), device=x.device, dtype=torch.float32)
            pb = torch.empty((S, R), device=x.device, dtype=torch.float32)
        if gx is not None or gy is not None or pw is not None:
            ddpm_fused_bwd(x, y, weight, bias, g, gx, gy, pw, pb, K)
        if pw is not None:
            gw = torch.empty_like(weight)
            gb = torch.empty_like(bias)
            ddpm_reduce_partials(pw, pb, gw, gb, K)
        return gx, gy, (gw if need_w else None), (gb if need_b else None), None


class DDPMFilter(torch.autograd.Function):
    """[x, d1, d3, d5] from x and materialised taps [N, 3CK^2, H, W]; the backward
    gives dX and the tap gradient (one fused pass)."""

    @staticmethod
    def forward(ctx, x, taps, K):
        N, C, H, W = x.shape
        out = torch.empty((N, 4 * C, H, W), device=x.device, dtype=x.dtype)
        ddpm_filter_fwd(x, taps, out, K)
        ctx.save_for_backward(x, taps)
        ctx.K = K
        return out

    @staticmethod
    def backward(ctx, grad_out):
        x, taps = ctx.saved_tensors
        need_x, need_t = ctx.needs_input_grad[:2]
        if not (need_x or need_t):
            return None, None, None
        gx = torch.empty_like(x) if need_x else None
        gt = torch.empty_like(taps) if need_t else None
        ddpm_filter_bwd(x, taps, grad_out.contiguous(), gx, gt, ctx.K)
        return gx, gt, None


def ddpm_fused(x, y, weight, bias, K):
    """Differentiable fused DDPM filter: weight [3CK^2, C], bias [3CK^2]."""
    _check_gpu(x, y, weight, bias)
    return DDPMFused.apply(x.contiguous(), y.contiguous(), weight.contiguous(), bias.contiguous(), K)


def ddpm_filter(x, taps, K):
    """Differentiable materialised DDPM filter over taps [N, 3CK^2, H, W]."""
    _check_gpu(x, taps)
    return DDPMFilter.apply(x.contiguous(), taps.contiguous(), K)


def choose_path(training, tokens, K, x_dtype, y_dtype, param_dtype, autocast, fused_inference=None,
                fused_training=None, min_tokens=None):
    """'fused' or 'materialised' for one call (host logic only).

    training: a gradient is needed; tokens: N*H*W; autocast: torch autocast is on
    for the device; fused_inference / fused_training: True, False or None (automatic);
    min_tokens: overrides the automatic threshold (None: AUTO_MIN_TOKENS)."""
    eligible = x_dtype == y_dtype == param_dtype and not autocast
    force = fused_training if training else fused_inference
    if force is False:
        return "materialised"
    if force is True:
        if eligible:
            return "fused"
        if training:
            raise ValueError("fused training needs x, y and the generator in one dtype and autocast off")
        return "materialised"
    if not eligible:
        return "materialised"
    limit = auto_min_tokens(training, param_dtype, K) if min_tokens is None else min_tokens
    return "fused" if (limit is not None and tokens >= limit) else "materialised"


class DDPM(nn.Module):
    """Dynamic Dilated Pyramid Module: ``DDPM(dim, kernel_size)(x, y)``.

    generator: 1x1 conv dim -> 3*dim*K^2 (with bias), row o = (b*dim + c)*K^2 + t
    for dilation b (1, 3, 5), channel c, tap t = ki*K + kj;
    filter:    [x, d1, d3, d5], zero padding D*(K-1)/2 per dilation D;
    fuse:      3x3 conv 4*dim -> dim, padding 1 (with bias).
    x and y are [N, dim, H, W], float32 or bfloat16, on the GPU (the HIP library)
    or on the CPU (the CPU path).
    spatial_tile_size / max_generated_bytes / recompute: the CPU path's token tile,
    the tap budget beyond which it streams tiles, and per-tile recompute in
    training (page section "使用").
    fused_generator_inference / fused_generator_training: True (fused), False
    (materialised) or None (automatic, see the module docstring); GPU only."""

    def __init__(self, dim=64, kernel_size=3, spatial_tile_size=DEFAULT_TILE_TOKENS,
                 max_generated_bytes=DEFAULT_MAX_GENERATED_BYTES, recompute=True, fused_generator_inference=None,
                 fused_generator_training=None):
        super().__init__()
        if kernel_size not in (1, 3, 5):
            raise ValueError("kernel_size must be 1, 3 or 5 (dilations 1, 3, 5 are fixed)")
        self.dim = dim
        self.kernel_size = kernel_size
        self.spatial_tile_size = spatial_tile_size
        self.max_generated_bytes = max_generated_bytes
        self.recompute = recompute
        self.fused_generator_inference = fused_generator_inference
        self.fused_generator_training = fused_generator_training
        self.generator = nn.Conv2d(dim, 3 * dim * kernel_size * kernel_size, 1)
        self.fuse = nn.Conv2d(4 * dim, dim, 3, padding=1)
        self.last_path = None  # which path the last forward took

    def path_for(self, x, y):
        training = torch.is_grad_enabled() and (x.requires_grad or y.requires_grad or
                                                any(p.requires_grad for p in self.generator.parameters()))
        N, _, H, W = x.shape
        return choose_path(training, N * H * W, self.kernel_size, x.dtype, y.dtype, self.generator.weight.dtype,
                           _autocast(), self.fused_generator_inference, self.fused_generator_training)

    def dynamic_filter(self, x, y):
        """[x, d1, d3, d5] (before the fuse conv)."""
        K = self.kernel_size
        R = 3 * self.dim * K * K
        if not x.is_cuda and not y.is_cuda and not self.generator.weight.is_cuda:
            w = self.generator.weight.view(R, self.dim)
            out, self.last_path = ddpm_cpu(x, y.to(w.dtype), w, self.generator.bias, K, self.spatial_tile_size,
                                           self.max_generated_bytes, self.recompute)
            return out
        _check_gpu(x, y)
        path = self.path_for(x, y)
        self.last_path = path
        if path == "fused":
            w = self.generator.weight.view(R, self.dim)
            return ddpm_fused(x, y, w, self.generator.bias, K)
        # materialised: torch makes the taps (autocast decides their dtype; otherwise y
        # is taken in the parameters' dtype), the library filters x in the taps' dtype
        if _autocast():
            taps = self.generator(y)
        else:
            taps = self.generator(y.to(self.generator.weight.dtype))
        if taps.dtype not in _SUPPORTED:
            # float16 autocast: the library filters float32 and bfloat16; float16
            # widens to float32 exactly
            taps = taps.float()
        return ddpm_filter(x.to(taps.dtype), taps, K)

    def forward(self, x, y):
        feats = self.dynamic_filter(x, y)
        return self.fuse(feats.to(self.fuse.weight.dtype) if not _autocast() else feats)
