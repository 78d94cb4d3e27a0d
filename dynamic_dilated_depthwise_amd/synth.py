"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds random-number recipes only -- none of the method's arithmetic --
so that the HIP path and the fp64 oracle can be fed identical tensors without
sharing any computation.

Recipe: ``torch.Generator('cpu').manual_seed(seed)`` then ``torch.randn`` in
float32 scaled by the standard deviation (the configs state variances, so
std = sqrt(var)).  bf16 cases round those float32 values with ``.to(bfloat16)``
(round-to-nearest-even); the oracle then receives the rounded values exactly.

Workload shapes follow the page "lartpang/DynamicConvolutionOperator": the main
shape B=1, C=64, K=3 at 128^2 and 256^2 ("RTX 5090 结果"), K=5 at 128^2, and the
non-aligned regression B=2, C=24, 15x17 ("验证与基准").  No public dataset is
involved; Gaussian features stand in for the HDFNet feature maps.
"""
import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Shape:
    N: int
    C: int
    H: int
    W: int
    K: int

    @property
    def R(self):
        return 3 * self.C * self.K * self.K

    @property
    def tokens(self):
        return self.N * self.H * self.W


# Named workloads: (shape, seed block).  Seeds are 1000*block + k with k = 0 for
# x, 1 for y, 2 for the generator weight, 3 for its bias, 4 for materialised taps
# and 5 for the output gradient.
WORKLOADS = {
    "tiny": (Shape(1, 8, 16, 16, 3), 1),
    "nonaligned": (Shape(2, 24, 15, 17, 3), 2),
    "bw_filter_128": (Shape(1, 64, 128, 128, 3), 3),
    "fused_inference_256": (Shape(1, 64, 256, 256, 3), 4),
    "fused_training_128_k5": (Shape(1, 64, 128, 128, 5), 5),
    "target_256": (Shape(1, 64, 256, 256, 3), 6),
}


def _randn(shape, seed, std):
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if std != 1.0:
        t = t * std
    return t


def make_inputs(shape: Shape, seed_block: int, dtype=torch.float32, *, taps=False, grad=False,
                w_var=None, b_var=0.01, tap_var=1.0 / 9.0):
    """Return a dict of CPU tensors in ``dtype``.

    x, y ~ N(0, 1); weight [3CK^2, C] ~ N(0, w_var) with w_var = 1/C by default;
    bias [3CK^2] ~ N(0, b_var); optional taps [N, 3CK^2, H, W] ~ N(0, tap_var);
    optional grad_out [N, 4C, H, W] ~ N(0, 1).
    """
    N, C, H, W, K = shape.N, shape.C, shape.H, shape.W, shape.K
    R = shape.R
    if w_var is None:
        w_var = 1.0 / C
    s = 1000 * seed_block
    d = {
        "x": _randn((N, C, H, W), s + 0, 1.0),
        "y": _randn((N, C, H, W), s + 1, 1.0),
        "weight": _randn((R, C), s + 2, math.sqrt(w_var)),
        "bias": _randn((R,), s + 3, math.sqrt(b_var)),
    }
    if taps:
        d["taps"] = _randn((N, R, H, W), s + 4, math.sqrt(tap_var))
    if grad:
        d["grad_out"] = _randn((N, 4 * C, H, W), s + 5, 1.0)
    return {k: v.to(dtype) for k, v in d.items()}

