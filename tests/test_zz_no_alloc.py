"""ddpm_fused_bwd_noalloc: the backward with its float32 partials in the library's
fixed device buffer, against ddpm_fused_bwd + ddpm_reduce_partials with a caller
workspace and the same split count.

Both run the same kernels on the same inputs, so every output must match bit for
bit.  Two calls in a row, the second on a smaller input, check that the shared
buffer carries nothing from one call into the next; a request beyond the buffer
must fail before anything runs.
"""
import pytest
import torch

import dynamic_dilated_depthwise_amd as ddpm
from dynamic_dilated_depthwise_amd import synth
from gpu_cases import TOL, announce, assert_close, dev, f64, gpu_bwd, inputs, orc

pytestmark = pytest.mark.gpu

S_ = synth.Shape


def _noalloc(d, K, S):
    x = d["x"]
    N, C, H, W = x.shape
    R = 3 * C * K * K
    gx, gy = torch.empty_like(x), torch.empty_like(x)
    gw = torch.empty((R, C), device="cuda", dtype=x.dtype)
    gb = torch.empty((R,), device="cuda", dtype=x.dtype)
    ddpm.ddpm_fused_bwd_noalloc(x, d["y"], d["weight"], d["bias"], d["grad_out"], gx, gy, gw, gb, K,
                                num_partials=S)
    torch.cuda.synchronize()
    return gx, gy, gw, gb


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_noalloc_matches_workspace_path_twice(dt):
    # first the 1x64x128^2 K=5 training workload (S=16: the largest partials a C=64
    # call needs), then a smaller ragged input that uses less of the buffer
    cases = [synth.WORKLOADS["fused_training_128_k5"], (S_(2, 24, 15, 17, 3), 301)]
    for shape, block in cases:
        K = shape.K
        announce("noalloc", shape, dt)
        h = inputs(shape, block, dt, grad=True)
        d = dev(h)
        S = ddpm.num_partials_for(shape.N, shape.C, shape.H, shape.W, K)
        ref = gpu_bwd(d, K, S)[:4]
        got = _noalloc(d, K, S)
        for name, a, b in zip(("grad_x", "grad_y", "grad_weight", "grad_bias"), got, ref):
            assert torch.equal(a, b), f"{name} differs from the workspace path ({shape}, {dt})"
    # the last call's results also against the oracle (same bar as the parity tests)
    a = {k: v.double().numpy() for k, v in h.items()}
    refs = orc().fused_bwd(a["x"], a["y"], a["weight"], a["bias"], a["grad_out"], K)
    for name, g, r in zip(("grad_x", "grad_y", "grad_weight", "grad_bias"), got, refs):
        assert_close(f64(g), r, TOL[dt]["grad"], name)


def test_noalloc_optional_outputs_and_limit():
    shape, block = S_(1, 16, 20, 24, 3), 302
    K = shape.K
    announce("noalloc optional outputs", shape)
    d = dev(inputs(shape, block, torch.float32, grad=True))
    S = 3
    ref = gpu_bwd(d, K, S)[:4]
    x = d["x"]
    R = 3 * shape.C * K * K
    gw = torch.empty((R, shape.C), device="cuda")
    gb = torch.empty((R,), device="cuda")
    ddpm.ddpm_fused_bwd_noalloc(x, d["y"], d["weight"], d["bias"], d["grad_out"], None, None, gw, gb, K,
                                num_partials=S)
    gx = torch.empty_like(x)
    ddpm.ddpm_fused_bwd_noalloc(x, d["y"], d["weight"], d["bias"], d["grad_out"], gx, None, None, None, K)
    torch.cuda.synchronize()
    assert torch.equal(gw, ref[2]) and torch.equal(gb, ref[3]) and torch.equal(gx, ref[0])

    # C=128, K=5, 16 partials need 16 * (9600*128 + 9600) floats = 79 MB > 32 MiB:
    # rejected by the size check before any launch (the tensors are never read)
    big = S_(1, 128, 4, 4, 5)
    db = dev(inputs(big, 303, torch.float32, grad=True))
    Rb = 3 * big.C * 25
    with pytest.raises(ddpm.DDPMError, match="SCRATCH_LIMIT"):
        ddpm.ddpm_fused_bwd_noalloc(db["x"], db["y"], db["weight"], db["bias"], db["grad_out"], None, None,
                                    torch.empty((Rb, big.C), device="cuda"), torch.empty((Rb,), device="cuda"),
                                    5, num_partials=16)
