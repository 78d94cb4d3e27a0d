"""HIP graph capture: the library allocates nothing, sets no memory and launches on
the caller's stream, so a whole step can be captured once and replayed.

One step (materialised filter and its backward, fused forward, fused backward,
partial reduce) is captured into a torch CUDA graph and replayed three times;
between replays the outputs are overwritten and unrelated eager work runs on the
same device.  Every replay must reproduce the eager results bit for bit (the
kernels are deterministic: every output element is stored once, no atomics).
"""
import pytest
import torch

import dynamic_dilated_depthwise_amd as ddpm
from dynamic_dilated_depthwise_amd import synth
from gpu_cases import announce, dev, inputs

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("name,shape", [("nonaligned_k3", synth.Shape(2, 24, 15, 17, 3)),
                                        ("c64_k5", synth.Shape(1, 64, 20, 72, 5)),
                                        # the row-staged backward kernels and 8-pixel filter runs
                                        ("c64_256", synth.Shape(1, 64, 256, 256, 3))],
                         ids=["nonaligned_k3", "c64_k5", "c64_256"])
def test_graph_replays_match_eager(name, shape, dt):
    dtype = DT[dt]
    K = shape.K
    d = dev(inputs(shape, 501, dtype, taps=True, grad=True))
    N, C, H, W = d["x"].shape
    R = 3 * C * K * K
    S = ddpm.num_partials_for(N, C, H, W, K)
    outs = {
        "filter": torch.empty((N, 4 * C, H, W), device="cuda", dtype=dtype),
        "filter_gx": torch.empty_like(d["x"]),
        "filter_gt": torch.empty_like(d["taps"]),
        "fused": torch.empty((N, 4 * C, H, W), device="cuda", dtype=dtype),
        "gx": torch.empty_like(d["x"]),
        "gy": torch.empty_like(d["x"]),
        "pw": torch.empty((S, R, C), device="cuda", dtype=torch.float32),
        "pb": torch.empty((S, R), device="cuda", dtype=torch.float32),
        "gw": torch.empty((R, C), device="cuda", dtype=dtype),
        "gb": torch.empty((R,), device="cuda", dtype=dtype),
    }

    def step():
        ddpm.ddpm_filter_fwd(d["x"], d["taps"], outs["filter"], K)
        ddpm.ddpm_filter_bwd(d["x"], d["taps"], d["grad_out"], outs["filter_gx"], outs["filter_gt"], K)
        ddpm.ddpm_fused_fwd(d["x"], d["y"], d["weight"], d["bias"], outs["fused"], K)
        ddpm.ddpm_fused_bwd(d["x"], d["y"], d["weight"], d["bias"], d["grad_out"], outs["gx"], outs["gy"],
                            outs["pw"], outs["pb"], K)
        ddpm.ddpm_reduce_partials(outs["pw"], outs["pb"], outs["gw"], outs["gb"], K)

    announce("graph capture", name, dt, shape)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # eager reference (also sets any per-kernel launch attributes)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    a = torch.randn(256, 256, device="cuda")
    for rep in range(3):
        for v in outs.values():
            v.fill_(float("nan") if v.is_floating_point() else 0)
        a = torch.tanh(a @ a.T / 256.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            ib = torch.int32 if v.dtype == torch.float32 else torch.int16
            same = torch.equal(v.view(ib), eager[k].view(ib))
            assert same, f"replay {rep}: {k} differs from the eager result"
