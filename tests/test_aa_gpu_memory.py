"""Peak temporary device memory of one DDPM training step, fused against
materialised (page "lartpang/DynamicConvolutionOperator", section "RTX 5090 结果":
the fused training path needs a fraction of the materialised path's temporary
memory because the tap tensor and its gradient are never stored).

Each case runs ``bench_module --memory-child`` in a fresh child process (its own
allocator, nothing cached), so this file is named to run before every other GPU
test: the children are started before this process makes any GPU call.  The
child reports the allocator's peak during one training step of the module's
dynamic filter minus what was allocated before it.
"""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _child(dt, path, H, K):
    print(f"[gpu case] memory child {dt} {path} {H} K={K}", flush=True)
    r = subprocess.run([sys.executable, "-m", "dynamic_dilated_depthwise_amd.bench_module", "--memory-child",
                        f"{dt},{path},{H},{K}"], cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-3000:]
    row = json.loads(r.stdout.strip().splitlines()[-1])
    print(row, flush=True)
    return row


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fused_training_temporary_memory(dt):
    fused = _child(dt, "fused", 128, 3)
    mat = _child(dt, "materialised", 128, 3)
    assert fused["path"] == "fused" and mat["path"] == "materialised"
    # the materialised step holds the taps (1 x 1728 x 128^2) and their gradient
    es = 4 if dt == "f32" else 2
    taps_mib = 1728 * 128 * 128 * es / 2 ** 20
    assert mat["temporary_peak_MiB"] >= 2 * taps_mib * 0.95, mat
    assert fused["temporary_peak_MiB"] <= 0.2 * mat["temporary_peak_MiB"], (fused, mat)
