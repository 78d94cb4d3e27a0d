"""bench.py host logic (no GPU): the one-GPU guard and the algorithmic work that
every roofline figure divides by, checked against closed forms written out here
for the 256x256, C=64, K=3 workload."""
import os
import subprocess
import sys

import pytest

import bench
from dynamic_dilated_depthwise_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_algorithmic_work_at_the_target_shape():
    shape = synth.Shape(1, 64, 256, 256, 3)
    P, C, R = 256 * 256, 64, 3 * 64 * 9
    a32 = bench.algorithmic(shape, 4, 16)
    a16 = bench.algorithmic(shape, 2, 16)
    # filter: 1728 tap planes + x read, 4 output planes written
    assert a32["filter"]["bytes"] == (1728 + 64 + 256) * 4 * 65536 == 536870912
    assert a16["filter"]["bytes"] == 536870912 // 2
    # every fused pass is one generator contraction: 2 * 1728 * 64 flops per token
    for k in ("fused_fwd", "bwd_dx", "bwd_dy", "bwd_dw"):
        assert a32[k]["flops"] == 2.0 * 1728 * 64 * 65536 == 14495514624.0
    # fused forward: x, y read and 4C written per token, plus the weight and bias once
    assert a32["fused_fwd"]["bytes"] == 6 * C * 4 * P + (R * C + R) * 4
    # materialised backward: x, taps, G read and dX, dtaps written
    assert a32["filter_bwd"]["bytes"] == (2 * 1728 + 6 * 64) * 4 * 65536 == 1006632960
    # reduce: 16 fp32 partials read, one gradient written in the dtype
    assert a16["reduce"]["bytes"] == 16 * (R * C + R) * 4 + (R * C + R) * 2


def test_every_kernel_has_a_bound_and_sources():
    names = set(bench.algorithmic(synth.Shape(1, 8, 16, 16, 3), 4, 1))
    assert names == set(bench.KERNEL_BOUND) == set(bench.KERNEL_SYMBOL) == set(bench.KERNEL_SOURCES)
    for srcs in bench.KERNEL_SOURCES.values():
        for f in srcs:
            assert os.path.exists(os.path.join(ROOT, "dynamic_dilated_depthwise_amd", "csrc", f)), f


def test_bench_module_cli():
    """The module benchmark's command line (no GPU: parsing only)."""
    import subprocess
    import sys as _sys
    from dynamic_dilated_depthwise_amd import bench_module as bm
    a = bm.parse_args(["--mode", "memory", "--dtypes", "bf16"])
    assert a.mode == "memory" and a.dtypes == ["bf16"] and a.ks == [3, 5]
    a = bm.parse_args(["--memory-child", "f32,fused,128,3"])
    assert a.memory_child == "f32,fused,128,3"
    for bad in (["--mode", "none"], ["--dtypes", "f16"], ["--memory-child", "f32,unfold,128,3"],
                ["--memory-child", "f32,fused"]):
        with pytest.raises(SystemExit):
            bm.parse_args(bad)
    r = subprocess.run([_sys.executable, "-m", "dynamic_dilated_depthwise_amd.bench_module", "--help"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0 and "--memory-child" in r.stdout


def test_cpu_baseline_sample_stops_after_its_floor():
    """The oracle baseline times at least three steps after one warm-up, keeps going
    until its time floor is met, and never passes its step cap."""
    shape = synth.Shape(1, 4, 8, 8, 3)
    h = synth.make_inputs(shape, 1, taps=True, grad=True)
    t = bench.run_cpu_baseline(h, shape, min_reps=3, min_s=0.0, max_reps=5)
    assert t["reps"] == 3
    t = bench.run_cpu_baseline(h, shape, min_reps=3, min_s=1e9, max_reps=5)
    assert t["reps"] == 5 and t["timed_s"] > 0
    for k in ("filter", "fused_fwd", "fused_bwd"):
        assert t[k] > 0
