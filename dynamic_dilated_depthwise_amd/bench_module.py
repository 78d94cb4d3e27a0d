"""Fused vs materialised DDPM on one MI355X: step time and peak temporary memory.

    python -m dynamic_dilated_depthwise_amd.bench_module [--mode speed|memory|all]

speed   For each dtype (float32, bfloat16), K (3, 5) and image size (16^2 .. 256^2,
        B=1, C=64) the module's dynamic filter (generator + filter, without the 3x3
        fuse conv, which both paths share) is timed on both paths: inference (no
        grad) and one training step (forward + backward of every input and
        parameter gradient), HIP events around 20 back-to-back repetitions after 3
        warm-up ones.  This is what the automatic training mode's token threshold
        is chosen from (page "lartpang/DynamicConvolutionOperator", section
        "CUDA Flash 式融合训练": the page's own thresholds were tuned on its GPU).
memory  Peak temporary device memory of one training step at B=1, C=64, K=3,
        256^2 and 128^2, per path and dtype (the page's "验证与基准" / "RTX 5090 结果"
        compare it between paths), each measured in a fresh process: the
        allocator's peak during the step minus what was allocated before it
        (inputs, parameters).

Each result is one JSON line on stdout; progress goes to stderr.  Inputs are seeded
Gaussians (dynamic_dilated_depthwise_amd.synth); the generator and fuse weights are
torch's default initialisation under a fixed seed.
"""
import argparse
import json
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from dynamic_dilated_depthwise_amd import synth  # noqa: E402
from dynamic_dilated_depthwise_amd.module import DDPM  # noqa: E402

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def log(*a):
    print("[bench_module]", *a, file=sys.stderr, flush=True)


def make(dtype, C, H, W, K, seed):
    torch.manual_seed(seed)
    m = DDPM(dim=C, kernel_size=K).to(device="cuda", dtype=dtype)
    h = synth.make_inputs(synth.Shape(1, C, H, W, K), seed, dtype, grad=True)
    x = h["x"].cuda().requires_grad_(True)
    y = h["y"].cuda().requires_grad_(True)
    g = h["grad_out"].cuda()
    return m, x, y, g


def step_fn(m, x, y, g, path, training):
    m.fused_generator_inference = path == "fused"
    m.fused_generator_training = path == "fused"
    params = list(m.generator.parameters())

    def run():
        if training:
            out = m.dynamic_filter(x, y)
            torch.autograd.grad(out, [x, y] + params, g)
        else:
            with torch.no_grad():
                m.dynamic_filter(x, y)
    return run


def time_fn(fn, reps=20, warm=3):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def run_speed(args):
    sizes = [16, 32, 64, 96, 128, 192, 256]
    for dt in args.dtypes:
        for K in args.ks:
            for s in sizes:
                m, x, y, g = make(DT[dt], 64, s, s, K, 7)
                row = {"kind": "path_speed", "dtype": dt, "B": 1, "C": 64, "H": s, "W": s, "K": K,
                       "tokens": s * s}
                for training in (False, True):
                    for path in ("fused", "materialised"):
                        ms = time_fn(step_fn(m, x, y, g, path, training))
                        assert m.last_path == path
                        row[f"{'train' if training else 'infer'}_{path}_ms"] = round(ms, 4)
                row["train_fused_speedup"] = round(row["train_materialised_ms"] / row["train_fused_ms"], 3)
                row["infer_fused_speedup"] = round(row["infer_materialised_ms"] / row["infer_fused_ms"], 3)
                log(row)
                print(json.dumps(row), flush=True)
                del m, x, y, g
                torch.cuda.empty_cache()


def memory_child(dt, path, H, K):
    m, x, y, g = make(DT[dt], 64, H, H, K, 7)
    fn = step_fn(m, x, y, g, path, True)
    fn()  # warm-up: library load, allocator, conv algorithm choice
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    fn()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()
    assert m.last_path == path
    return {"kind": "path_memory", "dtype": dt, "path": path, "B": 1, "C": 64, "H": H, "W": H, "K": K,
            "temporary_peak_MiB": round((peak - base) / 2**20, 1), "resident_MiB": round(base / 2**20, 1)}


def run_memory(args):
    for H in (256, 128):
        for dt in args.dtypes:
            for path in ("fused", "materialised"):
                cmd = [sys.executable, "-m", "dynamic_dilated_depthwise_amd.bench_module", "--memory-child",
                       f"{dt},{path},{H},3"]
                res = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=300)
                if res.returncode != 0:
                    log(res.stderr[-2000:])
                    raise SystemExit(f"memory child failed: {cmd}")
                line = res.stdout.strip().splitlines()[-1]
                log(line)
                print(line, flush=True)


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description="fused vs materialised DDPM: step time and peak temporary memory")
    ap.add_argument("--mode", choices=["speed", "memory", "all"], default="all")
    ap.add_argument("--dtypes", default="f32,bf16", help="comma-separated subset of f32,bf16")
    ap.add_argument("--ks", default="3,5", help="comma-separated kernel sizes for --mode speed")
    ap.add_argument("--memory-child", default=None, metavar="DT,PATH,H,K",
                    help="measure one training step's temporary memory in this process and print one JSON line "
                         "(DT f32|bf16, PATH fused|materialised)")
    args = ap.parse_args(argv)
    args.dtypes = args.dtypes.split(",")
    args.ks = [int(k) for k in args.ks.split(",")]
    for dt in args.dtypes:
        if dt not in DT:
            ap.error(f"unknown dtype {dt!r} (f32, bf16)")
    if args.memory_child:
        parts = args.memory_child.split(",")
        if len(parts) != 4 or parts[0] not in DT or parts[1] not in ("fused", "materialised"):
            ap.error("--memory-child takes DT,PATH,H,K, e.g. f32,fused,128,3")
    return args


def main(argv=None):
    args = parse_args(argv)
    assert torch.cuda.is_available(), "bench_module needs a GPU"
    if args.memory_child:
        dt, path, H, K = args.memory_child.split(",")
        print(json.dumps(memory_child(dt, path, int(H), int(K))), flush=True)
        return
    if args.mode in ("speed", "all"):
        run_speed(args)
    if args.mode in ("memory", "all"):
        run_memory(args)


if __name__ == "__main__":
    main()
