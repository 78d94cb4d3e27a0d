"""Benchmark of the DDPM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--dtype f32|bf16]
                    [--workload target_256] [--no-cpu-baseline] [--no-bf16]

One step is one pass of the whole hot path over one batch of synthetic input
(B=1, C=64, K=3, 256x256 by default):
  1. ddpm_filter_fwd       materialised taps [1, 1728, 256, 256] -> [x, d1, d3, d5]
  2. ddpm_fused_fwd        generator fused with the filter
  3. ddpm_fused_bwd (dX)   tap recompute + gather
  4. ddpm_fused_bwd (dY)   on-chip dK contracted with the generator weight
  5. ddpm_fused_bwd (dW)   on-chip dK reduced into 16 float32 token partials
  6. ddpm_reduce_partials  fixed-order sum of the partials
The backward of the materialised filter (ddpm_filter_bwd: dX and the tap
gradient) is timed the same way right after the steps, outside ms_per_step.
Each library call runs one kernel, so HIP events
recorded around every call on the launch stream give per-kernel durations over
the timed region.  All inputs are resident in HBM before timing starts.

After the steps every kernel is also launched alone, each time right after a 1 GiB
read that flushes L2 and the MALL ("cold": median, p10, p90), and a 1 GiB device
copy gives the attainable-bandwidth ceiling.  With --dtype f32 (the default) the
same measurement is then made for bfloat16 and carried as the line's "bf16"
object (its own steps, per-kernel figures, cold filter TB/s and roofline);
``value`` and ``dtype`` stay those of float32.

Printed on stdout: ONE JSON line.  ``value`` is the filter's effective bandwidth
in TB/s (algorithmic bytes / cold median filter duration; the warm in-step figure
is carried as ``filter_warm_TB_s``); the fused forward and forward+backward times
(in-step), per-kernel figures, the roofline of the dominant kernel (in-step HIP
events, as the kernel trace sees them) and the fp64 oracle timed on the host cores
are carried alongside.  Progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DDPM filter TB/s (% HBM peak) + fused fwd/bwd ms at B=1,C=64,K=3,256²"
HBM_PEAK_GBS = 8000.0             # MI355X HBM3E, 8 TB/s
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6}   # dense MFMA peaks


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic(shape, dtype_bytes, S):
    """Algorithmic bytes / flops per launch (only the method's own work)."""
    N, C, H, W, K = shape.N, shape.C, shape.H, shape.W, shape.K
    P = N * H * W
    R = 3 * C * K * K
    s = dtype_bytes
    gemm = 2.0 * R * C * P
    return {
        # taps + x read, 4 planes written
        "filter": {"bytes": (R + C + 4 * C) * s * P, "flops": 2.0 * R * P},
        # x, y read, out written (+ weight and bias once); one generator contraction
        "fused_fwd": {"bytes": 6 * C * s * P + (R * C + R) * s, "flops": gemm},
        # y, G (4C) read, dX written; generator recompute
        "bwd_dx": {"bytes": 6 * C * s * P + (R * C + R) * s, "flops": gemm},
        # x, G_b (3C) read, dY written; W^T dK
        "bwd_dy": {"bytes": 5 * C * s * P + R * C * s, "flops": gemm},
        # x, y, G_b read, partials written; dK y^T
        "bwd_dw": {"bytes": 5 * C * s * P + S * (R * C + R) * 4, "flops": gemm},
        # partials read, gradients written
        "reduce": {"bytes": S * (R * C + R) * 4 + (R * C + R) * s, "flops": 0.0},
        # materialised backward: x, taps, G (4C) read, dX and dtaps written
        "filter_bwd": {"bytes": (2 * R + 6 * C) * s * P, "flops": 2.0 * (2 * R + C) * P},
    }


KERNEL_BOUND = {"filter": "hbm", "fused_fwd": "mfma", "bwd_dx": "mfma", "bwd_dy": "mfma", "bwd_dw": "mfma",
                "reduce": "hbm", "filter_bwd": "hbm"}

# Kernel symbol and the source files that define it (for the traffic record's digest).
# dX at C = 64 on grids of more than two row segments per CU runs the row-staged
# kernels of bwd_dx_rows.hip (one per dtype); the bfloat16 forward at K = 3, C = 64
# runs the persistent kernel of fused_fwd_pers.hip.
KERNEL_SYMBOL = {"filter": "filter_fwd_kernel",
                 "fused_fwd": {"f32": "fused_fwd_kernel", "bf16": "fused_fwd_pers_kernel"},
                 "bwd_dx": {"f32": "bwd_dx_f32_kernel", "bf16": "bwd_dx_bf16_kernel"},
                 "bwd_dy": {"f32": "bwd_dy_f32_kernel", "bf16": "bwd_dy_bf16_kernel"},
                 "bwd_dw": "bwd_dw_rows_kernel", "reduce": "reduce_partials_kernel",
                 "filter_bwd": "filter_bwd_kernel"}
KERNEL_SOURCES = {
    "filter": ["filter_fwd.hip", "common.hpp"],
    "fused_fwd": ["fused_fwd.hip", "fused_fwd_pers.hip", "gen_mma.hpp", "common.hpp"],
    "bwd_dx": ["bwd_dx.hip", "bwd_dx_rows.hip", "gen_mma.hpp", "common.hpp"],
    "bwd_dy": ["fused_bwd.hip", "bwd_dy_rows.hip", "gen_mma.hpp", "common.hpp"],
    "bwd_dw": ["fused_bwd.hip", "bwd_dw_rows.hip", "gen_mma.hpp", "common.hpp"],
    "reduce": ["reduce.hip", "common.hpp"],
    "filter_bwd": ["filter_bwd.hip", "common.hpp"],
}
CSRC = os.path.join(ROOT, "dynamic_dilated_depthwise_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_digest(name):
    """sha256 over the source files of one kernel, in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(name, workload, dtype):
    """HBM bytes per launch of one kernel from the committed rocprofv3 counter record
    (FETCH_SIZE and WRITE_SIZE, calibrated against a plain copy), or None when there
    is no record or the kernel's sources changed since the counters were taken."""
    path = os.path.join(PROFILES, f"traffic_{workload}_{dtype}.md")
    if not os.path.exists(path):
        return None
    sym = KERNEL_SYMBOL[name]
    if isinstance(sym, dict):
        sym = sym[dtype]
    for line in open(path):
        parts = line.split()
        if len(parts) >= 4 and parts[0] == "traffic:" and parts[1] == sym:
            fields = dict(p.split("=", 1) for p in parts[2:] if "=" in p)
            if fields.get("source") == kernel_source_digest(name):
                return int(fields["bytes"])
            return None
    return None


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (or the platform string)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def run_cpu_baseline(h, shape, min_reps=3, min_s=12.0, max_reps=25):
    """The fp64 oracle on the same inputs: one warm-up step (filter, fused forward,
    fused backward), then timed steps until at least `min_reps` of them and `min_s`
    seconds of oracle work are done (at most `max_reps`); per-part medians."""
    import oracle
    orc = oracle.default()
    a = {k: v.double().numpy() for k, v in h.items()}
    K = shape.K
    parts = {
        "filter": lambda: orc.filter_fwd(a["x"], a["taps"], K),
        "fused_fwd": lambda: orc.fused_fwd(a["x"], a["y"], a["weight"], a["bias"], K),
        "fused_bwd": lambda: orc.fused_bwd(a["x"], a["y"], a["weight"], a["bias"], a["grad_out"], K),
    }
    t = {k: [] for k in parts}
    start = time.perf_counter()
    timed = 0.0
    rep = 0
    while rep <= min_reps or (timed < min_s and rep <= max_reps):
        for name, fn in parts.items():
            t0 = time.perf_counter()
            fn()
            if rep > 0:  # rep 0 is the warm-up
                dt = time.perf_counter() - t0
                t[name].append(dt)
                timed += dt
        rep += 1
    out = {k: sorted(v)[len(v) // 2] for k, v in t.items()}
    out["reps"] = rep - 1
    out["timed_s"] = timed
    out["total_s"] = time.perf_counter() - start
    return out


def measure(args, ddpm, synth, dt_name, log_prefix=""):
    """Time one dtype of the workload: the in-step per-kernel means over
    args.steps whole steps, the materialised backward beside them, and the cold
    launches.  Returns the measurements and the seeded host inputs."""
    dtype = torch.float32 if dt_name == "f32" else torch.bfloat16
    es = 4 if dt_name == "f32" else 2
    shape, block = synth.WORKLOADS[args.workload]
    N, C, H, W, K = shape.N, shape.C, shape.H, shape.W, shape.K
    R = shape.R
    S = ddpm.num_partials_for(N, C, H, W, K)
    log(f"{log_prefix}workload {args.workload} N={N} C={C} H={H} W={W} K={K} dtype={dt_name} S={S}")

    h = synth.make_inputs(shape, block, dtype, taps=True, grad=True)
    d = {k: v.to("cuda").contiguous() for k, v in h.items()}
    out_f = torch.empty((N, 4 * C, H, W), device="cuda", dtype=dtype)
    out = torch.empty_like(out_f)
    gx = torch.empty_like(d["x"])
    gy = torch.empty_like(d["x"])
    pw = torch.empty((S, R, C), device="cuda", dtype=torch.float32)
    pb = torch.empty((S, R), device="cuda", dtype=torch.float32)
    gw = torch.empty((R, C), device="cuda", dtype=dtype)
    gb = torch.empty((R,), device="cuda", dtype=dtype)
    gx_f = torch.empty_like(d["x"])
    gk_f = torch.empty_like(d["taps"])
    stream = torch.cuda.current_stream()

    calls = [
        ("filter", lambda: ddpm.ddpm_filter_fwd(d["x"], d["taps"], out_f, K, stream)),
        ("fused_fwd", lambda: ddpm.ddpm_fused_fwd(d["x"], d["y"], d["weight"], d["bias"], out, K, stream)),
        ("bwd_dx", lambda: ddpm.ddpm_fused_bwd(d["x"], d["y"], d["weight"], d["bias"], d["grad_out"], gx, None,
                                               None, None, K, stream)),
        ("bwd_dy", lambda: ddpm.ddpm_fused_bwd(d["x"], d["y"], d["weight"], d["bias"], d["grad_out"], None, gy,
                                               None, None, K, stream)),
        ("bwd_dw", lambda: ddpm.ddpm_fused_bwd(d["x"], d["y"], d["weight"], d["bias"], d["grad_out"], None, None,
                                               pw, pb, K, stream)),
        ("reduce", lambda: ddpm.ddpm_reduce_partials(pw, pb, gw, gb, K, stream)),
    ]
    # Timed beside the step, not inside it: the backward of the materialised filter
    # (dX and dtaps from the taps), the training counterpart of call 1.
    extra_calls = [
        ("filter_bwd", lambda: ddpm.ddpm_filter_bwd(d["x"], d["taps"], d["grad_out"], gx_f, gk_f, K, stream)),
    ]

    def step(events=None):
        for i, (name, fn) in enumerate(calls):
            if events is not None:
                events[i][0].record(stream)
            fn()
            if events is not None:
                events[i][1].record(stream)

    log(f"{log_prefix}warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K whole steps, events around every call on the launch stream.
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in calls]
          for _ in range(args.steps)]
    log(f"{log_prefix}timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    per = {name: sum(ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps)) / args.steps
           for i, (name, _) in enumerate(calls)}
    log(f"{log_prefix}per-call ms " + " ".join(f"{k}={v:.4f}" for k, v in per.items()))

    # The fused training sequence as a module runs it: the forward, one backward call
    # that launches dX, dY and the dW partials back to back, and the reduction, with
    # one event pair per sequence (the per-call events above add a marker of about
    # 5 us to every kernel they bracket).
    def train_seq():
        ddpm.ddpm_fused_fwd(d["x"], d["y"], d["weight"], d["bias"], out, K, stream)
        ddpm.ddpm_fused_bwd(d["x"], d["y"], d["weight"], d["bias"], d["grad_out"], gx, gy, pw, pb, K, stream)
        ddpm.ddpm_reduce_partials(pw, pb, gw, gb, K, stream)

    for _ in range(args.warmup):
        train_seq()
    sev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e0, e1 in sev:
        e0.record(stream)
        train_seq()
        e1.record(stream)
    torch.cuda.synchronize()
    seq_ts = sorted(e0.elapsed_time(e1) for e0, e1 in sev)
    train_seq_ms = seq_ts[len(seq_ts) // 2]
    log(f"{log_prefix}fused fwd+bwd sequence (one event pair) median ms={train_seq_ms:.4f}")

    for name, fn in extra_calls:
        for _ in range(args.warmup):
            fn()
        xev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for e0, e1 in xev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        per[name] = sum(e0.elapsed_time(e1) for e0, e1 in xev) / args.steps
        log(f"{log_prefix}{name} (outside the step) ms={per[name]:.4f}")

    # Cold launches: each kernel alone after a 1 GiB read that evicts L2 and the MALL
    # with clean lines, so its inputs come from HBM and no write-back of the flush
    # lands inside the timed launch (the step above runs its kernels back to back).
    cold = {}
    if args.cold_reps > 0:
        flush = torch.ones(1 << 28, device="cuda", dtype=torch.float32)
        sink = torch.empty((), device="cuda", dtype=torch.float32)
        for name, fn in calls + extra_calls:
            ts = []
            for _ in range(args.cold_reps):
                torch.sum(flush, dim=0, out=sink)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ts.sort()
            q = lambda f: ts[min(len(ts) - 1, int(round(f * (len(ts) - 1))))]
            cold[name] = {"median": q(0.5), "p10": q(0.1), "p90": q(0.9)}
        del flush, sink
        log(f"{log_prefix}cold median ms " + " ".join(f"{k}={v['median']:.4f}" for k, v in cold.items()))

    alg = algorithmic(shape, es, S)
    peak_t = MFMA_PEAK_TFLOPS[dt_name]
    kernels = {}
    for name, ms in per.items():
        a = alg[name]
        gbs = a["bytes"] / (ms * 1e-3) / 1e9
        tfl = a["flops"] / (ms * 1e-3) / 1e12
        kb = KERNEL_BOUND[name]
        kernels[name] = {
            "ms": round(ms, 5), "bound": kb, "alg_bytes": int(a["bytes"]), "alg_flops": a["flops"],
            "GB_s": round(gbs, 1), "TFLOP_s": round(tfl, 2),
            "frac": round(gbs / HBM_PEAK_GBS if kb == "hbm" else tfl / peak_t, 4),
            "in_step": name not in dict(extra_calls),
        }
        if name in cold:
            c = cold[name]
            kernels[name]["cold_ms"] = {k: round(v, 5) for k, v in c.items()}
            cg = a["bytes"] / (c["median"] * 1e-3) / 1e9
            ct = a["flops"] / (c["median"] * 1e-3) / 1e12
            kernels[name]["cold_frac"] = round(cg / HBM_PEAK_GBS if kb == "hbm" else ct / peak_t, 4)

    dom = max((n for n, _ in calls if n != "reduce"), key=lambda n: per[n])
    kd = kernels[dom]
    traffic = recorded_traffic(dom, args.workload, dt_name)
    if kd["bound"] == "hbm":
        roofline = {"kernel": dom, "bound": "hbm", "achieved": kd["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": kd["frac"], "traffic": traffic}
    else:
        roofline = {"kernel": dom, "bound": "mfma", "achieved": kd["TFLOP_s"], "peak": peak_t, "unit": "TFLOP/s",
                    "frac": kd["frac"], "traffic": traffic}
    for name in kernels:
        kernels[name]["hbm_traffic_bytes"] = recorded_traffic(name, args.workload, dt_name)

    filter_warm_tbs = kernels["filter"]["GB_s"] / 1e3
    if "filter" in cold:
        filter_tbs = alg["filter"]["bytes"] / (cold["filter"]["median"] * 1e-3) / 1e12
        value_timing = (f"median of {args.cold_reps} single filter launches, each after a 1 GiB read that "
                        "flushes L2 and MALL")
    else:
        filter_tbs = filter_warm_tbs
        value_timing = "mean filter launch inside the timed steps (warm)"
    fwd_ms = per["fused_fwd"]
    fwd_bwd_ms = per["fused_fwd"] + per["bwd_dx"] + per["bwd_dy"] + per["bwd_dw"] + per["reduce"]
    gen_tflops = alg["fused_fwd"]["flops"] / (fwd_ms * 1e-3) / 1e12
    res = {
        "dtype": dt_name, "shape": shape, "S": S, "h": h, "alg": alg, "ms_per_step": ms_per_step,
        "value_timing": value_timing, "filter_tbs": filter_tbs, "filter_warm_tbs": filter_warm_tbs,
        "filter_ms": per["filter"], "fwd_ms": fwd_ms, "fwd_bwd_ms": fwd_bwd_ms, "train_seq_ms": train_seq_ms,
        "gen_tflops": gen_tflops,
        "peak_t": peak_t, "kernels": kernels, "roofline": roofline,
    }
    del d, out_f, out, gx, gy, pw, pb, gw, gb, gx_f, gk_f
    torch.cuda.empty_cache()
    return res


def summary(m):
    """The per-dtype figures carried on the JSON line."""
    return {
        "value_TB_s": round(m["filter_tbs"], 4),
        "value_timing": m["value_timing"],
        "ms_per_step": round(m["ms_per_step"], 4),
        "filter_warm_TB_s": round(m["filter_warm_tbs"], 4),
        "filter_ms": round(m["filter_ms"], 5),
        "filter_hbm_frac": round(m["filter_tbs"] * 1e3 / HBM_PEAK_GBS, 4),
        "filter_warm_hbm_frac": m["kernels"]["filter"]["frac"],
        "fused_fwd_ms": round(m["fwd_ms"], 5),
        "fused_fwd_bwd_ms": round(m["fwd_bwd_ms"], 5),
        "fused_fwd_bwd_seq_ms": round(m["train_seq_ms"], 5),
        "fused_fwd_mfma_tflops": round(m["gen_tflops"], 2),
        "fused_fwd_mfma_frac": round(m["gen_tflops"] / m["peak_t"], 4),
        "kernels": m["kernels"],
        "roofline": m["roofline"],
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--dtype", choices=["f32", "bf16"], default="f32")
    ap.add_argument("--workload", default="target_256")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16", action="store_true",
                    help="with --dtype f32, skip the bfloat16 step that is otherwise timed after the float32 one "
                         "and carried as the line's \"bf16\" object")
    ap.add_argument("--copy-calibration-mib", type=int, default=1024,
                    help="before the steps, time a plain device-to-device copy of this many MiB "
                         "(a known-size kernel for scaling HBM counters, and the attainable-bandwidth ceiling); "
                         "0 skips it")
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="after the steps, time each kernel this many times alone, each after a read of "
                         "a 1 GiB buffer that evicts L2 and the MALL (0 skips it)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the DDPM hot path is timed on a single MI355X "
              "(--gpus 1); it has no multi-GPU mode (each GPU would run its own share of the batch).",
              file=sys.stderr)
        sys.exit(2)

    import dynamic_dilated_depthwise_amd as ddpm
    from dynamic_dilated_depthwise_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    stream = torch.cuda.current_stream()

    copy_cal = None
    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib * (1 << 20)
        src = torch.ones(nbytes // 4, device="cuda", dtype=torch.float32)
        dst = torch.empty_like(src)
        times = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = sorted(times)[len(times) // 2]
        copy_cal = {"bytes_read": nbytes, "bytes_written": nbytes, "median_ms": round(ms, 5),
                    "GB_s": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}
        log(f"copy calibration {copy_cal}")
        del src, dst

    m = measure(args, ddpm, synth, args.dtype)
    shape, S = m["shape"], m["S"]
    N, C, H, W, K = shape.N, shape.C, shape.H, shape.W, shape.K
    m_bf16 = None
    if args.dtype == "f32" and not args.no_bf16:
        m_bf16 = measure(args, ddpm, synth, "bf16", log_prefix="bf16: ")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle, one warm-up step then the median of >= 3 timed steps (>= 12 s) on the host cores")
        cores = len(os.sched_getaffinity(0))
        omp = os.environ.get("OMP_NUM_THREADS")
        threads = min(cores, int(omp)) if omp else cores
        t = run_cpu_baseline(m["h"], shape)
        f_bytes = m["alg"]["filter"]["bytes"]
        cpu = {"value": round(f_bytes / t["filter"] / 1e12, 5), "unit": "TB/s", "cores": threads, "kind": "oracle",
               "sample": f"the same {args.workload} workload in fp64 on the host ({cpu_model()}): one warm-up "
                         f"step (filter, fused fwd, fused bwd) then {t['reps']} timed steps, {t['timed_s']:.1f} s "
                         f"timed ({t['total_s']:.1f} s with the warm-up); value is the filter's algorithmic bytes / median oracle filter time",
               "cpu_model": cpu_model(),
               "filter_s": round(t["filter"], 4), "fused_fwd_s": round(t["fused_fwd"], 4),
               "fused_bwd_s": round(t["fused_bwd"], 4), "reps": t["reps"]}
        log(f"cpu baseline {cpu}")

    sm = summary(m)
    line = {
        "metric": METRIC,
        "value": sm.pop("value_TB_s"),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sm.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic (seeded Gaussian tensors of the workload's shapes)",
        "config": {"workload": f"DDPM {args.workload}: B={N} C={C} K={K} {H}x{W}, "
                               "filter + fused fwd + fused bwd (dX, dY, dW partials) + reduce",
                   "N": N, "C": C, "H": H, "W": W, "K": K, "num_partials": S},
    }
    line.update(sm)
    line["cpu_baseline"] = cpu
    if m_bf16 is not None:
        line["bf16"] = summary(m_bf16)
    if copy_cal is not None:
        line["copy_calibration"] = copy_cal
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
