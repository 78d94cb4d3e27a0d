"""GPU parity: the HIP library against the fp64 oracle, element by element.

Every case draws seeded inputs (``dynamic_dilated_depthwise_amd.synth``), runs the
library through its C ABI (via the thin binding) on the GPU and the oracle on the
host on exactly the same values, and compares whole tensors:
  * the named workloads at their full sizes (1x64x128^2 K=3 filter, 1x64x256^2
    K=3 fused forward / backward, 1x64x128^2 K=5 training) in the launch
    configuration the benchmark times;
  * small and ragged shapes that span several tiles with partial tiles at the
    right and bottom edges, K = 1, 3, 5, images smaller than the dilation reach,
    channel counts that are not multiples of the MFMA block, more than 64
    channels (the streamed generator path), the largest channel count, and
    tensors whose pointers are only element-aligned.
Tolerances are in ``gpu_cases.py``.
"""
import numpy as np
import pytest
import torch

import dynamic_dilated_depthwise_amd as ddpm
from dynamic_dilated_depthwise_amd import synth
from gpu_cases import (TOL, announce, assert_close, dev, f64, gpu_bwd, gpu_filter, gpu_filter_bwd, gpu_fused, inputs,
                       orc)

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}
S_ = synth.Shape

FWD_CASES = [
    ("tiny", None), ("nonaligned", None), ("bw_filter_128", None), ("fused_inference_256", None),
    ("fused_training_128_k5", None),
    ("k1", (S_(1, 8, 16, 16, 1), 101)), ("k5", (S_(1, 8, 16, 16, 5), 102)),
    ("nonaligned_k5", (S_(2, 24, 15, 17, 5), 103)), ("nonaligned_k1", (S_(2, 24, 15, 17, 1), 104)),
    ("one_pixel", (S_(1, 1, 1, 1, 3), 105)), ("one_row_k5", (S_(1, 3, 1, 7, 5), 106)),
    ("smaller_than_reach", (S_(1, 5, 3, 3, 3), 107)), ("ragged_tiles", (S_(3, 16, 9, 65, 3), 108)),
    ("c33", (S_(1, 33, 10, 8, 3), 109)), ("c70_streamed", (S_(1, 70, 12, 20, 3), 110)),
    ("c1024_max", (S_(1, 1024, 2, 2, 3), 111)), ("c2_k5_tall", (S_(2, 2, 37, 6, 5), 112)),
    ("c48_ragged", (S_(1, 48, 12, 70, 3), 113)), ("c64_w200_k5", (S_(1, 64, 9, 200, 5), 114)),
    # rows wider than one tile (several column tiles; the checked backward dX path)
    ("w520_wide", (S_(1, 4, 6, 520, 3), 115)), ("w1030_k5", (S_(1, 3, 5, 1030, 5), 116)),
    # rows of 256+ pixels with W % 8 == 0 (8-pixel bfloat16 runs) at K = 5 and K = 1
    ("w256_k5", (S_(1, 6, 13, 256, 5), 118)), ("w264_k1", (S_(2, 5, 3, 264, 1), 119)),
    # a batch of four mid-size images on the workload's channel count (full-size grids)
    ("batch4_c64_64", (S_(4, 64, 64, 64, 3), 117)),
    # bfloat16 K = 3, C = 64 with W % 8 == 0 (the persistent forward): ragged last row
    # band and column tile in a batch of two with uneven tile runs per workgroup, a
    # batch of three with an 8-column last tile, fewer tiles than workgroups, and an
    # image narrower and shorter than one tile
    ("c64_pers_ragged", (S_(2, 64, 130, 200, 3), 120)), ("c64_pers_batch3_w136", (S_(3, 64, 64, 136, 3), 121)),
    ("c64_pers_few_tiles", (S_(1, 64, 10, 72, 3), 122)), ("c64_pers_w8_h3", (S_(2, 64, 3, 8, 3), 123)),
    # the same channel count with W % 8 != 0: bfloat16 stays on the per-tile kernel
    ("c64_w68_per_tile", (S_(1, 64, 12, 68, 3), 124)),
]

BWD_CASES = [
    ("tiny", None), ("nonaligned", None), ("fused_training_128_k5", None), ("target_256", None),
    ("k1", (S_(1, 8, 16, 16, 1), 201)), ("k5", (S_(1, 8, 16, 16, 5), 202)),
    ("nonaligned_k5", (S_(2, 24, 15, 17, 5), 203)),
    ("one_pixel", (S_(1, 1, 1, 1, 3), 205)), ("smaller_than_reach", (S_(1, 5, 3, 3, 3), 207)),
    ("ragged_tiles", (S_(3, 16, 9, 65, 3), 208)), ("c33", (S_(1, 33, 10, 8, 3), 209)),
    ("c70_streamed", (S_(1, 70, 12, 20, 3), 210)), ("c2_k5_tall", (S_(2, 2, 37, 6, 5), 212)),
    ("c48_ragged", (S_(1, 48, 12, 70, 3), 213)), ("c64_w200_k5", (S_(1, 64, 9, 200, 5), 214)),
    ("batch4_c64_64", (S_(4, 64, 64, 64, 3), 215)),
    # grids of more than two workgroups per CU (four-wave dY, one wave group in dX)
    # at K = 5 and with a partial channel block count (C = 24, ragged rows)
    ("k5_large_grid", (S_(1, 64, 160, 256, 5), 216)), ("c24_large_grid", (S_(1, 24, 150, 300, 3), 217)),
    # two 64-channel blocks at K = 1, and a grid of two workgroups per CU (eight-wave
    # dY, two wave groups in dX) on the workload's channel count
    ("c128_k1_w64", (S_(1, 128, 12, 64, 1), 218)), ("c64_mid_grid", (S_(1, 64, 96, 192, 3), 219)),
    # C = 64 grids of more than two row segments per CU (the row-staged bf16 dX):
    # a partial last segment (100 = 64 + 36 columns) in a batch of two, K = 1 with one
    # segment per row, and K = 5 with a ragged 200-column row and 130 rows
    ("c64_w100_batch2", (S_(2, 64, 160, 100, 3), 220)), ("c64_k1_tall", (S_(1, 64, 520, 64, 1), 221)),
    ("c64_k5_w200", (S_(1, 64, 130, 200, 5), 222)),
    # C = 64 grids of at least one 256-pixel segment per CU (the row-staged bf16 dY):
    # K = 5 on a ragged 200-column row, two segments (256 + 8 columns), and a batch of
    # two at K = 1 with a ragged 136-column row
    ("c64_k5_w200_tall", (S_(1, 64, 264, 200, 5), 223)), ("c64_w264_two_seg", (S_(1, 64, 130, 264, 3), 224)),
    ("c64_k1_batch2_w136", (S_(2, 64, 128, 136, 1), 225)),
    # images shorter than the K = 5 reach (rows up to 10 away): on the row-staged
    # kernels most stages lie above or below the image at once
    ("c64_k5_short_images", (S_(16, 64, 8, 128, 5), 229)),
    # C = 64 grids too small for the 128-pixel halves (the bf16 dY quarters: 64-pixel
    # segments x 16 output channels): one segment per row, a ragged second segment at
    # K = 5, and K = 1 with a ragged 120-column row
    ("c64_64_quarters", (S_(1, 64, 64, 64, 3), 226)), ("c64_k5_w96_quarters", (S_(1, 64, 96, 96, 5), 227)),
    ("c64_k1_w120_quarters", (S_(1, 64, 40, 120, 1), 228)),
]


def _resolve(name, spec):
    return synth.WORKLOADS[name] if spec is None else spec


_ref_cache = {}


def _fwd_ref(key, a, K, taps):
    if key not in _ref_cache:
        o = orc()
        if taps:
            _ref_cache[key] = o.filter_fwd(a["x"], a["taps"], K)
        else:
            _ref_cache[key] = o.fused_fwd(a["x"], a["y"], a["weight"], a["bias"], K)
    return _ref_cache[key]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("name,spec", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_filter_fwd(name, spec, dt):
    shape, block = _resolve(name, spec)
    dtype = DT[dt]
    h = inputs(shape, block, dtype, taps=True)
    a = {k: f64(v) for k, v in h.items()}
    ref = _fwd_ref(("filter", name, dt), a, shape.K, taps=True)
    announce("filter_fwd", name, dt, shape)
    d = dev(h)
    out = gpu_filter(d, shape.K)
    C = shape.C
    assert torch.equal(out[:, :C].cpu().view(torch.int16 if dt == "bf16" else torch.int32),
                       h["x"].view(torch.int16 if dt == "bf16" else torch.int32)), "x block not bit-exact"
    assert_close(f64(out), ref, TOL[dtype]["out"], f"filter {name} {dt}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("name,spec", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_fused_fwd(name, spec, dt):
    shape, block = _resolve(name, spec)
    dtype = DT[dt]
    h = inputs(shape, block, dtype)
    a = {k: f64(v) for k, v in h.items()}
    ref = _fwd_ref(("fused", name, dt), a, shape.K, taps=False)
    announce("fused_fwd", name, dt, shape)
    out = gpu_fused(dev(h), shape.K)
    C = shape.C
    assert torch.equal(out[:, :C].cpu(), h["x"]), "x block not bit-exact"
    assert_close(f64(out), ref, TOL[dtype]["out"], f"fused {name} {dt}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("name,spec", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_fused_bwd(name, spec, dt):
    shape, block = _resolve(name, spec)
    dtype = DT[dt]
    h = inputs(shape, block, dtype, grad=True)
    a = {k: f64(v) for k, v in h.items()}
    refs = orc().fused_bwd(a["x"], a["y"], a["weight"], a["bias"], a["grad_out"], shape.K)
    announce("fused_bwd", name, dt, shape)
    gx, gy, gw, gb, _, _ = gpu_bwd(dev(h), shape.K)
    tol = TOL[dtype]["grad"]
    for what, got, ref in zip(("dx", "dy", "dweight", "dbias"), (gx, gy, gw, gb), refs):
        assert_close(f64(got), ref, tol, f"{what} {name} {dt}")


def _check_filter_bwd(gx, gk, ref, dtype, what):
    rdx, rdk = ref
    if gk is not None:
        exact = torch.from_numpy(rdk).to(dtype)
        bad = (gk.cpu() != exact)
        assert not bool(bad.any()), f"{what}: dtaps differs from the rounded exact product at " \
            f"{int(bad.sum())} elements"
    if gx is not None:
        assert_close(f64(gx), rdx, TOL[dtype]["grad"], f"{what} dx")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("name,spec", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_filter_bwd(name, spec, dt):
    shape, block = _resolve(name, spec)
    dtype = DT[dt]
    h = inputs(shape, block, dtype, taps=True, grad=True)
    a = {k: f64(v) for k, v in h.items()}
    ref = orc().filter_bwd(a["x"], a["taps"], a["grad_out"], shape.K)
    announce("filter_bwd", name, dt, shape)
    gx, gk = gpu_filter_bwd(dev(h), shape.K)
    _check_filter_bwd(gx, gk, ref, dtype, f"filter_bwd {name} {dt}")


FILTER_BWD_ONE_OUTPUT = ["nonaligned", "nonaligned_k5", "ragged_tiles", "one_row_k5", "c2_k5_tall", "c64_w200_k5",
                         "w520_wide"]


@pytest.mark.parametrize("want", ["dx", "dk"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("name", FILTER_BWD_ONE_OUTPUT)
def test_filter_bwd_one_output(name, dt, want):
    """Requesting one gradient runs a separate kernel instance; it must give the
    same values as the oracle (and hence as the instance computing both)."""
    spec = dict(FWD_CASES)[name]
    shape, block = _resolve(name, spec)
    dtype = DT[dt]
    h = inputs(shape, block, dtype, taps=True, grad=True)
    a = {k: f64(v) for k, v in h.items()}
    ref = orc().filter_bwd(a["x"], a["taps"], a["grad_out"], shape.K)
    announce("filter_bwd", want, name, dt, shape)
    gx, gk = gpu_filter_bwd(dev(h), shape.K, want_dx=want == "dx", want_dk=want == "dk")
    assert (gx is None) == (want != "dx") and (gk is None) == (want != "dk")
    _check_filter_bwd(gx, gk, ref, dtype, f"filter_bwd[{want}] {name} {dt}")


@pytest.mark.parametrize("shape", [S_(1, 64, 20, 72, 3), S_(2, 64, 9, 136, 3)], ids=["20x72", "batch2_9x136"])
def test_persistent_forward_bit_identical_to_per_tile(shape):
    """The persistent bf16 forward (K = 3, C = 64, 16-byte aligned tensors) and the
    per-tile kernel (taken when a pointer is only element-aligned) compute the same
    MFMA fragments, the same rounded taps and the same pair sums in the same order:
    their outputs agree bit for bit."""
    h = inputs(shape, 304, torch.bfloat16)

    def shifted(t):
        buf = torch.empty(t.numel() + 1, device="cuda", dtype=t.dtype)
        v = buf[1:].view(t.shape)
        v.copy_(t.to("cuda"))
        return v

    announce("persistent vs per-tile", shape)
    aligned = gpu_fused(dev(h), shape.K)
    d = {k: shifted(v) for k, v in h.items()}
    assert d["x"].data_ptr() % 16 != 0
    per_tile = gpu_fused(d, shape.K)
    torch.cuda.synchronize()
    assert torch.equal(aligned.view(torch.int16), per_tile.view(torch.int16))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_misaligned_pointers(dt):
    """Element-aligned (not 16-byte aligned) tensors take the scalar/unaligned paths."""
    dtype = DT[dt]
    shape = S_(2, 24, 15, 16, 3)
    h = inputs(shape, 301, dtype, taps=True, grad=True)
    a = {k: f64(v) for k, v in h.items()}

    def shifted(t):
        buf = torch.empty(t.numel() + 1, device="cuda", dtype=t.dtype)
        v = buf[1:].view(t.shape)
        v.copy_(t.to("cuda"))
        return v

    d = {k: shifted(v) for k, v in h.items()}
    assert d["x"].data_ptr() % 16 != 0
    announce("misaligned", dt, shape)
    o = orc()
    K = shape.K
    assert_close(f64(gpu_filter(d, K)), o.filter_fwd(a["x"], a["taps"], K), TOL[dtype]["out"], "filter")
    assert_close(f64(gpu_fused(d, K)), o.fused_fwd(a["x"], a["y"], a["weight"], a["bias"], K),
                 TOL[dtype]["out"], "fused")
    refs = o.fused_bwd(a["x"], a["y"], a["weight"], a["bias"], a["grad_out"], K)
    got = gpu_bwd(d, K)[:4]
    for what, g_, r_ in zip(("dx", "dy", "dweight", "dbias"), got, refs):
        assert_close(f64(g_), r_, TOL[dtype]["grad"], what)
    gx, gk = gpu_filter_bwd(d, K)
    _check_filter_bwd(gx, gk, o.filter_bwd(a["x"], a["taps"], a["grad_out"], K), dtype, "filter_bwd")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [S_(2, 24, 15, 17, 3), S_(1, 16, 20, 64, 3), S_(1, 64, 20, 72, 3)],
                         ids=["w17", "w64", "c64_w72"])
@pytest.mark.parametrize("S", [1, 3, 7, 16])
def test_partial_counts_agree(S, shape, dt):
    """Any split count gives the same reduced gradients.  With W = 64 the split
    boundaries fall at odd and even columns of aligned rows (vector run paths); with
    C = 64 and W = 72 the segment-staged kernel walks ranges that start mid-row and
    rows that end in a partial segment."""
    dtype = DT[dt]
    h = inputs(shape, 302, dtype, grad=True)
    a = {k: f64(v) for k, v in h.items()}
    _, _, dW, db = orc().fused_bwd(a["x"], a["y"], a["weight"], a["bias"], a["grad_out"], shape.K)
    announce("partials", S, shape, dt)
    _, _, gw, gb, pw, pb = gpu_bwd(dev(h), shape.K, S=S)
    tol = TOL[dtype]["grad"]
    assert_close(f64(gw), dW, tol, f"dweight S={S}")
    assert_close(f64(gb), db, tol, f"dbias S={S}")
    # the reduce kernel is an ascending-order fp32 sum of the partials
    ref = pw.cpu().double().sum(0).numpy()
    assert_close(f64(gw), ref, 1e-6 if dt == "f32" else 4e-3, "reduce of partials")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [S_(1, 8, 37, 45, 3), S_(1, 64, 37, 48, 3)], ids=["c8", "c64"])
def test_partials_follow_documented_ranges(shape, dt):
    """Each partial holds the sum over the token range the header documents: range s
    starts at floor(T*s/S) rounded down to 64 (float32) / 128 (bfloat16) tokens and
    the last ends at T.  The expected partial s is the oracle's gradient with
    grad_out zeroed outside range s (a token's dK, hence its contribution, is
    proportional to grad_out at that token).  C = 64 takes the segment-staged
    kernel."""
    dtype = DT[dt]
    S = 5
    K, T = shape.K, shape.N * shape.H * shape.W
    h = inputs(shape, 303, dtype, grad=True)
    a = {k: f64(v) for k, v in h.items()}
    announce("partial ranges", S, shape, dt)
    _, _, _, _, pw, pb = gpu_bwd(dev(h), K, S=S)
    step = 64 if dt == "f32" else 128
    starts = [T * s // S // step * step for s in range(S)] + [T]
    assert len(set(starts)) == S + 1  # the case has no empty range
    tol = TOL[dtype]["grad"]
    for s in range(S):
        mask = np.zeros(T)
        mask[starts[s]:starts[s + 1]] = 1.0
        g = a["grad_out"] * mask.reshape(shape.N, 1, shape.H, shape.W)
        _, _, dW, db = orc().fused_bwd(a["x"], a["y"], a["weight"], a["bias"], g, K)
        assert_close(f64(pw[s]), dW, tol, f"dweight partial {s} [{starts[s]}, {starts[s + 1]})")
        assert_close(f64(pb[s]), db, tol, f"dbias partial {s} [{starts[s]}, {starts[s + 1]})")


@pytest.mark.parametrize("name", ["nonaligned", "fused_training_128_k5"])
def test_bitwise_deterministic(name):
    shape, block = synth.WORKLOADS[name]
    d = dev(inputs(shape, block, torch.float32, grad=True, taps=True))
    announce("determinism", name)
    r1 = (gpu_filter(d, shape.K), gpu_fused(d, shape.K), *gpu_bwd(d, shape.K), *gpu_filter_bwd(d, shape.K))
    r2 = (gpu_filter(d, shape.K), gpu_fused(d, shape.K), *gpu_bwd(d, shape.K), *gpu_filter_bwd(d, shape.K))
    for u, v in zip(r1, r2):
        assert torch.equal(u, v)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_finite_difference_spot_check(dt):
    """<grad, v> from the GPU backward equals the central difference of
    L = <G, out> evaluated from GPU forwards; exact in exact arithmetic because L
    is affine in each of x, y, weight, bias taken alone.  In bfloat16 the perturbed
    tensors are rounded to bfloat16, so the direction is their exact difference,
    and the tap and output rounding add noise of about 2^-9 per term."""
    shape, block = synth.WORKLOADS["nonaligned"]
    dtype = DT[dt]
    h = inputs(shape, block, dtype, grad=True)
    d = dev(h)
    K = shape.K
    announce("fd", shape, dt)
    gx, gy, gw, gb, _, _ = gpu_bwd(d, K)
    grads = {"x": gx, "y": gy, "weight": gw, "bias": gb}
    G = f64(d["grad_out"])
    gen = torch.Generator().manual_seed(7)
    for name in ("x", "y", "weight", "bias"):
        v = torch.randn(d[name].shape, generator=gen).to("cuda")
        eps = 0.25
        base = d[name].double()
        tp = (base + eps * v).to(dtype).contiguous()
        tm = (base - eps * v).to(dtype).contiguous()
        Lp = float((f64(gpu_fused(dict(d, **{name: tp}), K)) * G).sum())
        Lm = float((f64(gpu_fused(dict(d, **{name: tm}), K)) * G).sum())
        delta = f64(tp) - f64(tm)  # = 2 eps v in float32
        fd = Lp - Lm
        gv = f64(grads[name])
        an = float((gv * delta).sum())
        # Cauchy-Schwarz scale of <grad, delta>.  A wrong or missing gradient term
        # moves <grad, delta> by about scale / sqrt(elements) (1e-2 of it here);
        # rounding keeps |fd - an| below 2e-5 of it in float32 and 1e-3 in bfloat16.
        scale = float(np.linalg.norm(gv) * np.linalg.norm(delta))
        tol = 2e-5 if dt == "f32" else 1e-3
        assert abs(fd - an) <= tol * scale + 1e-2, f"FD {name}: {fd} vs {an} (scale {scale:.3g})"


# Special values in x: the x block of both forward outputs is a copy of x, so every
# bit pattern must come through unchanged (signed zeros, infinities, NaNs with
# payloads and the sign bit set, subnormals), whatever the other blocks hold.
_SPECIAL_F32 = [0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00001, 0xFFA5A5A5, 0x7F800001,
                0x00000001, 0x807FFFFF, 0x3F800000]
_SPECIAL_BF16 = [0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC1, 0xFFA5, 0x7F81, 0x0001, 0x807F, 0x3F80]


def _with_specials(x, dt, seed):
    g = torch.Generator().manual_seed(seed)
    n = x.numel()
    pos = torch.randperm(n, generator=g)[: max(1, n // 7)]
    if dt == torch.float32:
        bits = x.view(torch.int32).reshape(-1).clone()
        pat = torch.tensor(_SPECIAL_F32, dtype=torch.int64).to(torch.int32)
    else:
        bits = x.view(torch.int16).reshape(-1).clone()
        pat = torch.tensor(_SPECIAL_BF16, dtype=torch.int64).to(torch.int16)
    bits[pos] = pat[torch.arange(pos.numel()) % pat.numel()]
    return bits.view(x.dtype).reshape(x.shape)


@pytest.mark.parametrize("path", ["filter", "fused"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [S_(2, 24, 15, 17, 3), S_(1, 64, 9, 130, 5), S_(1, 16, 6, 64, 1)],
                         ids=["nonaligned_k3", "c64_w130_k5", "w64_k1"])
def test_x_block_bit_exact_specials(shape, dt, path):
    dtype = DT[dt]
    h = inputs(shape, 301, dtype, taps=(path == "filter"))
    h["x"] = _with_specials(h["x"], dtype, 302)
    d = dev(h)
    announce("x block specials", path, dt, shape)
    out = gpu_filter(d, shape.K) if path == "filter" else gpu_fused(d, shape.K)
    ibits = torch.int32 if dtype == torch.float32 else torch.int16
    got = out[:, : shape.C].contiguous().cpu().view(ibits)
    want = h["x"].contiguous().view(ibits)
    assert torch.equal(got, want), f"x block differs in {int((got != want).sum())} elements"
