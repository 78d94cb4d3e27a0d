"""Host logic of the DDPM module: path choice, and CPU tensors taking the CPU path (no GPU)."""
import pytest
import torch

from dynamic_dilated_depthwise_amd.module import AUTO_MIN_TOKENS, DDPM, auto_min_tokens, choose_path

F32, BF16 = torch.float32, torch.bfloat16


def test_thresholds_table():
    for mode in ("train", "infer"):
        for dt in (F32, BF16):
            for K in (3, 5):
                assert (mode, dt, K) in AUTO_MIN_TOKENS
    assert auto_min_tokens(True, F32, 1) == auto_min_tokens(True, F32, 3)
    assert auto_min_tokens(True, BF16, 5) == 1      # measured: fused faster at every size
    assert auto_min_tokens(True, F32, 5) == 9216    # measured: fused faster from 96^2
    assert auto_min_tokens(True, F32, 3) == 1       # measured: fused faster at every size


def test_inference_path():
    assert choose_path(False, 10, 3, F32, F32, F32, False) == "fused"
    assert choose_path(False, 10, 5, BF16, BF16, BF16, False) == "fused"
    assert choose_path(False, 10, 5, F32, F32, F32, False) == "fused"
    assert choose_path(False, 10, 5, F32, F32, F32, False, min_tokens=11) == "materialised"
    assert choose_path(False, 10, 5, F32, F32, F32, False, fused_inference=True) == "fused"
    assert choose_path(False, 10, 3, F32, F32, F32, False, fused_inference=False) == "materialised"
    assert choose_path(False, 10, 3, F32, F32, F32, True) == "materialised"           # autocast
    assert choose_path(False, 10, 3, BF16, F32, F32, False) == "materialised"         # dtype mismatch
    assert choose_path(False, 10, 3, BF16, F32, F32, False, fused_inference=True) == "materialised"


def test_training_path():
    big = 1 << 20
    assert choose_path(True, big, 3, F32, F32, F32, False) == "fused"
    assert choose_path(True, 100, 3, F32, F32, F32, False) == "fused"
    assert choose_path(True, 100, 5, F32, F32, F32, False) == "materialised"
    assert choose_path(True, 9216, 5, F32, F32, F32, False) == "fused"
    assert choose_path(True, 9215, 5, F32, F32, F32, False) == "materialised"
    assert choose_path(True, 100, 3, BF16, BF16, BF16, False) == "fused"
    assert choose_path(True, 100, 5, BF16, BF16, BF16, False) == "fused"
    assert choose_path(True, 100, 5, BF16, BF16, BF16, False, min_tokens=101) == "materialised"
    assert choose_path(True, big, 5, BF16, BF16, BF16, False) == "fused"
    assert choose_path(True, big, 3, F32, F32, F32, True) == "materialised"           # autocast
    assert choose_path(True, big, 3, F32, F32, BF16, False) == "materialised"         # dtype mismatch
    assert choose_path(True, big, 3, F32, F32, F32, False, fused_training=False) == "materialised"
    assert choose_path(True, 1, 3, F32, F32, F32, False, fused_training=True) == "fused"
    assert choose_path(True, 10, 3, F32, F32, F32, False, min_tokens=11) == "materialised"
    assert choose_path(True, 11, 3, F32, F32, F32, False, min_tokens=11) == "fused"
    with pytest.raises(ValueError):
        choose_path(True, big, 3, F32, BF16, F32, False, fused_training=True)


def test_module_shapes_and_refusals():
    m = DDPM(dim=8, kernel_size=3)
    assert tuple(m.generator.weight.shape) == (3 * 8 * 9, 8, 1, 1)
    assert tuple(m.fuse.weight.shape) == (8, 32, 3, 3)
    with pytest.raises(ValueError):
        DDPM(dim=8, kernel_size=4)
    x = torch.randn(1, 8, 6, 6)
    out = m(x, x)                       # CPU tensors: the module's CPU path
    assert tuple(out.shape) == (1, 8, 6, 6) and m.last_path == "cpu_direct"
    # the library's autograd functions take device tensors only
    from dynamic_dilated_depthwise_amd.module import ddpm_fused
    w = m.generator.weight.view(3 * 8 * 9, 8)
    with pytest.raises(RuntimeError, match="CPU path"):
        ddpm_fused(x, x, w, m.generator.bias, 3)
