"""GPU parity: NVFP4 / FP8 quantizers (bit-exact against the oracle)."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import quant as Q
from tests.helpers import np_, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("R,C,seed", [(1, 16, 0), (3, 48, 1), (64, 256, 2), (257, 512, 3), (2048, 5120, 4)])
def test_nvfp4_quantize_bf16_bitexact(gpu_lib, R, C, seed):
    x = W.quant_tensor_host((R, C), seed=seed)
    codes, scales, gs = gpu_lib.nvfp4_quantize(to_dev_bf16(x))
    oc, os_, og = Q.nvfp4_quantize(x)
    assert np_(gs)[0] == og
    assert np.array_equal(np_(scales), os_)
    assert np.array_equal(np_(codes), oc)


def test_nvfp4_quantize_f32_input_and_subnormal_scales(gpu_lib):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((96, 320)) * 1e-3).astype(np.float32)
    x[7, 11] = 100.0
    x[9, :16] = 0.0
    x[9, 3] = -0.0
    codes, scales, gs = gpu_lib.nvfp4_quantize(to_dev_f32(x))
    oc, os_, og = Q.nvfp4_quantize(x)
    assert np_(gs)[0] == og and np.array_equal(np_(scales), os_) and np.array_equal(np_(codes), oc)
    assert ((os_ & 0x78) == 0).mean() > 0.3


def test_nvfp4_quantize_batched_and_static(gpu_lib):
    rng = np.random.default_rng(6)
    xs = [W.to_bf16_f32(rng.standard_normal((40, 128)).astype(np.float32) * s) for s in (0.02, 1.0, 300.0)]
    x = np.stack(xs)
    codes, scales, gs = gpu_lib.nvfp4_quantize(to_dev_bf16(x))
    for b in range(3):
        oc, os_, og = Q.nvfp4_quantize(xs[b])
        assert np_(gs)[b] == og and np.array_equal(np_(scales)[b], os_) and np.array_equal(np_(codes)[b], oc)
    static = torch.tensor([1e-3, 0.5, 2.0], dtype=torch.float32, device="cuda")
    codes, scales, gs = gpu_lib.nvfp4_quantize(to_dev_bf16(x), global_scale=static)
    for b in range(3):
        oc, os_, og = Q.nvfp4_quantize(xs[b], global_scale=np.float32(np_(static)[b]))
        assert np.array_equal(np_(scales)[b], os_) and np.array_equal(np_(codes)[b], oc)


def test_nvfp4_zero_tensor(gpu_lib):
    x = np.zeros((5, 32), np.float32)
    codes, scales, gs = gpu_lib.nvfp4_quantize(to_dev_bf16(x))
    assert np_(gs)[0] == 0 and not np_(scales).any() and not np_(codes).any()


def test_nvfp4_dequantize_bitexact(gpu_lib):
    x = W.quant_tensor_host((300, 640), seed=7)
    codes, scales, gs = gpu_lib.nvfp4_quantize(to_dev_bf16(x))
    d = gpu_lib.nvfp4_dequantize(codes, scales, gs)
    ref = Q.nvfp4_dequantize_f32(np_(codes), np_(scales), np_(gs)[0])
    assert np.array_equal(np_(d).view(np.uint32), ref.view(np.uint32))


def test_nvfp4_standalone_workload_full_size_sampled(gpu_lib):
    """32768 x 5120 Student-t tensor with outlier rows: full GPU run, oracle on sampled rows."""
    x = W.quant_tensor_device()
    codes, scales, gs = gpu_lib.nvfp4_quantize(x)
    d = gpu_lib.nvfp4_dequantize(codes, scales, gs)
    torch.cuda.synchronize()
    amax = float(x.abs().max().float())
    og = np.float32(np.float32(amax) / np.float32(2688))
    assert np_(gs)[0] == og
    rows = np.random.default_rng(8).choice(x.shape[0], 96, replace=False)
    xs = x[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    oc, os_, _ = Q.nvfp4_quantize(xs, global_scale=og)
    assert np.array_equal(np_(codes)[rows], oc)
    assert np.array_equal(np_(scales)[rows], os_)
    ref = Q.nvfp4_dequantize_f32(oc, os_, og)
    assert np.array_equal(np_(d)[rows].view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("R,C,bf16", [(1, 4, True), (64, 5120, True), (33, 2560, False), (7, 100, False)])
def test_fp8_quantize_bitexact(gpu_lib, R, C, bf16):
    x = W.quant_tensor_host((R, C), seed=R + C)
    if not bf16:
        x = (x * np.float32(1.2345671)).astype(np.float32)
    if R > 3:
        x[2] = 0.0
    codes, scales = gpu_lib.fp8_quantize(to_dev_bf16(x) if bf16 else to_dev_f32(x))
    oc, os_ = Q.fp8_quantize(x)
    assert np.array_equal(np_(scales), os_)
    assert np.array_equal(np_(codes), oc)
