"""GPU parity: NVFP4 / FP8 quantizers (bit-exact against the oracle)."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import quant as Q
from oracle import quant_c as QC
from tests.fullsize import bf16_bits
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


def _nbrs(v, k=2):
    """v and its float32 neighbours up to k ulps either way (positive v)."""
    v = np.asarray(v, np.float32)
    out, up, lo = [v], v, v
    for _ in range(k):
        up, lo = np.nextafter(up, np.float32(np.inf)), np.nextafter(lo, np.float32(0))
        out += [up, lo]
    return np.concatenate(out)


def test_nvfp4_quantize_decision_points(gpu_lib):
    """Values at and next to every decision point of the encoding, bit-exact against the oracle (f32
    input, static global scales): every E2M1 rounding point of x / d2, d2 = s_b S_g, for block scales
    across the E4M3 range and several global scales, and every E4M3 rounding point of the block scale."""
    t = np.float64([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for S in (1.0, 1.0 / 6.0, 3.7e-3, 2.0 ** -20, 0.73):
        S = np.float32(S)
        # one block per scale code: element 0 sets the block maximum (the scale); the oracle's scale of
        # that block gives the d2 whose decision points the other 15 elements then sit on
        tops = (np.float32(6.0) * F.E4M3_MAGNITUDES[1:127].astype(np.float32) * S).astype(np.float32)
        probe = np.zeros((len(tops), 16), np.float32)
        probe[:, 0] = tops
        sc = Q.nvfp4_quantize(probe, global_scale=S)[1].ravel()
        rows = []
        for top, code in zip(tops, sc):
            d2 = np.float32(np.float32(F.E4M3_MAGNITUDES[code]) * S)
            a = _nbrs((t * np.float64(d2)).astype(np.float32))
            a = np.concatenate([a, -a])
            a = a[np.abs(a) <= top]
            for i in range(0, len(a), 15):
                blk = np.zeros(16, np.float32)
                blk[0] = top
                blk[1:1 + len(a[i:i + 15])] = a[i:i + 15]
                rows.append(blk)
        n = len(rows) // 8 * 8
        x = np.stack(rows[:n]).reshape(n // 8, 128)
        codes, scales, _ = gpu_lib.nvfp4_quantize(to_dev_f32(x), global_scale=torch.tensor([S], device="cuda"))
        oc, os_, _ = Q.nvfp4_quantize(x, global_scale=S)
        assert np.array_equal(np_(scales), os_), S
        assert np.array_equal(np_(codes), oc), S
    # every E4M3 rounding point of the block scale: S = fl32(1/6) makes fl32(6 S) = 1
    S = np.float32(1.0 / 6.0)
    tab = F.E4M3_MAGNITUDES
    amax = _nbrs(((tab[1:-1] + tab[2:]) / 2).astype(np.float32), 1)
    x = np.zeros((len(amax), 16), np.float32)
    x[:, 5] = amax
    x[:, 9] = -amax * np.float32(0.37)
    x = x[: len(amax) // 8 * 8].reshape(-1, 128)
    codes, scales, _ = gpu_lib.nvfp4_quantize(to_dev_f32(x), global_scale=torch.tensor([S], device="cuda"))
    oc, os_, _ = Q.nvfp4_quantize(x, global_scale=S)
    assert np.array_equal(np_(scales), os_) and np.array_equal(np_(codes), oc)


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


def test_nvfp4_standalone_workload_full_size(gpu_lib):
    """32768 x 5120 Student-t tensor with outlier rows: every code, block scale and dequantized value
    (float32 and BF16 outputs) bit-exact against the oracle's own quantization of the same bf16 tensor."""
    x = W.quant_tensor_device()
    codes, scales, gs = gpu_lib.nvfp4_quantize(x)
    d32 = gpu_lib.nvfp4_dequantize(codes, scales, gs)
    torch.cuda.synchronize()
    oc, os_, og = QC.nvfp4_quantize(bf16_bits(x))
    assert np_(gs)[0].view(np.uint32) == og.view(np.uint32)
    assert np.array_equal(np_(codes), oc)
    assert np.array_equal(np_(scales), os_)
    ref = Q.nvfp4_dequantize_f32(oc, os_, og)
    assert np.array_equal(np_(d32).view(np.uint32), ref.view(np.uint32))
    del d32, ref
    rows = slice(0, 4096)
    d16 = gpu_lib.nvfp4_dequantize(codes[rows], scales[rows], gs, out_dtype=torch.bfloat16)
    ref16 = Q.nvfp4_dequantize_bf16(oc[rows], os_[rows], og)
    assert np.array_equal(np_(d16.float()).view(np.uint32), ref16.view(np.uint32))


def test_nvfp4_dequantize_bf16_rounds_once(gpu_lib):
    """BF16 output rounds the exact product q * s_b * S_g once: a global scale with a full 24-bit
    significand makes most products inexact in BF16, and some land on or near BF16 midpoints."""
    x = W.quant_tensor_host((256, 512), seed=9)
    codes, scales, gs = gpu_lib.nvfp4_quantize(to_dev_bf16(x))
    for g in (np_(gs)[0], np.float32(1.0 + 2.0 ** -9 + 2.0 ** -23), np.float32(3.0e-39)):
        gt = torch.tensor([g], dtype=torch.float32, device="cuda")
        d16 = gpu_lib.nvfp4_dequantize(codes, scales, gt, out_dtype=torch.bfloat16)
        ref = Q.nvfp4_dequantize_bf16(np_(codes), np_(scales), g)
        assert np.array_equal(np_(d16.float()).view(np.uint32), ref.view(np.uint32))


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
