"""GPU: routing and NVFP4 quantization of the same activations in one call (bsm_route_nvfp4_quantize).

The call must give, bit for bit, what bsm_route and bsm_nvfp4_quantize give separately; both of those are
checked against the oracle elsewhere (test_gpu_route, test_gpu_quant), and the decode shape is also checked
against the oracle directly here.  Cases cover the path where the router's pass over x supplies max|x|
(bf16 x and router weights, 256 experts, small batches: decode, a few tokens, a row of zeros, one large value,
all zeros) and the paths where the quantization takes its own pass (FP32 x, a batch past the small-batch
router, 64 experts).
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import quant as Q
from oracle import route as R
from tests.helpers import np_, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


def _bits(a):
    a = np_(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _both(gpu_lib, xt, wt, G, kg, k):
    ids, wts, (codes, scales, gs), scores = gpu_lib.route_nvfp4_quantize(xt, wt, G, kg, k, return_scores=True)
    ids2, wts2, scores2 = gpu_lib.route(xt, wt, G, kg, k, return_scores=True)
    c2, s2, g2 = gpu_lib.nvfp4_quantize(xt)
    torch.cuda.synchronize()
    fused = [ids, wts, scores, codes, scales, gs]
    sep = [ids2, wts2, scores2, c2, s2, g2]
    for name, a, b in zip(["ids", "weights", "scores", "codes", "scales", "global scale"], fused, sep):
        assert np.array_equal(_bits(a), _bits(b)), name
    return [np_(t) for t in fused]


def _x(T, H, seed, scale=1.0):
    """Seeded normal values rounded to bf16 (exact in both input dtypes)."""
    x = (np.random.default_rng(seed).standard_normal((T, H)) * scale).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


def test_route_quant_decode_shape_vs_oracle(gpu_lib):
    cfg = W.DECODE
    x, wr = W.activations(cfg), W.router_weights(cfg)
    ids, wts, scores, codes, scales, gs = _both(gpu_lib, to_dev_bf16(x), to_dev_bf16(wr), 8, 4, 8)
    oi, ow, os_, _ = R.route(x, wr, 8, 4, 8)
    assert np.array_equal(ids, oi) and np.array_equal(wts.view(np.uint32), ow.view(np.uint32))
    oc, osc, og = Q.nvfp4_quantize(x)
    assert np.array_equal(codes, oc) and np.array_equal(scales, osc)
    assert np.array_equal(gs.view(np.uint32), np.asarray(og, np.float32).reshape(1).view(np.uint32))


@pytest.mark.parametrize("T", [1, 5, 64, 300])
def test_route_quant_small_batches(gpu_lib, T):
    wr = W.router_weights(W.DECODE)
    x = _x(T, 5120, 100 + T, scale=3.0)
    _both(gpu_lib, to_dev_bf16(x), to_dev_bf16(wr), 8, 4, 8)


def test_route_quant_special_rows(gpu_lib):
    """A row of zeros adds nothing to max|x|, and one large value in another row sets it.  (Inputs stay
    finite: the router's contract leaves non-finite values unspecified.)"""
    wr = W.router_weights(W.DECODE)
    x = _x(16, 5120, 7)
    x[3] = 0.0
    x[5, 18] = -2.0**20
    xt = to_dev_bf16(x)
    _, _, _, codes, scales, gs = _both(gpu_lib, xt, to_dev_bf16(wr), 8, 4, 8)
    amax = np.abs(np_(xt.float())).max()  # 2^20
    assert gs[0] == np.float32(amax) / np.float32(2688.0)


def test_route_quant_wide_range(gpu_lib):
    """Blocks spread over 2^-12 .. 2^8 of each other: E4M3 block scales down to the subnormal codes and zero
    scales, where the division by s_b S_g and the quantizer's threshold table must agree bit for bit."""
    wr = W.router_weights(W.DECODE)
    x = _x(64, 5120, 21)
    t, j = np.meshgrid(np.arange(64), np.arange(5120 // 16), indexing="ij")
    x *= np.repeat(np.exp2(((t * 7 + j * 3) % 21) - 12.0), 16, axis=1).astype(np.float32)
    _, _, _, codes, scales, gs = _both(gpu_lib, to_dev_bf16(x), to_dev_bf16(wr), 8, 4, 8)
    assert (scales < 8).any() and (scales == 0).any()  # subnormal and zero block scales occur
    oc, osc, og = Q.nvfp4_quantize(x)
    assert np.array_equal(codes, oc) and np.array_equal(scales, osc)


def test_route_quant_all_zero(gpu_lib):
    wr = W.router_weights(W.DECODE)
    x = np.zeros((8, 5120), np.float32)
    _, _, _, codes, scales, gs = _both(gpu_lib, to_dev_bf16(x), to_dev_bf16(wr), 8, 4, 8)
    assert gs[0] == 0.0 and not scales.any()


@pytest.mark.parametrize("case", ["f32_x", "large_batch", "experts64"])
def test_route_quant_unfused_paths(gpu_lib, case):
    if case == "f32_x":
        wr = W.router_weights(W.DECODE)
        _both(gpu_lib, to_dev_f32(_x(40, 5120, 3)), to_dev_bf16(wr), 8, 4, 8)
    elif case == "large_batch":
        wr = W.router_weights(W.DECODE)
        _both(gpu_lib, to_dev_bf16(_x(2048, 5120, 4)), to_dev_bf16(wr), 8, 4, 8)
    else:
        wr = _x(64, 1024, 5, scale=0.02)
        _both(gpu_lib, to_dev_bf16(_x(33, 1024, 6)), to_dev_bf16(wr), 8, 2, 4)


def test_route_quant_workspace_reuse(gpu_lib):
    """A second call on the same workspace starts from a zeroed max|x| (a smaller x after a larger one)."""
    wr = to_dev_bf16(W.router_weights(W.DECODE))
    big, small = to_dev_bf16(_x(64, 5120, 8, scale=50.0)), to_dev_bf16(_x(32, 5120, 9))
    ws = torch.empty(gpu_lib.load().bsm_route_nvfp4_quantize_workspace_size(64, 5120, 256), dtype=torch.uint8,
                     device="cuda")
    gpu_lib.route_nvfp4_quantize(big, wr, 8, 4, 8, ws=ws)
    _, _, (c, s, g) = gpu_lib.route_nvfp4_quantize(small, wr, 8, 4, 8, ws=ws)
    c2, s2, g2 = gpu_lib.nvfp4_quantize(small)
    torch.cuda.synchronize()
    assert np.array_equal(np_(c), np_(c2)) and np.array_equal(np_(s), np_(s2))
    assert np_(g).view(np.uint32)[0] == np_(g2).view(np.uint32)[0]
