"""GPU: the allocation-free expert MLP (bsm_moe_expert_mlp_noalloc) against bsm_moe_expert_mlp.

Both run the same kernels, so the outputs must be bit-identical: two calls in a
row on the static scratch, the second with fewer tokens (the scratch keeps the
first call's contents), in both formats at the tiny and the Beam decode shape.
A call that needs more scratch than the static array holds is refused with a
clear error and writes nothing.
"""

import numpy as np
import pytest
import torch

import workloads as W
from tests.helpers import host_masters, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


def _pair(gpu_lib, cfg, gw, fmt, x, wr, router_bf16):
    xt = to_dev_bf16(x)
    ids, wts = gpu_lib.route(xt, to_dev_bf16(wr) if router_bf16 else to_dev_f32(wr), cfg.n_group, cfg.topk_group,
                             cfg.topk)
    xq = gpu_lib.quantize_activations(xt, fmt)
    ref = gpu_lib.moe_expert_mlp(gw, xq, ids, wts, cfg.combine_scale)
    out = torch.full_like(ref, float("nan"))
    gpu_lib.moe_expert_mlp_noalloc(gw, xq, ids, wts, out, cfg.combine_scale)
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_noalloc_tiny_two_calls(gpu_lib, fmt):
    cfg = W.TINY
    _, w13, w2 = host_masters(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, fmt)
    wr = W.router_weights(cfg)
    for T in (64, 5):
        ref, out = _pair(gpu_lib, cfg, gw, fmt, W.activations(cfg, T=T), wr, False)
        assert torch.equal(out, ref), f"tiny {fmt} T={T}"


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_noalloc_decode_two_calls(gpu_lib, fmt):
    cfg = W.DECODE
    w13, w2 = W.expert_weights_device(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, fmt)
    del w13, w2
    wr = W.router_weights(cfg)
    x = W.activations(cfg)
    for T in (64, 17):
        ref, out = _pair(gpu_lib, cfg, gw, fmt, x[:T], wr, True)
        assert torch.equal(out, ref), f"decode {fmt} T={T}"
        assert np.isfinite(out.cpu().numpy()).all()
    del gw
    torch.cuda.empty_cache()


def test_noalloc_refuses_oversize(gpu_lib):
    cfg = W.TINY
    _, w13, w2 = host_masters(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, "nvfp4")
    T = 40000  # about 110 MiB of scratch at this shape
    xq = gpu_lib.quantize_activations(torch.zeros((T, cfg.H), dtype=torch.bfloat16, device="cuda"), "nvfp4")
    ids = torch.zeros((T, cfg.topk), dtype=torch.int32, device="cuda")
    ids[:, 1] = 1
    wts = torch.full((T, cfg.topk), 0.5, dtype=torch.float32, device="cuda")
    out = torch.full((T, cfg.H), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(gpu_lib.BsmError, match="static scratch"):
        gpu_lib.moe_expert_mlp_noalloc(gw, xq, ids, wts, out)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
