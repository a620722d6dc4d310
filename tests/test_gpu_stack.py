"""GPU parity: stacked MoE layers on an FP32 residual stream (RMSNorm -> MoE -> depth-scaled residual).

Per layer, teacher-forced: the oracle consumes the GPU's stream input of that
layer.  RMSNorm within 1 ulp, routing / quantization / residual bit-exact, MoE
output within 1e-3 relative L2.  End-to-end drift over the stack is reported.
"""

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe as OM
from oracle import quant_c as QC
from oracle import route as OR
from tests.fullsize import DeviceExperts
from tests.helpers import np_, oracle_experts, rel_l2, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


def _ulps(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def _tiny_layers(gpu_lib, fmt, n_layers, seed_base=10):
    cfg = W.TINY
    layers_gpu, layers_orc = [], []
    for li in range(n_layers):
        masters = [W.expert_weights_host(cfg, e, layer=seed_base + li) for e in range(cfg.E)]
        w13 = to_dev_bf16(np.stack([np.concatenate([g, u]) for g, u, _ in masters]))
        w2 = to_dev_bf16(np.stack([d for _, _, d in masters]))
        wr = W.to_bf16_f32(W.router_weights(cfg, layer=seed_base + li))
        layers_gpu.append((to_dev_bf16(wr), gpu_lib.quantize_expert_weights(w13, w2, fmt)))
        layers_orc.append((wr, oracle_experts(masters, fmt)))
    return layers_gpu, layers_orc


def test_rmsnorm_with_gain(gpu_lib):
    """RMSNorm with a gain vector: fl32(fl32(x * r) * gamma), within 1 ulp of the oracle (r exactly rounded
    on both sides; the gain product is one binary32 multiply)."""
    rng = np.random.default_rng(41)
    x = (rng.standard_normal((37, 5120)) * 3).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(5120)).astype(np.float32)
    y = np_(gpu_lib.rmsnorm(to_dev_f32(x), 1e-6, gamma=to_dev_f32(g)))
    assert _ulps(y, OM.rmsnorm_f32(x, 1e-6, gamma=g)).max() <= 1
    y1 = np_(gpu_lib.rmsnorm(to_dev_f32(x), 1e-6))
    assert _ulps(y1, OM.rmsnorm_f32(x, 1e-6)).max() <= 1


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_stack_tiny_teacher_forced(gpu_lib, fmt):
    cfg = W.TINY
    T = 256
    x1 = W.activations(cfg, T=T)
    lg, lo = _tiny_layers(gpu_lib, fmt, 4)
    xf, trace = gpu_lib.moe_stack(to_dev_f32(x1), lg, cfg.n_group, cfg.topk_group, cfg.topk, keep=True)
    torch.cuda.synchronize()
    for i, (xin, n, ids, wts, m) in enumerate(trace, start=1):
        xin, n, ids, wts, m = np_(xin), np_(n), np_(ids), np_(wts), np_(m)
        n_ref = OM.rmsnorm_f32(xin)
        assert _ulps(n, n_ref).max() <= 1
        wr, experts = lo[i - 1]
        ref = OM.moe_layer(n, wr, experts, fmt, cfg.n_group, cfg.topk_group, cfg.topk)
        assert np.array_equal(ids, ref["ids"]) and np.array_equal(wts.view(np.uint32), ref["w"].view(np.uint32))
        assert rel_l2(m, ref["out"]) <= 1e-3
        nxt = np_(trace[i][0]) if i < len(trace) else np_(xf)
        assert np.array_equal(nxt.view(np.uint32), OM.scaled_residual_f32(xin, m, i + 1).view(np.uint32))
    xs, _ = OM.moe_stack(x1, lo, fmt, cfg.n_group, cfg.topk_group, cfg.topk)
    drift = rel_l2(np_(xf), xs[-1])
    print(f"stack tiny {fmt}: end-to-end drift after 4 layers rel L2 {drift:.3e}")


def test_stack_formats_against_unquantized(gpu_lib):
    """FP8 should stay closer to the unquantized stack than NVFP4 (reported; FP8 page vs NVFP4 page)."""
    cfg = W.TINY
    T = 128
    x1 = W.activations(cfg, T=T)
    outs = {}
    for fmt in ("nvfp4", "fp8"):
        lg, _ = _tiny_layers(gpu_lib, fmt, 4)
        outs[fmt] = np_(gpu_lib.moe_stack(to_dev_f32(x1), lg, cfg.n_group, cfg.topk_group, cfg.topk))
    # unquantized float64 stack on the same bf16 masters
    x = x1.astype(np.float64)
    for li in range(4):
        masters = [W.expert_weights_host(cfg, e, layer=10 + li) for e in range(cfg.E)]
        wr = W.to_bf16_f32(W.router_weights(cfg, layer=10 + li))
        n = OM.rmsnorm_f32(x.astype(np.float32))
        ids, w, _, _ = OR.route(n, wr, cfg.n_group, cfg.topk_group, cfg.topk)
        y = np.zeros_like(x)
        for t in range(T):
            for j in range(cfg.topk):
                g, u, d = (a.astype(np.float64) for a in masters[ids[t, j]])
                gg = g @ n[t]
                h = gg / (1 + np.exp(-gg)) * (u @ n[t])
                y[t] += 2.5 * w[t, j] * (d @ h)
        k = li + 2
        x = math.sqrt((k - 1) / k) * x + y / math.sqrt(k)
    e4, e8 = rel_l2(outs["nvfp4"], x), rel_l2(outs["fp8"], x)
    print(f"stack vs unquantized: NVFP4 rel L2 {e4:.3e}, FP8 rel L2 {e8:.3e}")
    assert e8 < e4


@pytest.mark.slow
@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_stack_full_size_teacher_forced(gpu_lib, fmt):
    """Beam shapes, 4096 tokens, 4 layers: per layer, teacher-forced, RMSNorm within 1 ulp, routing, activation
    quantization and residual bit-exact, MoE output within 1e-3 of the oracle's layer on the GPU's normed input.

    The oracle quantizes each layer's 256 experts itself from the same bf16 masters (checked bit-exactly
    against the GPU's quantized weights before use)."""
    cfg = W.STACK
    x1 = W.activations(cfg)
    layers, wrs = [], []
    for li in range(cfg.layers):
        w13, w2 = W.expert_weights_device(cfg, layer=li)
        wrs.append(W.router_weights(cfg, layer=li))
        layers.append((to_dev_bf16(wrs[-1]), gpu_lib.quantize_expert_weights(w13, w2, fmt)))
        del w13, w2
        torch.cuda.empty_cache()
    xf, trace = gpu_lib.moe_stack(to_dev_f32(x1), layers, cfg.n_group, cfg.topk_group, cfg.topk, keep=True)
    torch.cuda.synchronize()
    for i, (xin, n, ids, wts, m) in enumerate(trace, start=1):
        xin, n, m = np_(xin), np_(n), np_(m)
        assert _ulps(n, OM.rmsnorm_f32(xin)).max() <= 1
        w13, w2 = W.expert_weights_device(cfg, layer=i - 1)
        experts = DeviceExperts(w13, w2, layers[i - 1][1], fmt)
        ref = OM.moe_layer(n, wrs[i - 1], experts, fmt, cfg.n_group, cfg.topk_group, cfg.topk, q=QC)
        assert np.array_equal(np_(ids), ref["ids"]) and np.array_equal(np_(wts).view(np.uint32), ref["w"].view(np.uint32))
        xq = gpu_lib.quantize_activations(to_dev_f32(n), fmt)
        for a, b in zip(xq, ref["xq"]):
            assert np.array_equal(np_(a).reshape(np.shape(b)), b)
        err = rel_l2(m, ref["out"])
        print(f"stack {fmt} layer {i}: {len(experts.cache)} experts, MoE output rel L2 {err:.3e}", flush=True)
        assert err <= 1e-3
        nxt = np_(trace[i][0]) if i < len(trace) else np_(xf)
        assert np.array_equal(nxt.view(np.uint32), OM.scaled_residual_f32(xin, m, i + 1).view(np.uint32))
        del experts, w13, w2, ref
        torch.cuda.empty_cache()
