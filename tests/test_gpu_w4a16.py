"""GPU parity: weight-only W4A16 routed-expert MLP (NVFP4 weights, BF16 activations), stage by stage."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import moe as OM
from oracle import route as OR
from tests.helpers import host_masters, np_, oracle_experts, rel_l2, to_dev_bf16, to_dev_f32, ws_view

pytestmark = pytest.mark.gpu

# g, u and y accumulate in FP32 over K <= 5120 exactly decoded BF16 products:
# about sqrt(K) * 2^-24 relative per element, so 1e-5 per stage (as for W4A4).
H_TOL = 1e-5


def _stages(gpu_lib, cfg, T, ws):
    lay = gpu_lib.moe_workspace_layout("w4a16", cfg.E, cfg.H, cfg.I, T, cfg.topk)
    P = T * cfg.topk
    return {
        "row_pair": np_(ws_view(ws, lay, "row_pair", torch.int32, (P,))),
        "h": np_(ws_view(ws, lay, "h_f32", torch.float32, (P, cfg.I))),
        "y": np_(ws_view(ws, lay, "y_f32", torch.float32, (P, cfg.H))),
    }


def _check_layer(gpu_lib, cfg, T, x, wr, wr_dev, experts, gw):
    xt = to_dev_bf16(x)
    ids, wts = gpu_lib.route(xt, wr_dev, cfg.n_group, cfg.topk_group, cfg.topk)
    out, ws = gpu_lib.moe_expert_mlp_w4a16(gw, xt, ids, wts, cfg.combine_scale, return_workspace=True)
    torch.cuda.synchronize()
    oi, ow, _, _ = OR.route(x, wr, cfg.n_group, cfg.topk_group, cfg.topk)
    assert np.array_equal(np_(ids), oi)
    ref = OM.moe_expert_mlp(x.astype(np.float64), oi, ow, experts, "w4a16", cfg.combine_scale)
    st = _stages(gpu_lib, cfg, T, ws)
    counts, offsets, row_of_pair, pair_of_row = OM.permute(oi, cfg.E)
    assert np.array_equal(st["row_pair"], pair_of_row)
    # stage 1: h against the oracle's h (pair order)
    assert rel_l2(st["h"][row_of_pair], ref["h"]) <= H_TOL
    # stage 2: down projection from the GPU's h rounded to BF16 (teacher-forced)
    hb = F.bf16_round(st["h"]).astype(np.float64)
    y_ref = np.zeros_like(st["y"])
    for e in np.unique(oi):
        rows = np.arange(offsets[e], offsets[e + 1])
        y_ref[rows] = OM.gemm_f32(hb[rows], experts[int(e)].decoded()[2])
    assert rel_l2(st["y"], y_ref) <= H_TOL
    # stage 3: combine of the GPU's y
    comb = OM.combine_f32(st["y"][row_of_pair].reshape(T, cfg.topk, -1), np_(wts), cfg.combine_scale)
    assert rel_l2(np_(out), comb) <= 1e-6
    e2e = rel_l2(np_(out), ref["out"])
    print(f"w4a16 T={T}: max rows {counts.max()}, end-to-end rel L2 {e2e:.3e}")
    assert e2e <= 1e-3
    return counts


@pytest.mark.parametrize("T", [64, 37, 1000])
def test_w4a16_tiny_layer(gpu_lib, T):
    """Tiny layer: T = 64, a ragged T = 37, and T = 1000 (experts above 32 rows take the LDS-tiled kernel)."""
    cfg = W.TINY
    x, wr = W.activations(cfg, T=T), W.router_weights(cfg)
    masters, w13, w2 = host_masters(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, "nvfp4")
    experts = oracle_experts(masters, "w4a16")
    counts = _check_layer(gpu_lib, cfg, T, x, wr, to_dev_f32(wr), experts, gw)
    if T == 1000:
        assert counts.max() > 64


def test_w4a16_mid_shapes_many_rows(gpu_lib):
    """Hidden 1024, intermediate 512, 8 experts, 700 tokens: every expert in ragged 128-row tiles."""
    cfg = W.LayerConfig("mid", 7, T=700, H=1024, I=512, E=8, n_group=2, topk_group=1, topk=2, router_fp32=True)
    x, wr = W.activations(cfg), W.router_weights(cfg)
    masters, w13, w2 = host_masters(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, "nvfp4")
    counts = _check_layer(gpu_lib, cfg, cfg.T, x, wr, to_dev_f32(wr), oracle_experts(masters, "w4a16"), gw)
    assert counts.min() > 64


@pytest.mark.parametrize("T,topk,topk_group", [(64, 6, 2), (100, 2, 1)], ids=["one-chunk", "two-chunks"])
def test_w4a16_skinny_tiles_in_chunks(gpu_lib, T, topk, topk_group):
    """Hidden 2048, intermediate 1024, 8 experts: few-row experts with full 16-row tiles whose BF16 activation
    rows are staged in several chunks of K (one chunk of 64 tokens: 42-52 rows per expert; two chunks of 100
    tokens: 16-35 rows, the few-row kernel taking experts of at most 32)."""
    cfg = W.LayerConfig("skinny-chunks", 8, T=T, H=2048, I=1024, E=8, n_group=2, topk_group=topk_group,
                        topk=topk, router_fp32=True)
    x, wr = W.activations(cfg), W.router_weights(cfg)
    masters, w13, w2 = host_masters(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, "nvfp4")
    counts = _check_layer(gpu_lib, cfg, cfg.T, x, wr, to_dev_f32(wr), oracle_experts(masters, "w4a16"), gw)
    few = counts[counts <= (64 if T <= 64 else 32)]
    assert few.size > 0 and few.max() > 16


def test_w4a16_deterministic_and_matches_w4a4_weights(gpu_lib):
    cfg = W.TINY
    x, wr = W.activations(cfg), W.router_weights(cfg)
    _, w13, w2 = host_masters(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, "nvfp4")
    xt = to_dev_bf16(x)
    ids, wts = gpu_lib.route(xt, to_dev_f32(wr), cfg.n_group, cfg.topk_group, cfg.topk)
    o1 = gpu_lib.moe_expert_mlp_w4a16(gw, xt, ids, wts)
    o2 = gpu_lib.moe_expert_mlp_w4a16(gw, xt, ids, wts)
    assert torch.equal(o1, o2)
    with pytest.raises(gpu_lib.BsmError):
        gpu_lib.moe_expert_mlp_w4a16(gw, xt.float(), ids, wts)


def test_w4a16_decode_full_size_sampled(gpu_lib):
    """Beam decode shape: full GPU layer, oracle on one token's 8 pairs."""
    cfg = W.DECODE
    x, wr = W.activations(cfg), W.router_weights(cfg)
    w13, w2 = W.expert_weights_device(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, "nvfp4")
    xt = to_dev_bf16(x)
    ids, wts = gpu_lib.route(xt, to_dev_bf16(wr), 8, 4, 8)
    out, ws = gpu_lib.moe_expert_mlp_w4a16(gw, xt, ids, wts, 2.5, return_workspace=True)
    torch.cuda.synchronize()
    oi, ow, _, _ = OR.route(x, wr, 8, 4, 8)
    assert np.array_equal(np_(ids), oi)
    st = _stages(gpu_lib, cfg, cfg.T, ws)
    _, _, row_of_pair, _ = OM.permute(oi, cfg.E)
    t = 29
    rows = [int(row_of_pair[t * 8 + j]) for j in range(8)]
    ys = []
    for j, e in enumerate(int(e) for e in oi[t]):
        ex = OM.NVFP4Expert(w13[e, :cfg.I].float().cpu().numpy(), w13[e, cfg.I:].float().cpu().numpy(),
                            w2[e].float().cpu().numpy())
        wg, wu, wd = ex.decoded()
        xr = x[t:t + 1].astype(np.float64)
        h = OM.swiglu_f32(OM.gemm_f32(xr, wg), OM.gemm_f32(xr, wu))
        assert rel_l2(st["h"][rows[j]], h[0]) <= H_TOL
        hb_gpu = F.bf16_round(st["h"][rows[j]][None]).astype(np.float64)
        assert rel_l2(st["y"][rows[j]], OM.gemm_f32(hb_gpu, wd)[0]) <= H_TOL
        ys.append(OM.gemm_f32(F.bf16_round(h).astype(np.float64), wd)[0])
    ref_out = OM.combine_f32(np.stack(ys)[None], ow[t:t + 1], 2.5)[0]
    comb = OM.combine_f32(st["y"][rows][None], np_(wts)[t:t + 1], 2.5)[0]
    assert rel_l2(np_(out)[t], comb) <= 1e-6
    e2e = rel_l2(np_(out)[t], ref_out)
    print(f"w4a16 decode token {t}: end-to-end rel L2 {e2e:.3e}")
    assert e2e <= 1e-3
