"""GPU parity: routed-expert MLP, stage by stage and end to end, NVFP4 and FP8."""

import numpy as np
import pytest
import torch

import block_scaled_fp4_sigmoid_amd as bsm_mod
import workloads as W
from oracle import moe as OM
from oracle import quant as Q
from oracle import route as OR
from tests.helpers import host_masters, np_, oracle_experts, rel_l2, to_dev_bf16, to_dev_f32, ws_view

pytestmark = pytest.mark.gpu

# Stage tolerances (relative L2).  Both formats decode their operands exactly
# to FP16 (NVFP4 q * s_b: <= 6 significant bits; E4M3: 4) and accumulate in
# FP32 on the FP16 MFMA.  A K-term FP32 sum of products with random signs
# carries a relative error of order sqrt(K) * 2^-24 (about 4e-6 at K = 5120)
# per element, so the relative L2 over a stage sits near 1e-7..1e-6; h and y
# are gated at 1e-5 in both formats (layer outputs: 1e-3).
STAGE_TOL = 1e-5


def _weights_match(gpu_w, experts, fmt, ids):
    for e in ids:
        ex = experts[e]
        if fmt == "nvfp4":
            c13, s13, g13 = np_(gpu_w.w13_codes[e]), np_(gpu_w.w13_scales[e]), np_(gpu_w.w13_gs[e])
            I = c13.shape[0] // 2
            assert np.array_equal(c13[:I], ex.gate[0]) and np.array_equal(c13[I:], ex.up[0])
            assert np.array_equal(s13[:I], ex.gate[1]) and np.array_equal(s13[I:], ex.up[1])
            assert g13[0] == ex.gate[2] and g13[1] == ex.up[2]
            assert np.array_equal(np_(gpu_w.w2_codes[e]), ex.down[0])
            assert np.array_equal(np_(gpu_w.w2_scales[e]), ex.down[1]) and np_(gpu_w.w2_gs[e]) == ex.down[2]
        else:
            c13, s13 = np_(gpu_w.w13_codes[e]), np_(gpu_w.w13_scales[e])
            I = c13.shape[0] // 2
            assert np.array_equal(c13[:I], ex.gate[0]) and np.array_equal(c13[I:], ex.up[0])
            assert np.array_equal(s13[:I], ex.gate[1]) and np.array_equal(s13[I:], ex.up[1])
            assert np.array_equal(np_(gpu_w.w2_codes[e]), ex.down[0])
            assert np.array_equal(np_(gpu_w.w2_scales[e]), ex.down[1])


def _stages(gpu_lib, fmt, cfg, T, ws, P):
    lay = gpu_lib.moe_workspace_layout(fmt, cfg.E, cfg.H, cfg.I, T, cfg.topk)
    I, H = cfg.I, cfg.H
    st = {
        "counts": np_(ws_view(ws, lay, "counts", torch.int32, (cfg.E,))),
        "offsets": np_(ws_view(ws, lay, "offsets", torch.int32, (cfg.E + 1,))),
        "row_pair": np_(ws_view(ws, lay, "row_pair", torch.int32, (P,))),
        "pair_row": np_(ws_view(ws, lay, "pair_row", torch.int32, (P,))),
        "h": np_(ws_view(ws, lay, "h_f32", torch.float32, (P, I))),
        "y": np_(ws_view(ws, lay, "y_f32", torch.float32, (P, H))),
    }
    if fmt == "nvfp4":
        st["hc"] = np_(ws_view(ws, lay, "h_codes", torch.uint8, (P, I // 2)))
        st["hs"] = np_(ws_view(ws, lay, "h_scales", torch.uint8, (P, I // 16)))
        st["hg"] = np_(ws_view(ws, lay, "h_gs", torch.float32, (1,)))[0]
    else:
        st["hc"] = np_(ws_view(ws, lay, "h_codes", torch.uint8, (P, I)))
        st["hs"] = np_(ws_view(ws, lay, "h_scales", torch.float32, (P,)))
    return st


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_moe_tiny_layer_stagewise(gpu_lib, fmt):
    cfg = W.TINY
    x, wr = W.activations(cfg), W.router_weights(cfg)
    masters, w13, w2 = host_masters(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, fmt)
    experts = oracle_experts(masters, fmt)
    _weights_match(gw, experts, fmt, range(cfg.E))  # offline quantization (RTN) is bit-exact

    xt = to_dev_bf16(x)
    ids, wts = gpu_lib.route(xt, to_dev_f32(wr), cfg.n_group, cfg.topk_group, cfg.topk)
    xq = gpu_lib.quantize_activations(xt, fmt)
    out, ws = gpu_lib.moe_expert_mlp(gw, xq, ids, wts, cfg.combine_scale, return_workspace=True)
    torch.cuda.synchronize()

    ref = OM.moe_layer(x, wr, experts, fmt, cfg.n_group, cfg.topk_group, cfg.topk, cfg.combine_scale)
    assert np.array_equal(np_(ids), ref["ids"])
    assert np.array_equal(np_(wts).view(np.uint32), ref["w"].view(np.uint32))
    for a, b in zip(xq, ref["xq"]):
        assert np.array_equal(np_(a).reshape(np.shape(b)), b)

    P = cfg.T * cfg.topk
    st = _stages(gpu_lib, fmt, cfg, cfg.T, ws, P)
    counts, offsets, row_of_pair, pair_of_row = OM.permute(ref["ids"], cfg.E)
    assert np.array_equal(st["counts"], counts) and np.array_equal(st["offsets"], offsets)
    assert np.array_equal(st["row_pair"], pair_of_row) and np.array_equal(st["pair_row"], row_of_pair)

    # stage 1: h (GPU rows are in sorted order) against the oracle's h in pair order
    h_gpu = st["h"][row_of_pair]
    assert rel_l2(h_gpu, ref["h"]) <= STAGE_TOL
    # stage 2: the oracle's quantizer applied to the GPU's h reproduces the GPU's codes
    if fmt == "nvfp4":
        oc, os_, og = Q.nvfp4_quantize(st["h"])
        assert st["hg"] == og
    else:
        oc, os_ = Q.fp8_quantize(st["h"])
    assert np.array_equal(st["hc"], oc) and np.array_equal(st["hs"], os_)
    # stage 3: down projection from identical h codes
    if fmt == "nvfp4":
        hh = Q.nvfp4_dequantize_exact(oc, os_, og)
    else:
        hh = Q.fp8_dequantize_exact(oc, os_)
    y_ref = np.zeros_like(st["y"])
    for e in np.unique(ref["ids"]):
        rows = np.arange(offsets[e], offsets[e + 1])
        y_ref[rows] = OM.gemm_f32(hh[rows], experts[int(e)].decoded()[2])
    assert rel_l2(st["y"], y_ref) <= STAGE_TOL
    # stage 4: combine of the GPU's y
    comb = OM.combine_f32(st["y"][row_of_pair].reshape(cfg.T, cfg.topk, -1), np_(wts), cfg.combine_scale)
    assert rel_l2(np_(out), comb) <= 1e-6
    # end to end
    e2e = rel_l2(np_(out), ref["out"])
    print(f"tiny {fmt}: end-to-end rel L2 {e2e:.3e}")
    assert e2e <= 1e-3


def test_moe_static_h_scale_and_determinism(gpu_lib):
    cfg = W.TINY
    x, wr = W.activations(cfg), W.router_weights(cfg)
    masters, w13, w2 = host_masters(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, "nvfp4")
    xt = to_dev_bf16(x)
    ids, wts = gpu_lib.route(xt, to_dev_f32(wr), 4, 2, 2)
    xq = gpu_lib.quantize_activations(xt, "nvfp4")
    o1 = gpu_lib.moe_expert_mlp(gw, xq, ids, wts)
    o2 = gpu_lib.moe_expert_mlp(gw, xq, ids, wts)
    assert torch.equal(o1, o2)
    hs = torch.tensor([0.01], dtype=torch.float32, device="cuda")
    o3, ws = gpu_lib.moe_expert_mlp(gw, xq, ids, wts, h_global_scale=hs, return_workspace=True)
    torch.cuda.synchronize()
    st = _stages(gpu_lib, "nvfp4", cfg, cfg.T, ws, cfg.T * cfg.topk)
    oc, os_, _ = Q.nvfp4_quantize(st["h"], global_scale=np.float32(0.01))
    assert np.array_equal(st["hc"], oc) and np.array_equal(st["hs"], os_)


def test_moe_empty_experts_and_single_token(gpu_lib):
    """T = 1 (most experts empty) and a ragged T = 37 against the oracle."""
    cfg = W.TINY
    masters, w13, w2 = host_masters(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, "nvfp4")
    experts = oracle_experts(masters, "nvfp4")
    wr = W.router_weights(cfg)
    for T in (1, 37):
        x = W.activations(cfg, T=T)
        xt = to_dev_bf16(x)
        out, ids, wts = gpu_lib.moe_layer(xt, to_dev_f32(wr), gw, 4, 2, 2)
        ref = OM.moe_layer(x, wr, experts, "nvfp4", 4, 2, 2)
        assert np.array_equal(np_(ids), ref["ids"])
        assert rel_l2(np_(out), ref["out"]) <= 1e-3


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_moe_decode_full_size_sampled(gpu_lib, fmt):
    """Beam decode shape (64 tokens, 256 experts): full GPU layer, oracle on sampled pairs."""
    cfg = W.DECODE
    x, wr = W.activations(cfg), W.router_weights(cfg)
    w13, w2 = W.expert_weights_device(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, fmt)
    xt = to_dev_bf16(x)
    ids, wts = gpu_lib.route(xt, to_dev_bf16(wr), 8, 4, 8)
    xq = gpu_lib.quantize_activations(xt, fmt)
    out, ws = gpu_lib.moe_expert_mlp(gw, xq, ids, wts, 2.5, return_workspace=True)
    torch.cuda.synchronize()
    oi, ow, _, _ = OR.route(x, wr, 8, 4, 8)
    assert np.array_equal(np_(ids), oi) and np.array_equal(np_(wts), ow)
    P = cfg.T * cfg.topk
    st = _stages(gpu_lib, fmt, cfg, cfg.T, ws, P)
    counts, offsets, row_of_pair, pair_of_row = OM.permute(oi, cfg.E)
    assert np.array_equal(st["row_pair"], pair_of_row)
    # h quantization of all rows, bit-exact from the GPU's h
    if fmt == "nvfp4":
        oc, os_, og = Q.nvfp4_quantize(st["h"])
        assert st["hg"] == og
    else:
        oc, os_ = Q.fp8_quantize(st["h"])
        og = None
    assert np.array_equal(st["hc"], oc) and np.array_equal(st["hs"], os_)
    # sampled token: its 8 experts quantized by the oracle from the same bf16 masters
    t = 17
    es = [int(e) for e in oi[t]]
    cls = OM.NVFP4Expert if fmt == "nvfp4" else OM.FP8Expert
    experts = {}
    for e in es:
        g = w13[e, :cfg.I].float().cpu().numpy()
        u = w13[e, cfg.I:].float().cpu().numpy()
        d = w2[e].float().cpu().numpy()
        experts[e] = cls(g, u, d)
    _weights_match(gw, experts, fmt, es)
    xq_o, xh = OM.quantize_activations(x, fmt)
    for a, b in zip(xq, xq_o):
        assert np.array_equal(np_(a).reshape(np.shape(b)), b)
    rows = [int(row_of_pair[t * 8 + j]) for j in range(8)]
    y_gpu = st["y"][rows]
    hh = (Q.nvfp4_dequantize_exact(oc[rows], os_[rows], og) if fmt == "nvfp4"
          else Q.fp8_dequantize_exact(oc[rows], os_[rows]))
    acc_e2e = []
    for j, e in enumerate(es):
        wg, wu, wd = experts[e].decoded()
        g = OM.gemm_f32(xh[t:t + 1], wg)
        u = OM.gemm_f32(xh[t:t + 1], wu)
        h = OM.swiglu_f32(g, u)
        assert rel_l2(st["h"][rows[j]], h[0]) <= STAGE_TOL
        assert rel_l2(y_gpu[j], OM.gemm_f32(hh[j:j + 1], wd)[0]) <= STAGE_TOL
        # end to end for this pair: oracle's own h, quantized with the call's h scale
        if fmt == "nvfp4":
            hq = Q.nvfp4_quantize(h, global_scale=og)
            hq_hat = Q.nvfp4_dequantize_exact(*hq)
        else:
            hq_hat = Q.fp8_dequantize_exact(*Q.fp8_quantize(h))
        acc_e2e.append(OM.gemm_f32(hq_hat, wd)[0])
    ref_out = OM.combine_f32(np.stack(acc_e2e)[None], ow[t:t + 1], 2.5)[0]
    comb = OM.combine_f32(y_gpu[None], np_(wts)[t:t + 1], 2.5)[0]
    assert rel_l2(np_(out)[t], comb) <= 1e-6
    e2e = rel_l2(np_(out)[t], ref_out)
    print(f"decode {fmt} token {t}: end-to-end rel L2 {e2e:.3e}")
    assert e2e <= 1e-3


# hidden 1024, intermediate 512, 8 experts: two column tiles of the many-row kernels in both GEMMs
MID = W.LayerConfig("mid", 7, T=700, H=1024, I=512, E=8, n_group=2, topk_group=1, topk=2, router_fp32=True)


@pytest.mark.parametrize("fmt,T", [("nvfp4", 300), ("nvfp4", 1000), ("fp8", 300), ("fp8", 1000)])
def test_moe_tiny_shapes_many_tokens(gpu_lib, fmt, T):
    """Tiny layer with many tokens: experts with 33-64 rows (up to four 16-row tiles, T = 300) and above 64 rows
    (LDS-tiled kernel, T = 1000) next to small ones, ragged tiles."""
    _many_tokens(gpu_lib, W.TINY, fmt, T)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_moe_mid_shapes_many_rows(gpu_lib, fmt):
    """Every expert above 64 rows in ragged 128-row tiles, several column tiles per GEMM; every row checked."""
    _many_tokens(gpu_lib, MID, fmt, MID.T)


# Every expert has 35-61 rows here, so the few-row kernel gets full 16-row tiles; with K = 2048 (gate/up)
# and 1024 (down) their staged activation rows come in several chunks of K (NVFP4: 2 super-steps of 512
# per chunk at 16 rows, FP8: 3 of 256).
SKC = W.LayerConfig("skinny-chunks", 8, T=200, H=2048, I=1024, E=8, n_group=2, topk_group=1, topk=2,
                    router_fp32=True)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_moe_skinny_tiles_in_chunks(gpu_lib, fmt):
    """Few-row experts with full 16-row tiles whose activation rows are staged in several chunks of K."""
    _many_tokens(gpu_lib, SKC, fmt, SKC.T)


def _many_tokens(gpu_lib, cfg, fmt, T):
    x, wr = W.activations(cfg, T=T), W.router_weights(cfg)
    masters, w13, w2 = host_masters(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, fmt)
    experts = oracle_experts(masters, fmt)
    xt = to_dev_bf16(x)
    ids, wts = gpu_lib.route(xt, to_dev_f32(wr), cfg.n_group, cfg.topk_group, cfg.topk)
    xq = gpu_lib.quantize_activations(xt, fmt)
    out, ws = gpu_lib.moe_expert_mlp(gw, xq, ids, wts, cfg.combine_scale, return_workspace=True)
    torch.cuda.synchronize()
    ref = OM.moe_layer(x, wr, experts, fmt, cfg.n_group, cfg.topk_group, cfg.topk, cfg.combine_scale)
    assert np.array_equal(np_(ids), ref["ids"])
    counts = np.bincount(ref["ids"].ravel(), minlength=cfg.E)
    assert counts.max() > (64 if T >= 700 else 32)
    P = T * cfg.topk
    st = _stages(gpu_lib, fmt, cfg, T, ws, P)
    _, offsets, row_of_pair, _ = OM.permute(ref["ids"], cfg.E)
    h_err = rel_l2(st["h"][row_of_pair], ref["h"])
    print(f"{cfg.name} {fmt} T={T}: h rel L2 {h_err:.3e}")
    assert h_err <= STAGE_TOL
    if fmt == "nvfp4":
        oc, os_, og = Q.nvfp4_quantize(st["h"])
        hh = Q.nvfp4_dequantize_exact(oc, os_, og)
    else:
        oc, os_ = Q.fp8_quantize(st["h"])
        hh = Q.fp8_dequantize_exact(oc, os_)
    assert np.array_equal(st["hc"], oc) and np.array_equal(st["hs"], os_)
    y_ref = np.zeros_like(st["y"])
    for e in np.unique(ref["ids"]):
        rows = np.arange(offsets[e], offsets[e + 1])
        y_ref[rows] = OM.gemm_f32(hh[rows], experts[int(e)].decoded()[2])
    y_err = rel_l2(st["y"], y_ref)
    print(f"{cfg.name} {fmt} T={T}: y rel L2 {y_err:.3e}")
    assert y_err <= STAGE_TOL
    e2e = rel_l2(np_(out), ref["out"])
    print(f"{cfg.name} {fmt} T={T}: max rows {counts.max()}, end-to-end rel L2 {e2e:.3e}")
    assert e2e <= 1e-3


def test_moe_prefill_full_size_sampled(gpu_lib):
    """Beam prefill shape (8192 tokens, Zipf-skewed router) in NVFP4: full GPU layer, oracle on sampled rows."""
    cfg = W.PREFILL
    x, wr = W.activations(cfg), W.router_weights(cfg)
    w13, w2 = W.expert_weights_device(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, "nvfp4")
    xt = to_dev_bf16(x)
    ids, wts = gpu_lib.route(xt, to_dev_bf16(wr), 8, 4, 8)
    xq = gpu_lib.quantize_activations(xt, "nvfp4")
    out, ws = gpu_lib.moe_expert_mlp(gw, xq, ids, wts, 2.5, return_workspace=True)
    torch.cuda.synchronize()
    oi, ow, _, _ = OR.route(x, wr, 8, 4, 8)
    assert np.array_equal(np_(ids), oi)
    P = cfg.T * cfg.topk
    st = _stages(gpu_lib, "nvfp4", cfg, cfg.T, ws, P)
    counts, offsets, row_of_pair, pair_of_row = OM.permute(oi, cfg.E)
    assert np.array_equal(st["row_pair"], pair_of_row) and np.array_equal(st["counts"], counts)
    assert counts.max() > 1000
    # global h scale from all rows; sampled rows' codes bit-exact
    og = np.float32(np.float32(np.abs(st["h"]).max()) / np.float32(2688))
    assert st["hg"] == og
    rng = np.random.default_rng(3)
    big = int(np.argmax(counts))
    tok = [int(np.nonzero((oi == big).any(1))[0][5]), int(rng.integers(cfg.T))]
    sx = Q.nvfp4_global_scale(x)
    assert np_(xq[2])[0] == sx
    xq_o, xh = OM.quantize_activations(x[tok], "nvfp4", global_scale=sx)
    assert np.array_equal(np_(xq[0])[tok], xq_o[0]) and np.array_equal(np_(xq[1])[tok], xq_o[1])
    for t_i, t in enumerate(tok):
        es = [int(e) for e in oi[t]]
        rows = [int(row_of_pair[t * 8 + j]) for j in range(8)]
        oc, os_, _ = Q.nvfp4_quantize(st["h"][rows], global_scale=og)
        assert np.array_equal(st["hc"][rows], oc) and np.array_equal(st["hs"][rows], os_)
        hh = Q.nvfp4_dequantize_exact(oc, os_, og)
        ys = []
        for j, e in enumerate(es[:4]):  # 4 of the token's experts (oracle weight quantization is slow)
            ex = OM.NVFP4Expert(w13[e, :cfg.I].float().cpu().numpy(), w13[e, cfg.I:].float().cpu().numpy(),
                                w2[e].float().cpu().numpy())
            wg, wu, wd = ex.decoded()
            h = OM.swiglu_f32(OM.gemm_f32(xh[t_i:t_i + 1], wg), OM.gemm_f32(xh[t_i:t_i + 1], wu))
            assert rel_l2(st["h"][rows[j]], h[0]) <= 1e-5
            assert rel_l2(st["y"][rows[j]], OM.gemm_f32(hh[j:j + 1], wd)[0]) <= 1e-5
        comb = OM.combine_f32(st["y"][rows][None], np_(wts)[t:t + 1], 2.5)[0]
        assert rel_l2(np_(out)[t], comb) <= 1e-6
