"""GPU parity: routed-expert MLP, stage by stage and end to end, NVFP4 and FP8."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe as OM
from oracle import quant as Q
from tests.helpers import host_masters, moe_stages, np_, oracle_experts, rel_l2, to_dev_bf16, to_dev_f32, weights_match

pytestmark = pytest.mark.gpu

# Stage tolerances (relative L2).  Both formats decode their operands exactly
# to FP16 (NVFP4 q * s_b: <= 6 significant bits; E4M3: 4) and accumulate in
# FP32 on the FP16 MFMA.  A K-term FP32 sum of products with random signs
# carries a relative error of order sqrt(K) * 2^-24 (about 4e-6 at K = 5120)
# per element, so the relative L2 over a stage sits near 1e-7..1e-6; h and y
# are gated at 1e-5 in both formats (layer outputs: 1e-3).
STAGE_TOL = 1e-5


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_moe_tiny_layer_stagewise(gpu_lib, fmt):
    cfg = W.TINY
    x, wr = W.activations(cfg), W.router_weights(cfg)
    masters, w13, w2 = host_masters(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, fmt)
    experts = oracle_experts(masters, fmt)
    weights_match(gw, experts, fmt, range(cfg.E))  # offline quantization (RTN) is bit-exact

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
    st = moe_stages(gpu_lib, fmt, cfg, cfg.T, ws, P)
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
    st = moe_stages(gpu_lib, "nvfp4", cfg, cfg.T, ws, cfg.T * cfg.topk)
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


# hidden 1024, intermediate 512, 8 experts: two column tiles of the many-row kernels in both GEMMs
MID = W.LayerConfig("mid", 7, T=700, H=1024, I=512, E=8, n_group=2, topk_group=1, topk=2, router_fp32=True)


@pytest.mark.parametrize("fmt,T", [("nvfp4", 300), ("nvfp4", 1000), ("fp8", 300), ("fp8", 1000)])
def test_moe_tiny_shapes_many_tokens(gpu_lib, fmt, T):
    """Tiny layer with many tokens (several permutation chunks): experts of at most 32 rows in 16-row tiles of
    the few-row kernel, and above 32 rows in 128-row tiles of the many-row kernel (33-64 rows at T = 300:
    one or two live 32-row sub-tiles; more at T = 1000), ragged tiles."""
    _many_tokens(gpu_lib, W.TINY, fmt, T)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_moe_mid_shapes_many_rows(gpu_lib, fmt):
    """Every expert above 64 rows in ragged 128-row tiles, several column tiles per GEMM; every row checked."""
    _many_tokens(gpu_lib, MID, fmt, MID.T)


# Few-row experts with full 16-row tiles; with K = 2048 (gate/up) and 1024 (down) their staged activation
# rows come in several chunks of K (NVFP4: 2 super-steps of 512 per chunk at 16 rows, FP8: 3 of 256).
# SKC: one permutation chunk (64 tokens, top-6 of 8), every expert at 42-52 rows, so up to four 16-row tiles
# per expert.  SKM: two chunks (100 tokens, top-2), experts at 16-35 rows: up to 32 rows stay in the
# few-row kernel (one or two 16-row tiles), the one above in the many-row kernel.
SKC = W.LayerConfig("skinny-chunks", 8, T=64, H=2048, I=1024, E=8, n_group=2, topk_group=2, topk=6,
                    router_fp32=True)
SKM = W.LayerConfig("skinny-chunks", 8, T=100, H=2048, I=1024, E=8, n_group=2, topk_group=1, topk=2,
                    router_fp32=True)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("cfg", [SKC, SKM], ids=["one-chunk", "two-chunks"])
def test_moe_skinny_tiles_in_chunks(gpu_lib, fmt, cfg):
    """Few-row experts with full 16-row tiles whose activation rows are staged in several chunks of K."""
    counts = _many_tokens(gpu_lib, cfg, fmt, cfg.T)
    few = counts[counts <= (64 if cfg.T <= 64 else 32)]
    assert few.size > 0 and few.max() > 16


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
    _check_stages(gpu_lib, cfg, fmt, T, ref["ids"], experts, ref, out, ws)
    return counts


def _check_stages(gpu_lib, cfg, fmt, T, ids, experts, ref, out, ws):
    """h of every row at the stage gate, h codes and scales bit-exact from the GPU's own h, y of every row
    from those codes at the stage gate, and the layer output within 1e-3 of the oracle's."""
    P = T * cfg.topk
    st = moe_stages(gpu_lib, fmt, cfg, T, ws, P)
    _, offsets, row_of_pair, _ = OM.permute(ids, cfg.E)
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
    for e in np.unique(ids):
        rows = np.arange(offsets[e], offsets[e + 1])
        y_ref[rows] = OM.gemm_f32(hh[rows], experts[int(e)].decoded()[2])
    y_err = rel_l2(st["y"], y_ref)
    print(f"{cfg.name} {fmt} T={T}: y rel L2 {y_err:.3e}")
    assert y_err <= STAGE_TOL
    e2e = rel_l2(np_(out), ref["out"])
    counts = np.bincount(np.asarray(ids).ravel(), minlength=cfg.E)
    print(f"{cfg.name} {fmt} T={T}: max rows {counts.max()}, end-to-end rel L2 {e2e:.3e}")
    assert e2e <= 1e-3


# Experts whose row counts sit on each side of the kernel choices with several permutation chunks: 16 / 17
# (one or two few-row tiles), 32 / 33 (few-row kernel / many-row kernel), 64 / 65 and 128 + 1 (a full
# 128-row tile and a one-row ragged one); the last expert takes the remaining 44 rows.
SPLIT = W.LayerConfig("split", 9, T=200, H=1024, I=512, E=8, n_group=2, topk_group=2, topk=2, router_fp32=True)
SPLIT_ROWS = [16, 17, 32, 33, 64, 65, 129]


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_moe_expert_split_boundaries(gpu_lib, fmt):
    """Given ids (not routed) with the expert row counts above; every stage against the oracle's expert MLP."""
    cfg = SPLIT
    T, k, E = cfg.T, cfg.topk, cfg.E
    counts = SPLIT_ROWS + [T * k - sum(SPLIT_ROWS)]
    labels = np.repeat(np.arange(E), counts)  # sorted; slots t and t + T never share an expert (max 129 < T)
    ids_np = np.stack([labels[:T], labels[T:]], axis=1).astype(np.int32)
    rng = np.random.default_rng(11)
    ids_np = ids_np[rng.permutation(T)]  # spread every expert's rows over the permutation chunks
    w_np = rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    w_np = (w_np / w_np.sum(axis=1, keepdims=True)).astype(np.float32)
    x = W.activations(cfg, T=T)
    masters, w13, w2 = host_masters(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, fmt)
    experts = oracle_experts(masters, fmt)
    xt = to_dev_bf16(x)
    xq = gpu_lib.quantize_activations(xt, fmt)
    ids = torch.from_numpy(ids_np).cuda()
    out, ws = gpu_lib.moe_expert_mlp(gw, xq, ids, torch.from_numpy(w_np).cuda(), cfg.combine_scale,
                                     return_workspace=True)
    torch.cuda.synchronize()
    _, x_hat = OM.quantize_activations(x, fmt)
    ref = OM.moe_expert_mlp(x_hat, ids_np, w_np, experts, fmt, cfg.combine_scale)
    st = moe_stages(gpu_lib, fmt, cfg, T, ws, T * k)
    assert np.array_equal(st["counts"], np.asarray(counts))
    _check_stages(gpu_lib, cfg, fmt, T, ids_np, experts, ref, out, ws)


@pytest.mark.parametrize("T", [64, 300])
def test_moe_out_of_range_ids_are_dropped(gpu_lib, T):
    """Expert ids outside [0, E) are dropped, through the one-chunk (T = 64) and the chunked (T = 300)
    permutation: no row, pair_row -1, nothing combined.  With a static h global scale the other rows do not
    depend on which pairs exist, so the output equals the run where those pairs go to a valid expert with
    weight 0, bit for bit."""
    cfg = W.TINY
    _, w13, w2 = host_masters(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, "nvfp4")
    xt = to_dev_bf16(W.activations(cfg, T=T))
    ids, wts = gpu_lib.route(xt, to_dev_f32(W.router_weights(cfg)), cfg.n_group, cfg.topk_group, cfg.topk)
    xq = gpu_lib.quantize_activations(xt, "nvfp4")
    bad = ids.clone()
    bad[3, 0] = -1
    bad[T - 1, 1] = cfg.E + 5
    bad[T // 2, 0] = 1 << 30
    drop = bad != ids
    fixed_w = wts.clone()
    fixed_w[drop] = 0.0
    hs = torch.tensor([0.002], dtype=torch.float32, device="cuda")
    out_bad, ws = gpu_lib.moe_expert_mlp(gw, xq, bad, wts, h_global_scale=hs, return_workspace=True)
    out_ref = gpu_lib.moe_expert_mlp(gw, xq, ids, fixed_w, h_global_scale=hs)
    torch.cuda.synchronize()
    st = moe_stages(gpu_lib, "nvfp4", cfg, T, ws, T * cfg.topk)
    assert (st["pair_row"][np_(drop).ravel()] == -1).all()
    assert st["counts"].sum() == T * cfg.topk - int(drop.sum())
    assert torch.equal(out_bad, out_ref)
