"""GPU: the pair layout of the expert weights (bsm_codes_to_pairs, and for NVFP4 the lane-ordered copies of
the block scales from bsm_scales_to_lanes).

The codes are the canonical NVFP4 / FP8 codes ("NVFP4 quantization" and "FP8 quantization" pages,
"Quantization scheme"); only their order in memory changes.  Checked here:
  - both permutations against their definitions, written independently (reshape, transpose, byte order);
  - the routed-expert MLP on pair-layout weights gives the same output, bit for bit, as on the canonical
    layout (the kernels feed the same operands to the same MFMA lanes in the same order), at a mid shape
    with few-row and many-row experts and at the Beam decode and prefill shapes, in NVFP4, FP8 and W4A16.
The canonical path itself is checked against the oracle elsewhere (test_gpu_moe, test_gpu_layer_fullsize).
"""

import numpy as np
import pytest
import torch

import workloads as W
from tests.helpers import np_, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


def _pairs_reference(codes):
    """In each block of 16 rows, row m = 8 h + p, 64-byte chunk c goes to double row p, line c, half h."""
    rb = codes.shape[-1]
    x = codes.reshape(-1, 2, 8, rb // 64, 64)
    return np.ascontiguousarray(x.transpose(0, 2, 3, 1, 4)).reshape(codes.shape)


@pytest.mark.parametrize("rows,rb", [(16, 64), (48, 128), (5120, 2560), (5120, 320)])
def test_codes_to_pairs_definition(gpu_lib, rows, rb):
    rng = np.random.default_rng(rows + rb)
    c = rng.integers(0, 256, size=(rows, rb), dtype=np.uint8)
    out = gpu_lib.codes_to_pairs(torch.from_numpy(c).cuda())
    torch.cuda.synchronize()
    got = np_(out)
    assert np.array_equal(got, _pairs_reference(c))
    assert not np.array_equal(got, c)


def _lanes_reference(scales):
    """Per 16-row block and 32-byte span st (512 values): the block's 16 rows in order, each row's block b
    at byte 8 * (lane group) + 2 * (piece) + (block of the piece), with piece b // 8 and lane group
    (b // 2) % 4."""
    rows, rb = scales.shape
    x = scales.reshape(rows // 16, 16, rb // 32, 32).transpose(0, 2, 1, 3)  # block, span, row, byte
    pos = np.array([8 * ((b // 2) % 4) + 2 * (b // 8) + b % 2 for b in range(32)])
    out = np.empty_like(x)
    out[..., pos] = x
    return np.ascontiguousarray(out).reshape(rows, rb)


@pytest.mark.parametrize("rows,rb", [(16, 32), (48, 64), (5120, 320), (5120, 160)])
def test_scales_to_lanes_definition(gpu_lib, rows, rb):
    rng = np.random.default_rng(7 * rows + rb)
    s = rng.integers(0, 127, size=(rows, rb), dtype=np.uint8)
    out = gpu_lib.scales_to_lanes(torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    got = np_(out)
    assert np.array_equal(got, _lanes_reference(s))
    assert np.array_equal(np.sort(got, axis=None), np.sort(s, axis=None))


def _outputs(gpu_lib, cfg, fmt, T, w13, w2):
    """Layer output on the canonical and on the pair layout of the same quantized weights."""
    x, wr = W.activations(cfg, T=T), W.router_weights(cfg)
    xt = to_dev_bf16(x) if not isinstance(x, torch.Tensor) else x
    wrt = to_dev_f32(wr) if not isinstance(wr, torch.Tensor) else wr
    ids, wts = gpu_lib.route(xt, wrt, cfg.n_group, cfg.topk_group, cfg.topk)
    gw = gpu_lib.quantize_expert_weights(w13, w2, "nvfp4" if fmt == "w4a16" else fmt)
    gp = gpu_lib.to_pair_layout(gw)
    assert gp.layout == gpu_lib.LAYOUT_PAIRS and gp.w13_scales is gw.w13_scales
    assert (gp.w13_scales_lanes is None) == (fmt == "fp8")
    if fmt == "w4a16":
        o_rows = gpu_lib.moe_expert_mlp_w4a16(gw, xt, ids, wts, cfg.combine_scale)
        o_pairs = gpu_lib.moe_expert_mlp_w4a16(gp, xt, ids, wts, cfg.combine_scale)
    else:
        xq = gpu_lib.quantize_activations(xt, fmt)
        o_rows = gpu_lib.moe_expert_mlp(gw, xq, ids, wts, cfg.combine_scale)
        o_pairs = gpu_lib.moe_expert_mlp(gp, xq, ids, wts, cfg.combine_scale)
    torch.cuda.synchronize()
    counts = np.bincount(np_(ids).ravel(), minlength=cfg.E)
    return np_(o_rows), np_(o_pairs), counts


# hidden 1024, intermediate 512 (multiples of the few-row K step, 512), 8 experts
MIDP = W.LayerConfig("mid-pairs", 9, T=700, H=1024, I=512, E=8, n_group=2, topk_group=1, topk=2, router_fp32=True)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8", "w4a16"])
@pytest.mark.parametrize("T", [64, 700])
def test_moe_pairs_bitexact_mid(gpu_lib, fmt, T):
    """T = 64: every expert below 64 rows (few-row kernel); T = 700: experts above 64 rows (many-row kernel)."""
    from tests.helpers import host_masters

    _, w13, w2 = host_masters(MIDP)
    o_rows, o_pairs, counts = _outputs(gpu_lib, MIDP, fmt, T, w13, w2)
    assert (counts.max() <= 64) if T == 64 else (counts.max() > 64)
    assert np.isfinite(o_rows).all()
    assert np.array_equal(o_rows.view(np.uint32), o_pairs.view(np.uint32))


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("cfg", [W.DECODE, W.PREFILL], ids=["decode64", "prefill8192"])
def test_moe_pairs_bitexact_beam(gpu_lib, cfg, fmt):
    w13, w2 = W.expert_weights_device(cfg)
    x = to_dev_bf16(W.activations(cfg))
    wr = to_dev_f32(W.router_weights(cfg))
    ids, wts = gpu_lib.route(x, wr, cfg.n_group, cfg.topk_group, cfg.topk)
    gw = gpu_lib.quantize_expert_weights(w13, w2, fmt)
    del w13, w2
    gp = gpu_lib.to_pair_layout(gw)
    xq = gpu_lib.quantize_activations(x, fmt)
    o_rows = gpu_lib.moe_expert_mlp(gw, xq, ids, wts, cfg.combine_scale)
    o_pairs = gpu_lib.moe_expert_mlp(gp, xq, ids, wts, cfg.combine_scale)
    torch.cuda.synchronize()
    a, b = np_(o_rows), np_(o_pairs)
    assert np.isfinite(a).all()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    del gw, gp
    torch.cuda.empty_cache()
