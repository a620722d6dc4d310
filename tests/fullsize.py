"""Full-size (Beam-shaped) oracle comparisons shared by the layer and stack parity tests.

The oracle quantizes every expert it touches from the same bf16 masters the
GPU quantized (copied back from the device), with its C quantizers, and those
codes are compared bit-exactly with the GPU's weights before the oracle uses
them; no oracle input comes from the GPU's quantization.

Comparison protocol (per layer): routing ids and weights bit-exact, activation
codes bit-exact; h of every row within 1e-5 relative L2 of the oracle's h;
the oracle's quantizer applied to the GPU's h reproduces the GPU's h codes
bit-exactly; y from those identical h codes within 1e-5; the combine of the
GPU's y within 1e-6; the layer output within 1e-3 of the oracle's own
end-to-end output; every h code on which the GPU's and the oracle's own
quantizations differ is a near-tie (the two h values behind it within 1e-5 of
the row's RMS, so the codes differ only because a rounding midpoint lies
between them).
"""

import numpy as np
import torch

from oracle import formats as F
from oracle import moe as OM
from oracle import quant_c as QC
from oracle import route as OR
from oracle.quant import unpack_e2m1
from tests.helpers import moe_stages, np_, rel_l2, to_dev_bf16, weights_match, ws_view

STAGE_TOL = 1e-5
LAYER_TOL = 1e-3
TIE_TOL = 1e-5

def bf16_bits(t):
    """A device bf16 tensor as its uint16 bit patterns on the host (the C quantizers read them exactly)."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceExperts:
    """Mapping e -> oracle expert, quantized by the oracle from the device bf16 masters on first use.

    Each expert's GPU-quantized weights are compared bit-exactly with the oracle's codes, scales and
    global scales before the oracle uses them.
    """

    def __init__(self, w13, w2, gpu_weights, fmt):
        self.w13, self.w2, self.gw, self.fmt = w13, w2, gpu_weights, fmt
        self.I = w13.shape[1] // 2
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            cls = OM.FP8Expert if self.fmt == "fp8" else OM.NVFP4Expert
            ex = cls(bf16_bits(self.w13[e, :self.I]), bf16_bits(self.w13[e, self.I:]), bf16_bits(self.w2[e]), q=QC)
            weights_match(self.gw, {e: ex}, self.fmt, [e])
            self.cache[e] = ex
        return self.cache[e]


def code_flips(fmt, h_ref, h_gpu, q_ref, q_gpu):
    """Explain every h code on which the oracle's quantization of its own h differs from the GPU's codes.

    Elements counted: codes that differ, and every element of an NVFP4 block whose E4M3 scale differs
    (the block maximum moved across a scale midpoint).  Nearest rounding is monotone, so a code differs
    only where a rounding midpoint lies between the two quotients; the difference is a near-tie when
    the two h values behind it are close: |h_gpu - h_oracle| within TIE_TOL of the RMS of the oracle's
    h over that row (the FP32 accumulation error of g and u scales with the row, not with the element,
    so a relative bound per element would reject small elements with cancellation).
    Returns (differing scales, differing elements, worst |h_gpu - h_oracle| / RMS over them).
    """
    h_ref = np.asarray(h_ref, np.float32)
    h_gpu = np.asarray(h_gpu, np.float32)
    P, C = h_ref.shape
    if fmt == "nvfp4":
        sdiff = q_ref[1] != q_gpu[1]
        cdiff = unpack_e2m1(q_ref[0]) != unpack_e2m1(q_gpu[0])
        flip = cdiff | np.repeat(sdiff, 16, axis=1)
        n_scale = int(sdiff.sum())
    else:
        flip = q_ref[0] != q_gpu[0]
        n_scale = int((q_ref[1] != q_gpu[1]).sum())
    rows, cols = np.nonzero(flip)
    worst = 0.0
    if len(rows):
        rms = np.sqrt(np.mean(h_ref.astype(np.float64) ** 2, axis=1))
        err = np.abs(h_gpu[rows, cols].astype(np.float64) - h_ref[rows, cols]) / np.maximum(rms[rows], 1e-300)
        worst = float(err.max())
    return n_scale, int(flip.sum()), worst


def check_layer(gpu_lib, fmt, cfg, x, wr, w13, w2, gw, label):
    """Run the GPU layer (route -> quantize -> expert MLP) on bf16 x and compare it with the oracle in full."""
    T = x.shape[0]
    xt = to_dev_bf16(x)
    ids, wts = gpu_lib.route(xt, to_dev_bf16(wr), cfg.n_group, cfg.topk_group, cfg.topk)
    xq = gpu_lib.quantize_activations(xt, fmt)
    out, ws = gpu_lib.moe_expert_mlp(gw, xq, ids, wts, cfg.combine_scale, return_workspace=True)
    torch.cuda.synchronize()
    P = T * cfg.topk
    st = moe_stages(gpu_lib, fmt, cfg, T, ws, P)
    out = np_(out)
    del ws
    torch.cuda.empty_cache()

    print(f"{label}: GPU layer done, oracle routing", flush=True)
    # routing, activation quantization: bit-exact
    oi, ow, _, _ = OR.route(x, wr, cfg.n_group, cfg.topk_group, cfg.topk)
    assert np.array_equal(np_(ids), oi), f"{label}: routing ids differ"
    assert np.array_equal(np_(wts).view(np.uint32), ow.view(np.uint32)), f"{label}: routing weights differ"
    xq_o, x_hat = OM.quantize_activations(x, fmt, q=QC)
    for a, b in zip(xq, xq_o):
        assert np.array_equal(np_(a).reshape(np.shape(b)), b), f"{label}: activation quantization differs"
    counts, offsets, row_of_pair, pair_of_row = OM.permute(oi, cfg.E)
    assert np.array_equal(st["row_pair"], pair_of_row) and np.array_equal(st["counts"], counts)

    # the oracle's own layer on its own quantization of the same masters
    print(f"{label}: oracle expert MLP over {int((counts > 0).sum())} experts", flush=True)
    experts = DeviceExperts(w13, w2, gw, fmt)
    ref = OM.moe_expert_mlp(x_hat, oi, ow, experts, fmt, cfg.combine_scale, q=QC)
    res = {"active": int((counts > 0).sum()), "max_rows": int(counts.max())}

    # stage 1: h of every row
    res["h"] = rel_l2(st["h"][row_of_pair], ref["h"])
    assert res["h"] <= STAGE_TOL, f"{label}: h rel L2 {res['h']:.3e}"
    # stage 2: the oracle's quantizer on the GPU's h reproduces the GPU's h codes
    if fmt == "nvfp4":
        hq_g = QC.nvfp4_quantize(st["h"])
        assert st["hg"].view(np.uint32) == hq_g[2].view(np.uint32), f"{label}: h global scale differs"
        hh = QC.nvfp4_dequantize_exact(*hq_g)
    else:
        hq_g = QC.fp8_quantize(st["h"])
        hh = QC.fp8_dequantize_exact(*hq_g)
    assert np.array_equal(st["hc"], hq_g[0]) and np.array_equal(st["hs"], hq_g[1]), f"{label}: h codes differ"
    print(f"{label}: oracle down projection from the GPU's h codes", flush=True)
    # stage 3: the down projection from those identical h codes, every row
    y_tf = np.zeros_like(st["y"])
    for e in np.nonzero(counts)[0]:
        rows = np.arange(offsets[e], offsets[e + 1])
        y_tf[rows] = OM.gemm_f32(hh[rows], experts[e].decoded_down())
    del hh
    res["y"] = rel_l2(st["y"], y_tf)
    assert res["y"] <= STAGE_TOL, f"{label}: y rel L2 {res['y']:.3e}"
    del y_tf
    # stage 4: the combine of the GPU's y
    comb = OM.combine_f32(st["y"][row_of_pair].reshape(T, cfg.topk, -1), ow, cfg.combine_scale)
    res["combine"] = rel_l2(out, comb)
    assert res["combine"] <= 1e-6, f"{label}: combine rel L2 {res['combine']:.3e}"
    del comb
    # h code differences against the oracle's own quantization of its own h are near-ties
    hg_pairs = st["h"][row_of_pair]
    if fmt == "nvfp4":
        q_gp = (st["hc"][row_of_pair], st["hs"][row_of_pair], st["hg"])
        res["h_gs_rel"] = abs(float(st["hg"]) / float(ref["hq"][2]) - 1.0)
    else:
        q_gp = (st["hc"][row_of_pair], st["hs"][row_of_pair])
    ns, nc, worst = code_flips(fmt, ref["h"], hg_pairs, ref["hq"], q_gp)
    del hg_pairs
    res["h_scale_flips"], res["h_code_flips"], res["flip_h_err"] = ns, nc, worst
    print(f"{label}: {res}", flush=True)
    assert worst <= TIE_TOL, f"{label}: an h code differs from the oracle's by more than a near-tie ({worst:.3e})"
    # end to end
    res["out"] = rel_l2(out, ref["out"])
    print(f"{label}: layer output rel L2 {res['out']:.3e}", flush=True)
    assert res["out"] <= LAYER_TOL, f"{label}: layer output rel L2 {res['out']:.3e}"
    return res


def check_layer_w4a16(gpu_lib, cfg, x, wr, w13, w2, gw, label):
    """The weight-only layer (NVFP4 weights, BF16 x and h) on bf16 x against the oracle in full: routing
    bit-exact; h of every row within 1e-5; y from the GPU's own h rounded to BF16 within 1e-5; the combine
    of the GPU's y within 1e-6; the output within 1e-3 of the oracle's own end-to-end layer."""
    T = x.shape[0]
    xt = to_dev_bf16(x)
    ids, wts = gpu_lib.route(xt, to_dev_bf16(wr), cfg.n_group, cfg.topk_group, cfg.topk)
    out, ws = gpu_lib.moe_expert_mlp_w4a16(gw, xt, ids, wts, cfg.combine_scale, return_workspace=True)
    torch.cuda.synchronize()
    P = T * cfg.topk
    lay = gpu_lib.moe_workspace_layout("w4a16", cfg.E, cfg.H, cfg.I, T, cfg.topk)
    h = np_(ws_view(ws, lay, "h_f32", torch.float32, (P, cfg.I)))
    y = np_(ws_view(ws, lay, "y_f32", torch.float32, (P, cfg.H)))
    row_pair = np_(ws_view(ws, lay, "row_pair", torch.int32, (P,)))
    out = np_(out)
    del ws
    torch.cuda.empty_cache()
    print(f"{label}: GPU layer done, oracle routing", flush=True)
    oi, ow, _, _ = OR.route(x, wr, cfg.n_group, cfg.topk_group, cfg.topk)
    assert np.array_equal(np_(ids), oi), f"{label}: routing ids differ"
    assert np.array_equal(np_(wts).view(np.uint32), ow.view(np.uint32)), f"{label}: routing weights differ"
    counts, offsets, row_of_pair, pair_of_row = OM.permute(oi, cfg.E)
    assert np.array_equal(row_pair, pair_of_row)
    print(f"{label}: oracle expert MLP over {int((counts > 0).sum())} experts", flush=True)
    experts = DeviceExperts(w13, w2, gw, "nvfp4")
    ref = OM.moe_expert_mlp(x.astype(np.float64), oi, ow, experts, "w4a16", cfg.combine_scale, q=QC)
    res = {"active": int((counts > 0).sum()), "max_rows": int(counts.max())}
    res["h"] = rel_l2(h[row_of_pair], ref["h"])
    assert res["h"] <= STAGE_TOL, f"{label}: h rel L2 {res['h']:.3e}"
    hb = F.bf16_round(h).astype(np.float64)
    y_tf = np.zeros_like(y)
    for e in np.nonzero(counts)[0]:
        rows = np.arange(offsets[e], offsets[e + 1])
        y_tf[rows] = OM.gemm_f32(hb[rows], experts[e].decoded_down())
    del hb
    res["y"] = rel_l2(y, y_tf)
    assert res["y"] <= STAGE_TOL, f"{label}: y rel L2 {res['y']:.3e}"
    del y_tf
    comb = OM.combine_f32(y[row_of_pair].reshape(T, cfg.topk, -1), ow, cfg.combine_scale)
    res["combine"] = rel_l2(out, comb)
    assert res["combine"] <= 1e-6, f"{label}: combine rel L2 {res['combine']:.3e}"
    res["out"] = rel_l2(out, ref["out"])
    print(f"{label}: {res}", flush=True)
    assert res["out"] <= LAYER_TOL, f"{label}: layer output rel L2 {res['out']:.3e}"
    return res
