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
quantizations differ is a near-tie (the oracle's quotient within 1e-5
relative of a rounding midpoint of the format).
"""

import numpy as np
import torch

from oracle import formats as F
from oracle import moe as OM
from oracle import quant_c as QC
from oracle import route as OR
from oracle.quant import unpack_e2m1
from tests.helpers import moe_stages, np_, rel_l2, to_dev_bf16, weights_match

STAGE_TOL = 1e-5
LAYER_TOL = 1e-3
TIE_TOL = 1e-5

E2M1_MID = (F.E2M1_MAGNITUDES[:-1] + F.E2M1_MAGNITUDES[1:]) / 2
E4M3_MID = (F.E4M3_MAGNITUDES[:-1] + F.E4M3_MAGNITUDES[1:]) / 2


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


def _near_midpoint(r, mids, tol=TIE_TOL):
    """|r| lies within tol * |r| of one of the (increasing) midpoints."""
    r = np.abs(np.asarray(r, np.float64))
    j = np.clip(np.searchsorted(mids, r), 1, len(mids) - 1)
    d = np.minimum(np.abs(r - mids[j - 1]), np.abs(r - mids[j]))
    return d <= tol * r


def nvfp4_flips(h_ref, q_ref, q_gpu):
    """Where two NVFP4 quantizations of (nearly) the same h differ, check each difference is a near-tie.

    Blocks whose E4M3 scale differs: the oracle's a_b / fl32(6 S_g) lies within TIE_TOL of an E4M3
    midpoint.  Elements of blocks with equal scales whose codes differ: the oracle's x / fl32(s_b S_g)
    lies within TIE_TOL of an E2M1 midpoint.  Returns (scale flips, code flips, all near-ties).
    """
    c_r, s_r, g_r = q_ref
    c_g, s_g, _ = q_gpu
    P, nb = s_r.shape
    blk = np.asarray(h_ref, np.float32).reshape(P, nb, 16)
    sdiff = s_r != s_g
    ok = True
    if sdiff.any():
        ab = np.abs(blk[sdiff]).max(-1)
        d1 = np.float32(np.float32(6.0) * g_r)
        ok &= bool(_near_midpoint(ab / d1, E4M3_MID).all())
    q_r = unpack_e2m1(c_r).reshape(P, nb, 16)
    q_g = unpack_e2m1(c_g).reshape(P, nb, 16)
    cdiff = (q_r != q_g) & ~sdiff[..., None]
    if cdiff.any():
        sb = F.e4m3_decode(s_r).astype(np.float32)
        d2 = (sb * g_r).astype(np.float32)
        r = blk / np.broadcast_to(d2[..., None], blk.shape)
        ok &= bool(_near_midpoint(r[cdiff], E2M1_MID).all())
    return int(sdiff.sum()), int(cdiff.sum()), ok


def fp8_flips(h_ref, q_ref, q_gpu):
    """FP8 per row: every differing code's oracle quotient x / s lies within TIE_TOL of an E4M3 midpoint."""
    c_r, s_r = q_ref
    c_g, _ = q_gpu
    diff = c_r != c_g
    ok = True
    if diff.any():
        r = np.asarray(h_ref, np.float32) / s_r[:, None]
        ok = bool(_near_midpoint(r[diff], E4M3_MID).all())
    return 0, int(diff.sum()), ok


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
    if fmt == "nvfp4":
        q_gp = (st["hc"][row_of_pair], st["hs"][row_of_pair], st["hg"])
        ns, nc, ok = nvfp4_flips(ref["h"], ref["hq"], q_gp)
    else:
        q_gp = (st["hc"][row_of_pair], st["hs"][row_of_pair])
        ns, nc, ok = fp8_flips(ref["h"], ref["hq"], q_gp)
    res["h_scale_flips"], res["h_code_flips"] = ns, nc
    assert ok, f"{label}: an h code differs from the oracle's away from a rounding midpoint"
    # end to end
    res["out"] = rel_l2(out, ref["out"])
    print(f"{label}: {res}", flush=True)
    assert res["out"] <= LAYER_TOL, f"{label}: layer output rel L2 {res['out']:.3e}"
    return res
