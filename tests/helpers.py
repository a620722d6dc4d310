"""Shared helpers for the GPU parity tests (host <-> device, comparisons, oracle weights)."""

import numpy as np
import torch

import workloads as W
from oracle import moe as OM

DEV = "cuda"


def to_dev_bf16(a):
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)
    out = t.to(torch.bfloat16)
    assert torch.equal(out.float(), t), "values are not bf16-exact"
    return out


def to_dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def np_(t):
    return t.detach().cpu().numpy()


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def host_masters(cfg, layer=0):
    """Per-expert (gate, up, down) bf16 masters drawn on the host, and their device W13/W2."""
    masters = [W.expert_weights_host(cfg, e, layer) for e in range(cfg.E)]
    w13 = np.stack([np.concatenate([g, u]) for g, u, _ in masters])
    w2 = np.stack([d for _, _, d in masters])
    return masters, to_dev_bf16(w13), to_dev_bf16(w2)


def oracle_experts(masters, fmt, ids=None):
    cls = OM.FP8Expert if fmt == "fp8" else OM.NVFP4Expert  # W4A16 uses the NVFP4 weights
    keep = range(len(masters)) if ids is None else sorted(set(int(e) for e in np.asarray(ids).ravel()))
    return {e: cls(*masters[e]) for e in keep}


def ws_view(ws, lay, key, dtype, shape):
    """Typed view of a stage buffer inside the expert-MLP workspace."""
    n = int(np.prod(shape))
    itemsize = torch.tensor([], dtype=dtype).element_size()
    start = lay[key]
    return ws[start:start + n * itemsize].view(dtype).reshape(shape)


def weights_match(gpu_w, experts, fmt, ids):
    """The GPU-quantized weights of experts ``ids`` equal the oracle experts' codes, scales and global scales."""
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


def moe_stages(gpu_lib, fmt, cfg, T, ws, P):
    """The expert-MLP workspace's stage buffers (permutation, h, h codes and scales, y) on the host."""
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
