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
