"""Seeded synthetic inputs for the Beam-shaped MoE expert path.

This module only draws random numbers and casts them to the input dtypes; it
holds none of the method's arithmetic (no quantization, routing or GEMM), so
both the HIP path and the CPU oracle may take their inputs from it.

Shapes follow the pages: hidden 5120 ("Reflection releases Beam", "Model
architecture and attention"); 256 experts in 8 groups of 32, keep 4 groups,
top 8, intermediate 2560 ("Mixture-of-Experts details").  The value
distributions are synthetic stand-ins for Beam's weights and activations,
which the pages do not publish:
* activations bf16 N(0, 1); router weights N(0, 0.05) (bf16, fp32 in the tiny
  layer); expert weights bf16 N(0, 0.02);
* the standalone quantize tensor is Student-t(3) * 0.5 with 1 % of the rows
  multiplied by 50 (outlier rows);
* the prefill layer skews expert popularity by scaling router row e by
  c_e = C_MAX * rank_e^(-gamma) (rank_e a seeded permutation of 1..256), which
  leaves the router itself unbiased; gamma is stored in
  ``prefill_router_skew.json`` (written by ``calibrate_prefill_skew.py``).

Normals are drawn in float64 from ``numpy.random.default_rng(SeedSequence(
[config_id, tensor_tag, layer, expert]))``, scaled, rounded to float32 and then
to bf16 (round-to-nearest-even).  The large expert weight tensors can instead
be drawn on the GPU with torch's Philox generator (one seeded generator per
expert and tensor), so a 10-billion-parameter layer is ready in well under a
second; a test that needs those weights on the host copies them from the GPU.
"""

import json
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))

# tensor tags
T_X, T_WR, T_WG, T_WU, T_WD, T_QX, T_RANK = 1, 2, 3, 4, 5, 6, 7


@dataclass(frozen=True)
class LayerConfig:
    name: str
    config_id: int
    T: int
    H: int
    I: int
    E: int
    n_group: int
    topk_group: int
    topk: int
    combine_scale: float = 2.5
    router_fp32: bool = False
    layers: int = 1
    zipf_skew: bool = False
    x_std: float = 1.0
    wr_std: float = 0.05
    w_std: float = 0.02


TINY = LayerConfig("tiny", 1, T=64, H=256, I=128, E=16, n_group=4, topk_group=2, topk=2, router_fp32=True)
DECODE = LayerConfig("decode", 3, T=64, H=5120, I=2560, E=256, n_group=8, topk_group=4, topk=8)
PREFILL = LayerConfig("prefill", 4, T=8192, H=5120, I=2560, E=256, n_group=8, topk_group=4, topk=8, zipf_skew=True)
STACK = LayerConfig("stack", 5, T=4096, H=5120, I=2560, E=256, n_group=8, topk_group=4, topk=8, layers=4)
# the prefill layer without the popularity skew: every expert active (about 256 rows each)
PREFILL_UNIFORM = LayerConfig("prefill-uniform", 4, T=8192, H=5120, I=2560, E=256, n_group=8, topk_group=4,
                              topk=8)
CONFIGS = {c.name: c for c in (TINY, DECODE, PREFILL, STACK, PREFILL_UNIFORM)}

QUANT_SHAPE = (32768, 5120)  # standalone quantize workload
QUANT_OUTLIER_FRACTION = 0.01
QUANT_OUTLIER_FACTOR = 50.0

C_MAX = 1.6  # largest router-row scale: keeps sigma(logit) near 5.7 (no mass saturation)


def _rng(*tags):
    return np.random.default_rng(np.random.SeedSequence([int(t) for t in tags]))


def to_bf16_f32(a):
    """Round float32 values to bf16 (RNE) and return them as float32 (exactly)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def normal_host(shape, std, *tags, bf16=True):
    """float64 N(0,1) * std -> float32 (-> bf16); returned as a float32 array."""
    a = (_rng(*tags).standard_normal(shape) * std).astype(np.float32)
    return to_bf16_f32(a) if bf16 else a


def activations(cfg, layer=0, T=None):
    """x [T, H] bf16 values as float32."""
    return normal_host((T or cfg.T, cfg.H), cfg.x_std, cfg.config_id, T_X, layer, 0)


def prefill_skew_gamma():
    with open(os.path.join(_HERE, "prefill_router_skew.json")) as f:
        return float(json.load(f)["gamma"])


def router_row_scales(cfg, gamma=None):
    """c_e = C_MAX * rank_e^-gamma for the skewed (prefill) layer, else ones."""
    if not cfg.zipf_skew:
        return np.ones(cfg.E)
    g = prefill_skew_gamma() if gamma is None else gamma
    rank = _rng(cfg.config_id, T_RANK, 0, 0).permutation(cfg.E) + 1
    return C_MAX * rank.astype(np.float64) ** (-g)


def router_weights(cfg, layer=0, gamma=None):
    """W_r [E, H]: fp32 for the tiny layer, bf16 values (as float32) otherwise."""
    base = _rng(cfg.config_id, T_WR, layer, 0).standard_normal((cfg.E, cfg.H)) * cfg.wr_std
    base = base * router_row_scales(cfg, gamma)[:, None]
    a = base.astype(np.float32)
    return a if cfg.router_fp32 else to_bf16_f32(a)


def expert_weights_host(cfg, e, layer=0):
    """(W_gate [I, H], W_up [I, H], W_down [H, I]) bf16 values as float32, drawn on the host."""
    g = normal_host((cfg.I, cfg.H), cfg.w_std, cfg.config_id, T_WG, layer, e)
    u = normal_host((cfg.I, cfg.H), cfg.w_std, cfg.config_id, T_WU, layer, e)
    d = normal_host((cfg.H, cfg.I), cfg.w_std, cfg.config_id, T_WD, layer, e)
    return g, u, d


def _torch_seed(*tags):
    return int(np.random.SeedSequence([int(t) for t in tags]).generate_state(1, np.uint64)[0] >> 1)


def expert_weights_device(cfg, layer=0, device="cuda", experts=None):
    """W13 [E, 2I, H] (rows 0..I-1 gate, I..2I-1 up) and W2 [E, H, I], bf16 on ``device``.

    Each expert's tensors come from their own seeded Philox generator, so any
    subset can be regenerated alone.  ``experts``: optional list of expert ids
    (then the leading dimension is len(experts)).
    """
    ids = list(range(cfg.E)) if experts is None else list(experts)
    w13 = torch.empty((len(ids), 2 * cfg.I, cfg.H), dtype=torch.bfloat16, device=device)
    w2 = torch.empty((len(ids), cfg.H, cfg.I), dtype=torch.bfloat16, device=device)
    gen = torch.Generator(device=device)
    for i, e in enumerate(ids):
        for tag, dst in ((T_WG, w13[i, :cfg.I]), (T_WU, w13[i, cfg.I:]), (T_WD, w2[i])):
            gen.manual_seed(_torch_seed(cfg.config_id, tag, layer, e))
            r = torch.randn(dst.shape, generator=gen, device=device, dtype=torch.float32)
            dst.copy_((r * cfg.w_std).to(torch.bfloat16))
    return w13, w2


def quant_tensor_device(device="cuda", shape=QUANT_SHAPE, seed=2):
    """Standalone quantize input: Student-t(3) * 0.5, 1 % of rows x50, bf16 on ``device``."""
    R, C = shape
    gen = torch.Generator(device=device)
    gen.manual_seed(_torch_seed(seed, T_QX, 0, 0))
    z = torch.randn((R, C), generator=gen, device=device, dtype=torch.float32)
    # chi-square(3) as a sum of three squared normals, drawn in row blocks to bound memory
    chi = torch.zeros((R, C), device=device, dtype=torch.float32)
    for _ in range(3):
        chi.addcmul_(n := torch.randn((R, C), generator=gen, device=device, dtype=torch.float32), n)
    x = z / torch.sqrt(chi / 3.0) * 0.5
    n_out = int(round(QUANT_OUTLIER_FRACTION * R))
    rows = torch.from_numpy(_rng(seed, T_QX, 1, 0).choice(R, n_out, replace=False)).to(device)
    x[rows] *= QUANT_OUTLIER_FACTOR
    return x.to(torch.bfloat16)


def quant_tensor_host(shape, seed=2):
    """Host version of the standalone quantize input at a reduced shape (CPU tests)."""
    R, C = shape
    rng = _rng(seed, T_QX, 0, 1)
    x = (rng.standard_t(3, size=(R, C)) * 0.5).astype(np.float32)
    n_out = max(1, int(round(QUANT_OUTLIER_FRACTION * R)))
    rows = _rng(seed, T_QX, 1, 1).choice(R, n_out, replace=False)
    x[rows] *= np.float32(QUANT_OUTLIER_FACTOR)
    return to_bf16_f32(x)
