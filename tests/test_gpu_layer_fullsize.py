"""GPU parity of whole Beam-shaped MoE layers against the oracle, every token and every row.

"Reflection releases Beam" news page, "Mixture-of-Experts details": hidden
5120, 256 SwiGLU experts of intermediate 2560 in 8 groups of 32, the best 4
groups by their top-2 score sums, top 8 experts, normalized weights, x2.5.
NVFP4 ("NVFP4 quantization" page, "Quantization scheme") and FP8_DYNAMIC
("FP8 quantization" page, "Quantization scheme") weights and activations, and
the weight-only variant (NVFP4 weights, BF16 activations: "Beam-1.0 auf 4x
NVIDIA RTX PRO 6000 Blackwell Server Edition", "NVFP4 auf Blackwell gegen FP8
auf Hopper").

Decode: 64 tokens (about 222 active experts).  Prefill: 8192 tokens with the
Zipf-like router skew (67 active experts, the largest above 4000 rows).  The
oracle quantizes every active expert itself from the same bf16 masters; the
stage-by-stage protocol is in tests/fullsize.py.  Each case takes tens of
seconds of host time (oracle GEMMs in binary64).
"""

import pytest
import torch

import workloads as W
from tests.fullsize import check_layer, check_layer_w4a16

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _layer(gpu_lib, cfg, fmt):
    x, wr = W.activations(cfg), W.router_weights(cfg)
    w13, w2 = W.expert_weights_device(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, fmt)
    res = check_layer(gpu_lib, fmt, cfg, x, wr, w13, w2, gw, f"{cfg.name}-{cfg.T} {fmt}")
    del w13, w2, gw
    torch.cuda.empty_cache()
    return res


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_layer_decode64_full(gpu_lib, fmt):
    res = _layer(gpu_lib, W.DECODE, fmt)
    assert res["active"] > 200


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_layer_prefill8192_full(gpu_lib, fmt):
    res = _layer(gpu_lib, W.PREFILL, fmt)
    assert res["max_rows"] > 1000


@pytest.mark.parametrize("cfg", [W.DECODE, W.PREFILL], ids=["decode64", "prefill8192"])
def test_layer_w4a16_full(gpu_lib, cfg):
    x, wr = W.activations(cfg), W.router_weights(cfg)
    w13, w2 = W.expert_weights_device(cfg)
    gw = gpu_lib.quantize_expert_weights(w13, w2, "nvfp4")
    res = check_layer_w4a16(gpu_lib, cfg, x, wr, w13, w2, gw, f"{cfg.name}-{cfg.T} w4a16")
    assert res["max_rows"] > (1000 if cfg.T > 64 else 1)
