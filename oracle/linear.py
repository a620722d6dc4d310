"""Dense FP8_DYNAMIC (W8A8) linear projections and dense SwiGLU MLP.

TEST INFRASTRUCTURE ONLY -- part of the CPU oracle; never used by the product path.

Sources:
* "FP8 quantization" page, "Quantization scheme": the FP8_DYNAMIC checkpoint
  quantizes the attention query, key, value, output and gate projections and
  the dense MLPs' gate, up and down projections; E4M3 weights with a fixed
  scale per output channel, activation scales computed per token at run time.
  "Quantization method": values are divided by their scale and rounded to the
  nearest FP8 value (RTN).
* "Reflection releases Beam" news page, "Model architecture and attention":
  hidden 5120, 48 query heads and 8 key-value heads (head dimension 128 from
  "Long context handling and cache growth"), a sigmoid gate per channel of
  every head before the output projection; "Mixture-of-Experts details": the
  first three layers are dense SwiGLU MLPs.

Readings:
* a linear y = x W^T on FP8 operands is y[t, n] = fl32(s_x[t] s_w[n] sum_k
  q_x[t, k] q_w[n, k]), the product of the exactly decoded operands rounded
  once (the GPU accumulates in FP32); output FP32;
* the dense SwiGLU MLP is the expert MLP of the MoE path with one expert that
  every token selects with weight 1 and combine scale 1 (h quantized per row).

Parity: the linear is pinned by closed forms in the tests (unit and power-of-two
scales make every sum an exact float32 integer multiple of a power of two; a
one-hot weight row returns the decoded activation column); the dense MLP
inherits the expert MLP's pins.
"""

import numpy as np

from . import moe, quant


def fp8_linear(x, w):
    """x [T, K], w [N, K] float32 values -> (x codes/scales, w codes/scales, y [T, N] float32)."""
    xq = quant.fp8_quantize(x)
    wq = quant.fp8_quantize(w)
    y = moe.gemm_f32(quant.fp8_dequantize_exact(*xq), quant.fp8_dequantize_exact(*wq))
    return xq, wq, y


def fp8_dense_mlp(x, w_gate, w_up, w_down):
    """Dense FP8 SwiGLU MLP: one expert, every token routed to it with weight 1, scale 1."""
    T = x.shape[0]
    ex = moe.FP8Expert(w_gate, w_up, w_down)
    xq, xh = moe.quantize_activations(x, "fp8")
    ids = np.zeros((T, 1), np.int32)
    wts = np.ones((T, 1), np.float32)
    res = moe.moe_expert_mlp(xh, ids, wts, {0: ex}, "fp8", combine_scale=1.0)
    res["xq"] = xq
    res["expert"] = ex
    return res
