"""Dense FP8_DYNAMIC (W8A8) linear projections and dense SwiGLU MLP.

TEST INFRASTRUCTURE ONLY -- part of the CPU oracle; never used by the product path.

Sources:
* "FP8 quantization" page, "Quantization scheme": in the FP8_DYNAMIC
  checkpoint the attention projections (q, k, v, o and the head gate) and the
  three projections of each dense MLP are FP8 too; a weight row has one fixed
  E4M3 scale, an activation row a scale found per token at run time.
  "Quantization method": RTN, the closest E4M3 value to value / scale.
* "Reflection releases Beam" news page, "Model architecture and attention":
  hidden 5120, 8 KV heads and 48 query heads (128 dimensions each, from "Long
  context handling and cache growth"), and a per-channel sigmoid gate on each
  head's output ahead of the o projection; "Mixture-of-Experts details":
  layers 1 to 3 use dense SwiGLU MLPs instead of experts.

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


def fp8_linear(x, w, q=quant):
    """x [T, K], w [N, K] float32 values -> (x codes/scales, w codes/scales, y [T, N] float32).

    q: quantizer module (``oracle.quant`` or the bit-identical ``oracle.quant_c``)."""
    xq = q.fp8_quantize(x)
    wq = q.fp8_quantize(w)
    y = moe.gemm_f32(q.fp8_dequantize_exact(*xq), q.fp8_dequantize_exact(*wq))
    return xq, wq, y


def fp8_dense_mlp(x, w_gate, w_up, w_down, q=quant):
    """Dense FP8 SwiGLU MLP: one expert, every token routed to it with weight 1, scale 1."""
    T = x.shape[0]
    ex = moe.FP8Expert(w_gate, w_up, w_down, q=q)
    xq, xh = moe.quantize_activations(x, "fp8", q=q)
    ids = np.zeros((T, 1), np.int32)
    wts = np.ones((T, 1), np.float32)
    res = moe.moe_expert_mlp(xh, ids, wts, {0: ex}, "fp8", combine_scale=1.0, q=q)
    res["xq"] = xq
    res["expert"] = ex
    return res
