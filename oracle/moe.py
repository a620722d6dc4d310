"""Routed-expert MoE MLP (NVFP4 W4A4 and FP8_DYNAMIC W8A8), RMSNorm and residual.

TEST INFRASTRUCTURE ONLY -- part of the CPU oracle; never used by the product path.

Sources:
* "Reflection releases Beam" news page, "Mixture-of-Experts details": the
  experts are SwiGLU MLPs (hidden 5120, intermediate 2560); the layer output
  is the sum of the chosen experts' outputs, each weighted by its score over
  the sum of the chosen scores, times 2.5.
  "Residual stream and numerical decisions": the SwiGLU product and the norms
  run in FP32; the embedding counts as step 1, and step k scales the stream by
  sqrt((k-1)/k) before adding the sublayer output scaled by 1/sqrt(k).
* "NVFP4 quantization" page, "Quantization scheme": W4A4 -- the expert
  weights and the expert inputs are NVFP4; of the whole model, just the gate,
  up and down matrices of the routed experts are NVFP4.
* "FP8 quantization" page, "Quantization scheme": W8A8 with per-output-channel
  weight scales and per-token activation scales.
* "Beam-1.0 auf 4x NVIDIA RTX PRO 6000 Blackwell Server Edition" page,
  section "NVFP4 auf Blackwell gegen FP8 auf Hopper" (and the H100 line of the
  "NVFP4 quantization" page, "Hardware compatibility and serving"): without
  FP4 arithmetic the NVFP4 experts run weight-only (W4A16) -- FP4 weights,
  BF16 activations, 16-bit arithmetic speed.

Readings (listed with the others in the design notes):
* SwiGLU h = fl32(silu(g) * u), silu(g) = g / (1 + exp(-g)), evaluated in
  float64 from the float32 g and u, no clamp, no bias;
* g, u and the down projection y are fl32 of the exact dot products of the
  exactly decoded operands (float64 GEMMs; their rounding error is far below
  the comparison tolerance);
* the intermediate h of the NVFP4 path carries ONE dynamic global scale over
  all (token, expert) rows of the call; the FP8 path quantizes h per row;
* weight-only W4A16: the activations are the BF16 inputs themselves (no
  activation quantization) and h is rounded to BF16 (nearest, ties to even)
  before the down projection, the 16-bit activation type of the layer;
* out[t] = fl32(2.5 * sum_j w[t, j] * y[t, j]) in float64, output float32;
* rows of expert e are ordered by (token, slot) -- the stable order.
* RMSNorm: ms = fl32(mean(x^2)) with the mean in float64, r = fl32(1 /
  sqrt(ms + eps)) in float64, n = fl32(x * r), eps = 1e-6, gain 1 (a given
  gain gamma multiplies after that rounding: fl32(n * gamma)).
* residual: x <- fl32(a_k * x + b_k * m), a_k = fl32(sqrt((k-1)/k)),
  b_k = fl32(1/sqrt(k)), evaluated in float64.

Parity: the expert MLP is pinned by closed forms: unit scales make every
product sum an exact float32 integer multiple of 1/4; identical experts make
the output independent of the routing (2.5 * one expert); a single selected
expert reduces to a textbook NumPy SwiGLU MLP.  The residual weights satisfy
a_k^2 + b_k^2 = 1 (pinned).  SwiGLU and RMSNorm values themselves are checked
against a direct float64 evaluation only (tolerance parity).
"""

import numpy as np

from . import formats, quant
from .route import route as _route

F32 = np.float32


# --------------------------------------------------------------------------
# permutation (a5): rows of each expert in stable (token, slot) order
# --------------------------------------------------------------------------


def permute(ids, n_experts):
    """Return (counts [E], offsets [E+1], row_of_pair [T*k], pair_of_row [T*k]).

    Pair p = t*k + j.  Expert e owns rows offsets[e] .. offsets[e+1]-1; inside
    an expert the pairs appear in increasing p (the stable order).
    """
    ids = np.asarray(ids).reshape(-1)
    counts = np.bincount(ids, minlength=n_experts).astype(np.int32)
    offsets = np.zeros(n_experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    pair_of_row = np.argsort(ids, kind="stable").astype(np.int32)
    row_of_pair = np.empty_like(pair_of_row)
    row_of_pair[pair_of_row] = np.arange(len(ids), dtype=np.int32)
    return counts, offsets, row_of_pair, pair_of_row


# --------------------------------------------------------------------------
# stages
# --------------------------------------------------------------------------


def swiglu_f32(g, u):
    """h = fl32(silu(g) * u) with silu(g) = g / (1 + exp(-g)) in float64."""
    g64 = np.asarray(g, np.float32).astype(np.float64)
    u64 = np.asarray(u, np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        silu = g64 / (1.0 + np.exp(-g64))
    return (silu * u64).astype(np.float32)


def gemm_f32(a_hat, b_hat):
    """fl32(a_hat @ b_hat.T) on exactly decoded float64 operands."""
    return (np.asarray(a_hat, np.float64) @ np.asarray(b_hat, np.float64).T).astype(np.float32)


def combine_f32(y_pairs, w, scale):
    """out[t] = fl32(scale * sum_j w[t, j] * y[t, j]), sum in float64.

    y_pairs: [T, k, H] float32; w: [T, k] float32.
    """
    acc = np.einsum("tk,tkh->th", np.asarray(w, np.float64), np.asarray(y_pairs, np.float64))
    return (np.float64(scale) * acc).astype(np.float32)


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------


class NVFP4Expert:
    """One expert's gate / up / down projections quantized to NVFP4 (RTN).

    ``q``: the quantizer module, ``oracle.quant`` or its C transcription
    ``oracle.quant_c`` (bit-identical, for full-size experts).
    """

    def __init__(self, w_gate, w_up, w_down, q=quant):
        self.q = q
        self.gate = q.nvfp4_quantize(w_gate)
        self.up = q.nvfp4_quantize(w_up)
        self.down = q.nvfp4_quantize(w_down)

    def decoded_gate_up(self):
        return tuple(self.q.nvfp4_dequantize_exact(*p) for p in (self.gate, self.up))

    def decoded_down(self):
        return self.q.nvfp4_dequantize_exact(*self.down)

    def decoded(self):
        return self.decoded_gate_up() + (self.decoded_down(),)


class FP8Expert:
    """One expert's gate / up / down projections quantized per output channel."""

    def __init__(self, w_gate, w_up, w_down, q=quant):
        self.q = q
        self.gate = q.fp8_quantize(w_gate)
        self.up = q.fp8_quantize(w_up)
        self.down = q.fp8_quantize(w_down)

    def decoded_gate_up(self):
        return tuple(self.q.fp8_dequantize_exact(*p) for p in (self.gate, self.up))

    def decoded_down(self):
        return self.q.fp8_dequantize_exact(*self.down)

    def decoded(self):
        return self.decoded_gate_up() + (self.decoded_down(),)


# --------------------------------------------------------------------------
# the expert MLP over routed pairs
# --------------------------------------------------------------------------


def quantize_activations(x, fmt, global_scale=None, q=quant):
    """Quantize activations and return (packed quantities, exact decoded float64).

    Weight-only W4A16 keeps the BF16 activations: (None, x) with x BF16-exact.
    """
    if fmt == "w4a16":
        x = np.asarray(x, np.float32)
        assert np.array_equal(formats.bf16_round(x), x), "W4A16 activations must be BF16 values"
        return None, x.astype(np.float64)
    if fmt == "nvfp4":
        xq = q.nvfp4_quantize(x, global_scale)
        return xq, q.nvfp4_dequantize_exact(*xq)
    xq = q.fp8_quantize(x)
    return xq, q.fp8_dequantize_exact(*xq)


def moe_expert_mlp(x_hat, ids, w, experts, fmt, combine_scale=2.5, h_global_scale=None, q=quant):
    """Expert MLP on decoded activations.

    x_hat: [T, H] exactly decoded (float64) quantized activations (W4A16: the
    BF16 activations).  ids, w: [T, k] router output.  experts: mapping
    e -> NVFP4Expert (NVFP4, W4A16) / FP8Expert (only the experts that appear
    in ids are touched, each decoded once per projection pass).  fmt: "nvfp4",
    "fp8" or "w4a16".  q: quantizer module for h (``oracle.quant`` or the
    bit-identical ``oracle.quant_c``).
    Returns a dict with the stages in pair order p = t*k + j:
      g, u, h: [P, I] float32; hq: quantized h; y: [P, H] float32; out: [T, H].
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = ids.reshape(-1)
    tok = np.repeat(np.arange(T), k)
    P = T * k
    g = u = y = None
    rows_of = {int(e): np.nonzero(flat == e)[0] for e in np.unique(flat)}
    for e, rows in rows_of.items():
        wg, wu = experts[e].decoded_gate_up()
        xe = x_hat[tok[rows]]
        ge = gemm_f32(xe, wg)
        ue = gemm_f32(xe, wu)
        if g is None:
            I = wg.shape[0]
            g = np.zeros((P, I), np.float32)
            u = np.zeros((P, I), np.float32)
        g[rows] = ge
        u[rows] = ue
    h = swiglu_f32(g, u)
    if fmt == "nvfp4":
        hq = q.nvfp4_quantize(h, h_global_scale)
        h_hat = q.nvfp4_dequantize_exact(*hq)
    elif fmt == "w4a16":
        hq = None
        h_hat = formats.bf16_round(h).astype(np.float64)
    else:
        hq = q.fp8_quantize(h)
        h_hat = q.fp8_dequantize_exact(*hq)
    for e, rows in rows_of.items():
        ye = gemm_f32(h_hat[rows], experts[e].decoded_down())
        if y is None:
            y = np.zeros((P, ye.shape[1]), np.float32)
        y[rows] = ye
    out = combine_f32(y.reshape(T, k, -1), w, combine_scale)
    return {"g": g, "u": u, "h": h, "hq": hq, "y": y, "out": out}


def moe_layer(x, w_router, experts, fmt, n_group, topk_group, topk, combine_scale=2.5, q=quant):
    """One MoE layer: route -> quantize x -> expert MLP.  x: [T, H] float32-exact."""
    ids, w, scores, rstats = _route(x, w_router, n_group, topk_group, topk)
    xq, x_hat = quantize_activations(x, fmt, q=q)
    res = moe_expert_mlp(x_hat, ids, w, experts, fmt, combine_scale, q=q)
    res.update(ids=ids, w=w, scores=scores, xq=xq, route_stats=rstats)
    return res


# --------------------------------------------------------------------------
# RMSNorm and depth-scaled residual
# --------------------------------------------------------------------------


def rmsnorm_f32(x, eps=1e-6, gamma=None):
    """n = fl32(x * r) (times the gain: fl32(fl32(x * r) * gamma) when gamma is given)."""
    x64 = np.asarray(x, np.float32).astype(np.float64)
    ms = np.mean(x64 * x64, axis=1).astype(np.float32).astype(np.float64)
    r = (1.0 / np.sqrt(ms + eps)).astype(np.float32)
    n = (np.asarray(x, np.float32) * r[:, None]).astype(np.float32)
    if gamma is not None:
        n = (n * np.asarray(gamma, np.float32)[None, :]).astype(np.float32)
    return n


def residual_weights(k):
    """(a_k, b_k) = (fl32(sqrt((k-1)/k)), fl32(1/sqrt(k))) for residual step k >= 2."""
    return F32(np.sqrt((k - 1) / k)), F32(1.0 / np.sqrt(k))


def scaled_residual_f32(x, m, k):
    a, b = residual_weights(k)
    return (np.float64(a) * np.asarray(x, np.float64) + np.float64(b) * np.asarray(m, np.float64)).astype(np.float32)


def moe_stack(x1, layers, fmt, n_group, topk_group, topk, eps=1e-6, combine_scale=2.5, q=quant):
    """Stack of MoE layers on a float32 residual stream (embedding = step 1).

    layers: list of (w_router, experts).  Layer i (1-based) is residual step i+1.
    Returns the list of stream states [x1, x2, ...] and per-layer stage dicts.
    """
    xs = [np.asarray(x1, np.float32)]
    stages = []
    for i, (wr, experts) in enumerate(layers, start=1):
        n = rmsnorm_f32(xs[-1], eps)
        res = moe_layer(n, wr, experts, fmt, n_group, topk_group, topk, combine_scale, q=q)
        xs.append(scaled_residual_f32(xs[-1], res["out"], i + 1))
        res["normed"] = n
        stages.append(res)
    return xs, stages
