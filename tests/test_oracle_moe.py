"""Pins for the oracle's expert MLP, combine, permutation, RMSNorm and residual.

Method ("Reflection releases Beam" news page): SwiGLU experts whose outputs
are mixed with the chosen scores renormalized to one, the total times 2.5
("Mixture-of-Experts details"); residual weights 1/sqrt(k) and sqrt((k-1)/k) whose squares sum to
one ("Residual stream and numerical decisions").
"""

import numpy as np
import pytest
import torch

from oracle import moe as M
from oracle import quant as Q


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _experts(E, H, I, seed, fmt="nvfp4"):
    rng = np.random.default_rng(seed)
    cls = M.FP8Expert if fmt == "fp8" else M.NVFP4Expert
    out = {}
    for e in range(E):
        wg = _bf16(rng.standard_normal((I, H)) * 0.02)
        wu = _bf16(rng.standard_normal((I, H)) * 0.02)
        wd = _bf16(rng.standard_normal((H, I)) * 0.02)
        out[e] = cls(wg, wu, wd)
    return out


def test_permute_is_stable_grouping():
    rng = np.random.default_rng(0)
    T, k, E = 50, 4, 12
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, row_of_pair, pair_of_row = M.permute(ids, E)
    # brute force: walk experts in order, pairs in order
    rows = []
    for e in range(E):
        rows += [p for p in range(T * k) if ids.reshape(-1)[p] == e]
    assert list(pair_of_row) == rows
    assert all(row_of_pair[p] == r for r, p in enumerate(rows))
    assert list(counts) == [int((ids == e).sum()) for e in range(E)]
    assert offsets[-1] == T * k and offsets[0] == 0


def test_exact_gemm_with_unit_scales():
    """All block scales 1 and S_g = 1: sums of E2M1 products are exact float32 multiples of 1/4."""
    rng = np.random.default_rng(1)
    T, H, N = 9, 64, 24
    qa = rng.integers(0, 16, size=(T, H)).astype(np.uint8)
    qb = rng.integers(0, 16, size=(N, H)).astype(np.uint8)
    pack = lambda q: (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    one = 0x38  # E4M3 code of 1.0
    sa = np.full((T, H // 16), one, np.uint8)
    sb = np.full((N, H // 16), one, np.uint8)
    a = Q.nvfp4_dequantize_exact(pack(qa), sa, np.float32(1))
    b = Q.nvfp4_dequantize_exact(pack(qb), sb, np.float32(1))
    got = M.gemm_f32(a, b)
    from oracle.formats import e2m1_decode
    va = (e2m1_decode(qa) * 4).astype(np.int64)  # integers
    vb = (e2m1_decode(qb) * 4).astype(np.int64)
    exact = (va @ vb.T)  # 16 * true value
    assert np.array_equal(got, (exact / 16.0).astype(np.float32))
    assert np.all(exact / 16.0 == got)  # representable exactly


def test_swiglu_reference_values():
    g = np.array([0.0, 1.0, -1.0, 20.0, -20.0, 3.5], np.float32)
    u = np.array([2.0, 2.0, 2.0, 1.0, 1.0, -0.5], np.float32)
    h = M.swiglu_f32(g, u)
    silu = g.astype(np.float64) / (1 + np.exp(-g.astype(np.float64)))
    assert h[0] == 0.0
    assert np.allclose(h, silu * u, rtol=1e-7, atol=0)
    assert abs(h[1] - 2 * 0.7310585786300049) < 1e-6


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8", "w4a16"])
def test_identical_experts_make_output_routing_independent(fmt):
    rng = np.random.default_rng(2)
    T, H, I, E, k = 16, 64, 32, 6, 3
    one = _experts(1, H, I, 3, fmt)[0]
    experts = {e: one for e in range(E)}
    x = _bf16(rng.standard_normal((T, H)))
    xq, xh = M.quantize_activations(x, fmt)
    ids_a = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    ids_b = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    w = (w / w.sum(1, keepdims=True)).astype(np.float32)
    ra = M.moe_expert_mlp(xh, ids_a, w, experts, fmt)
    rb = M.moe_expert_mlp(xh, ids_b, w, experts, fmt)
    assert np.array_equal(ra["out"], rb["out"])
    # out = 2.5 * expert(x) * sum(w); all k copies of y are equal
    y0 = ra["y"].reshape(T, k, H)[:, 0]
    ref = 2.5 * y0.astype(np.float64) * w.astype(np.float64).sum(1, keepdims=True)
    assert np.allclose(ra["out"], ref, rtol=1e-6, atol=1e-9)


def test_single_expert_matches_textbook_swiglu_mlp():
    """k = 1 with weight 1: out = 2.5 * W_d . Q(silu(W_g x) * (W_u x)), written with plain numpy."""
    rng = np.random.default_rng(4)
    T, H, I, E = 12, 64, 32, 4
    experts = _experts(E, H, I, 5)
    x = _bf16(rng.standard_normal((T, H)))
    xq, xh = M.quantize_activations(x, "nvfp4")
    ids = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    w = np.ones((T, 1), np.float32)
    res = M.moe_expert_mlp(xh, ids, w, experts, "nvfp4")
    # textbook: per token, its expert's dense MLP on decoded operands
    G = np.zeros((T, I)); U = np.zeros((T, I))
    for t in range(T):
        wg, wu, wd = experts[int(ids[t, 0])].decoded()
        G[t] = np.float32(wg @ xh[t])
        U[t] = np.float32(wu @ xh[t])
    h = (G / (1 + np.exp(-G)) * U).astype(np.float32)
    assert np.array_equal(h, res["h"])
    hc, hs, hg = Q.nvfp4_quantize(h)
    hh = Q.nvfp4_dequantize_exact(hc, hs, hg)
    out = np.zeros((T, H), np.float32)
    for t in range(T):
        wd = experts[int(ids[t, 0])].decoded()[2]
        out[t] = np.float32(2.5 * np.float32(wd @ hh[t]))
    assert np.array_equal(out, res["out"])


def test_residual_weights_and_zero_sublayer_stack():
    for k in range(2, 50):
        a, b = M.residual_weights(k)
        assert abs(float(a) ** 2 + float(b) ** 2 - 1) < 4e-7
    rng = np.random.default_rng(6)
    x1 = rng.standard_normal((4, 32)).astype(np.float32)
    x = x1
    for k in range(2, 6):
        x = M.scaled_residual_f32(x, np.zeros_like(x), k)
    # prod_k sqrt((k-1)/k) over k = 2..5 = sqrt(1/5)
    assert np.allclose(x, x1 * np.sqrt(1 / 5), rtol=4 * 2 ** -23)
    # equal contributions: stream after adding m at every step with m == x1 and x1 as embedding
    x = x1
    for k in range(2, 6):
        x = M.scaled_residual_f32(x, x1, k)
    assert np.allclose(x, x1 * np.sqrt(5), rtol=1e-6)


def _zero_experts(E, H, I, fmt):
    cls = M.FP8Expert if fmt == "fp8" else M.NVFP4Expert
    z = np.zeros((I, H), np.float32)
    ex = cls(z, z, np.zeros((H, I), np.float32))
    return {e: ex for e in range(E)}


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_stack_step_indices(fmt):
    """moe_stack: the embedding is residual step 1 and MoE layer i is step i + 1.

    With every expert zero, each layer only rescales the stream: x_(i+1) = fl32(a_(i+1) x_i), so after
    four layers x_5 = x_1 sqrt(1/5) up to four roundings.  With one non-zero layer j, its output m_j
    reaches the final stream with weight b_(j+1) * prod_(k > j+1) a_k = 1/sqrt(5), the embedding's
    weight too: x_5 = (x_1 + m_j) / sqrt(5).  A step index shifted by one breaks both (a_1 = 0 would
    zero the stream; weights 1/2 instead of 1/sqrt(5)).
    """
    rng = np.random.default_rng(31)
    T, H, I, E = 16, 64, 32, 8
    x1 = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    zero = (wr, _zero_experts(E, H, I, fmt))
    xs, stages = M.moe_stack(x1, [zero] * 4, fmt, 2, 1, 2)
    for i in range(1, 5):
        assert not stages[i - 1]["out"].any()
        a, _ = M.residual_weights(i + 1)
        assert np.array_equal(xs[i], (np.float64(a) * xs[i - 1].astype(np.float64)).astype(np.float32))
    assert np.allclose(xs[4], x1 * np.sqrt(1 / 5), rtol=5 * 2 ** -23, atol=0)
    # one non-zero layer (j = 2): identical experts, so m_2 does not depend on the routing
    r2 = np.random.default_rng(32)
    cls = M.FP8Expert if fmt == "fp8" else M.NVFP4Expert
    same = cls(_bf16(r2.standard_normal((I, H)) * 0.3), _bf16(r2.standard_normal((I, H)) * 0.3),
               _bf16(r2.standard_normal((H, I)) * 0.3))
    live = (wr, {e: same for e in range(E)})
    xs, stages = M.moe_stack(x1, [zero, live, zero, zero], fmt, 2, 1, 2)
    m2 = stages[1]["out"].astype(np.float64)
    assert np.abs(m2).max() > 0.1 * np.abs(x1).max()
    ref = (x1.astype(np.float64) + m2) / np.sqrt(5)
    assert np.allclose(xs[4], ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())


def test_rmsnorm_unit_rms():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((8, 5120)) * 3).astype(np.float32)
    n = M.rmsnorm_f32(x)
    rms = np.sqrt((n.astype(np.float64) ** 2).mean(1))
    assert np.allclose(rms, 1.0, atol=1e-6)
    assert np.array_equal(M.rmsnorm_f32(np.zeros((1, 16), np.float32)), np.zeros((1, 16), np.float32))


def test_layer_tiny_runs_and_is_deterministic():
    rng = np.random.default_rng(8)
    T, H, I, E = 32, 256, 128, 16
    experts = _experts(E, H, I, 9)
    x = _bf16(rng.standard_normal((T, H)))
    wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    r1 = M.moe_layer(x, wr, experts, "nvfp4", 4, 2, 2)
    r2 = M.moe_layer(x, wr, experts, "nvfp4", 4, 2, 2)
    assert np.array_equal(r1["out"], r2["out"])
    assert np.isfinite(r1["out"]).all() and np.abs(r1["out"]).max() > 0


def test_weight_only_single_expert_matches_textbook_mlp():
    """W4A16, k = 1, weight 1: out = 2.5 * W_d . bf16(silu(W_g x) * (W_u x)) on the raw BF16 x,
    written with plain numpy and torch's BF16 conversion."""
    import torch
    rng = np.random.default_rng(8)
    T, H, I, E = 10, 64, 32, 3
    experts = _experts(E, H, I, 9)
    x = _bf16(rng.standard_normal((T, H)))
    xq, xh = M.quantize_activations(x, "w4a16")
    assert xq is None and np.array_equal(xh, x.astype(np.float64))
    ids = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    w = np.ones((T, 1), np.float32)
    res = M.moe_expert_mlp(xh, ids, w, experts, "w4a16")
    out = np.zeros((T, H), np.float32)
    for t in range(T):
        wg, wu, wd = experts[int(ids[t, 0])].decoded()
        g = np.float64(np.float32(wg @ x[t].astype(np.float64)))
        u = np.float64(np.float32(wu @ x[t].astype(np.float64)))
        h = np.float32(g / (1 + np.exp(-g)) * u)
        hb = torch.from_numpy(h).to(torch.bfloat16).double().numpy()
        out[t] = np.float32(2.5 * np.float32(wd @ hb))
    assert np.array_equal(out, res["out"])
    assert res["hq"] is None


def test_weight_only_rejects_non_bf16_activations():
    x = np.float32([[1.0 + 2.0 ** -12, 1.0]])
    with pytest.raises(AssertionError):
        M.quantize_activations(x, "w4a16")
