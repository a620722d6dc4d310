"""Pins of the dense FP8 linear / MLP oracle against closed forms."""

import numpy as np

from oracle import linear as L
from oracle import moe as M
from oracle import quant as Q


def test_linear_exact_with_power_of_two_scales():
    # rows whose absolute maxima are 448 * 2^j give power-of-two scales; integer entries <= 16
    # are exact E4M3 values, so every product sum is an exact small integer times a power of two
    rng = np.random.default_rng(0)
    T, K, N = 5, 256, 24
    x = rng.integers(-16, 17, (T, K)).astype(np.float32)
    w = rng.integers(-16, 17, (N, K)).astype(np.float32)
    x[:, 0] = 448.0 * 2.0 ** rng.integers(-3, 3, T)
    w[:, 0] = 448.0 * 2.0 ** rng.integers(-3, 3, N)
    xq, wq, y = L.fp8_linear(x, w)
    assert np.all(np.log2(xq[1]) == np.round(np.log2(xq[1])))
    assert np.array_equal(Q.fp8_dequantize_exact(*xq), x.astype(np.float64))
    ref = (x.astype(np.int64) @ w.astype(np.int64).T).astype(np.float64)  # exact integers
    assert np.array_equal(y, ref.astype(np.float32))


def test_linear_one_hot_weight_row_selects_a_column():
    rng = np.random.default_rng(1)
    T, K = 7, 64
    x = rng.standard_normal((T, K)).astype(np.float32)
    w = np.zeros((3, K), np.float32)
    w[0, 5] = 448.0      # row scale 1: decoded weight 448 exactly
    w[1, 17] = -896.0    # row scale 2
    w[2, 63] = 224.0     # row scale 1/2
    xq, wq, y = L.fp8_linear(x, w)
    assert list(wq[1]) == [1.0, 2.0, 0.5]
    xh = Q.fp8_dequantize_exact(*xq)
    assert np.array_equal(y[:, 0], (448.0 * xh[:, 5]).astype(np.float32))
    assert np.array_equal(y[:, 1], (-896.0 * xh[:, 17]).astype(np.float32))
    assert np.array_equal(y[:, 2], (224.0 * xh[:, 63]).astype(np.float32))


def test_dense_mlp_is_the_one_expert_moe_with_unit_weight():
    rng = np.random.default_rng(2)
    T, H, I = 6, 64, 32
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg, wu, wd = (rng.standard_normal(s).astype(np.float32) * 0.05 for s in ((I, H), (I, H), (H, I)))
    res = L.fp8_dense_mlp(x, wg, wu, wd)
    # textbook: g, u, h, per-row FP8 h, down projection, no combine weighting
    xh = Q.fp8_dequantize_exact(*Q.fp8_quantize(x))
    gq, uq, dq = (Q.fp8_dequantize_exact(*Q.fp8_quantize(m)) for m in (wg, wu, wd))
    g = (xh @ gq.T).astype(np.float32).astype(np.float64)
    u = (xh @ uq.T).astype(np.float32).astype(np.float64)
    h = (g / (1 + np.exp(-g)) * u).astype(np.float32)
    assert np.array_equal(h, res["h"])
    hh = Q.fp8_dequantize_exact(*Q.fp8_quantize(h))
    assert np.array_equal((hh @ dq.T).astype(np.float32), res["out"])
