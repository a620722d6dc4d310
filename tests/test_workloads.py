"""Seeded input generators: determinism, shapes, dtypes, distributions."""

import hashlib

import numpy as np

import workloads as W


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


def test_host_generators_are_deterministic_and_bf16_exact():
    a = W.activations(W.TINY)
    b = W.activations(W.TINY)
    assert _h(a) == _h(b) and a.shape == (64, 256) and a.dtype == np.float32
    assert np.array_equal(W.to_bf16_f32(a), a)
    wr = W.router_weights(W.TINY)
    assert wr.shape == (16, 256) and not np.array_equal(W.to_bf16_f32(wr), wr)  # fp32 router weights
    g, u, d = W.expert_weights_host(W.TINY, 3)
    assert g.shape == (128, 256) and d.shape == (256, 128)
    assert abs(g.std() - 0.02) < 0.002 and abs(a.std() - 1) < 0.05
    g2, _, _ = W.expert_weights_host(W.TINY, 4)
    assert not np.array_equal(g, g2)


def test_prefill_router_skew_is_calibrated():
    c = W.router_row_scales(W.PREFILL)
    assert abs(c.max() - W.C_MAX) < 1e-12 and c.min() < 1e-6
    assert np.array_equal(W.router_row_scales(W.DECODE), np.ones(256))
    assert 2.0 < W.prefill_skew_gamma() < 5.0


def test_quant_tensor_host_has_outlier_rows():
    x = W.quant_tensor_host((1000, 64))
    rowmax = np.abs(x).max(1)
    assert (rowmax > 20).sum() >= 10
    assert np.array_equal(W.to_bf16_f32(x), x)
