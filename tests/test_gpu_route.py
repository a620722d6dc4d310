"""GPU parity: group-limited sigmoid router (ids, weights and scores bit-exact)."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import route as R
from tests.helpers import np_, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


def _run(gpu_lib, x, wr, G, kg, k, x_bf16=True, w_bf16=True):
    xt = to_dev_bf16(x) if x_bf16 else to_dev_f32(x)
    wt = to_dev_bf16(wr) if w_bf16 else to_dev_f32(wr)
    ids, wts, scores, ws = gpu_lib.route(xt, wt, G, kg, k, return_scores=True, return_workspace=True)
    diag = gpu_lib.route_diagnostics(ws, x.shape[0], x.shape[1], wr.shape[0])
    torch.cuda.synchronize()
    return np_(ids), np_(wts), np_(scores), np_(diag)


def _check(gpu, x, wr, G, kg, k):
    ids, wts, scores, diag = gpu
    oi, ow, os_, st = R.route(x, wr, G, kg, k)
    assert np.array_equal(scores.view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(ids, oi)
    assert np.array_equal(wts.view(np.uint32), ow.view(np.uint32))
    return diag, st


def test_route_tiny_fp32_router(gpu_lib):
    cfg = W.TINY
    x, wr = W.activations(cfg), W.router_weights(cfg)
    _check(_run(gpu_lib, x, wr, cfg.n_group, cfg.topk_group, cfg.topk, w_bf16=False), x, wr, 4, 2, 2)


def test_route_decode_shape(gpu_lib):
    cfg = W.DECODE
    x, wr = W.activations(cfg), W.router_weights(cfg)
    diag, st = _check(_run(gpu_lib, x, wr, 8, 4, 8), x, wr, 8, 4, 8)


def test_route_prefill_shape_full(gpu_lib):
    cfg = W.PREFILL
    x, wr = W.activations(cfg), W.router_weights(cfg)
    diag, st = _check(_run(gpu_lib, x, wr, 8, 4, 8), x, wr, 8, 4, 8)
    print("route prefill diag", diag, "oracle refinements", st["logits_refined"], st["sigmoid_refined"])


def test_route_fp32_stream_input(gpu_lib):
    # the stacked layers route an FP32 residual-stream input with bf16 router weights
    rng = np.random.default_rng(11)
    x = rng.standard_normal((300, 5120)).astype(np.float32)
    wr = W.router_weights(W.DECODE)
    _check(_run(gpu_lib, x, wr, 8, 4, 8, x_bf16=False), x, wr, 8, 4, 8)


def test_route_ties_and_saturation(gpu_lib):
    rng = np.random.default_rng(12)
    H, E = 256, 64
    x = W.to_bf16_f32(rng.standard_normal((96, H)).astype(np.float32))
    wr = W.to_bf16_f32((rng.standard_normal((E, H)) * 0.05).astype(np.float32))
    wr[10] = wr[3]            # identical logits -> exact score ties, lower index must win
    wr[40] = wr[33]
    wr[50:54] = wr[50] * 64   # large logits -> sigmoid saturates to 1.0f (ties at 1.0)
    x[5] = 0.0                # all-zero token: every score 0.5
    _check(_run(gpu_lib, x, wr, 8, 4, 8), x, wr, 8, 4, 8)
    _check(_run(gpu_lib, x, wr, 8, 8, 8), x, wr, 8, 8, 8)  # all groups kept == plain top-k
    _check(_run(gpu_lib, x, wr, 4, 1, 3), x, wr, 4, 1, 3)


def test_route_exact_fallback_paths(gpu_lib):
    """Cancelling dot products and float32-midpoint logits go through the exact superaccumulator."""
    rng = np.random.default_rng(13)
    T, H, E = 64, 512, 16
    x = rng.standard_normal((T, H)).astype(np.float32)
    w = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    x[:, 0] = 2.0 ** 20
    x[:, 1] = -(2.0 ** 20)
    w[:, 0] = 1.0
    w[:, 1] = 1.0  # the two large terms cancel exactly; the binary64 bound is wide
    x[3, :] = 0.0
    x[3, :2] = [1.0, 2.0 ** -24]
    # products spanning more than 120 bits (2^30 against about 2^-125): past the
    # fixed-point window, into the superaccumulator
    x[5, 0] = 2.0 ** 30
    x[5, 1] = -(2.0 ** 30)
    x[5, 2] = 2.0 ** -120
    ids, wts, scores, diag = _run(gpu_lib, x, w, 4, 2, 4, x_bf16=False, w_bf16=False)
    _check((ids, wts, scores, diag), x, w, 4, 2, 4)
    assert diag[0] > 0  # the fallback ran


@pytest.mark.parametrize("T,H,E,x_bf16", [(1000, 200, 520, False), (4100, 256, 200, True)])
def test_route_tiled_ragged_with_fallbacks(gpu_lib, T, H, E, x_bf16):
    """At least 128 tiles of 64 x 64 select the tiled logits kernel: ragged token and expert tiles, H with
    (256) and without (200) whole K steps of 32, and cancelling rows that need the exact recomputation."""
    rng = np.random.default_rng(T + H)
    x = rng.standard_normal((T, H)).astype(np.float32)
    w = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    if x_bf16:
        x = W.to_bf16_f32(x)
    w = W.to_bf16_f32(w)
    rows = np.arange(7, T, 97)
    x[rows, 0] = 2.0 ** 20
    x[rows, 1] = -(2.0 ** 20)
    w[:, 0] = 1.0
    w[:, 1] = 1.0
    ids, wts, scores, diag = _run(gpu_lib, x, w, 8, 4, 8, x_bf16=x_bf16)
    _check((ids, wts, scores, diag), x, w, 8, 4, 8)
    assert diag[0] > 0  # the tiled kernel's exact fallback ran


@pytest.mark.parametrize("G,kg,k", [(8, 4, 8), (1, 1, 32), (2, 1, 5), (16, 3, 8), (32, 32, 32), (64, 2, 8)])
def test_route_256_experts_group_sizes(gpu_lib, G, kg, k):
    """256 experts take the one-wave-per-token selection: groups of 4 to 256 experts (1 to 64 lanes), a ragged
    last workgroup of tokens, equal logits in different groups, saturated scores and an all-zero token whose
    group sums all tie."""
    rng = np.random.default_rng(14 + G)
    T, H, E = 37, 256, 256
    x = W.to_bf16_f32(rng.standard_normal((T, H)).astype(np.float32))
    wr = W.to_bf16_f32((rng.standard_normal((E, H)) * 0.05).astype(np.float32))
    wr[200] = wr[7]
    wr[131] = wr[129]
    wr[64:68] = wr[64] * 64
    x[5] = 0.0
    _check(_run(gpu_lib, x, wr, G, kg, k), x, wr, G, kg, k)


@pytest.mark.parametrize("T,E,H", [(2050, 256, 272), (2050, 256, 1024), (37, 64, 528), (64, 256, 2048)])
def test_route_int8_digit_path_edges(gpu_lib, T, E, H):
    """bf16 x and w take the int8 digit path (at least 128 tiles of 64 x 64: one pass over K; fewer: K cut into
    splits whose exact partials are added afterwards): H with a zero-padded last chunk (272, 528) and without,
    ragged token and expert tiles, all-zero token and expert rows, bf16 subnormals, rows below 2^-100 (digits from
    the integer fields) and near 2^100, rows whose values span more than the 30-bit digit window (truncation residuals: the rounding proven by the bound or the logit recomputed
    exactly) and cancelling rows."""
    rng = np.random.default_rng(H)
    x = W.to_bf16_f32(rng.standard_normal((T, H)).astype(np.float32))
    w = W.to_bf16_f32((rng.standard_normal((E, H)) * 0.05).astype(np.float32))
    x[3] = 0.0
    w[17] = 0.0
    x[9, :40] = W.to_bf16_f32(rng.standard_normal(40).astype(np.float32) * np.float32(2.0 ** -130))  # subnormal
    x[11, 5] = 2.0 ** 12           # one large value: most of the row falls below the window
    x[13, 7] = 2.0 ** -40          # one value below the window of an otherwise ordinary row
    w[30, 0] = 2.0 ** 9
    w[41, 2] = 2.0 ** -50
    x[15] = W.to_bf16_f32(rng.standard_normal(H).astype(np.float32) * np.float32(2.0 ** -118))  # integer digits
    w[43] = W.to_bf16_f32(rng.standard_normal(H).astype(np.float32) * np.float32(2.0 ** -110))
    x[17] = W.to_bf16_f32(rng.standard_normal(H).astype(np.float32) * np.float32(2.0 ** 100))   # huge logits
    rows = np.arange(20, T, 211)
    x[rows, 0] = 2.0 ** 20
    x[rows, 1] = -(2.0 ** 20)
    w[:, 0] = w[:, 1] = 1.0
    w[30, 0] = 2.0 ** 9
    ids, wts, scores, diag = _run(gpu_lib, x, w, 8, 4, 8)
    _check((ids, wts, scores, diag), x, w, 8, 4, 8)
    assert diag[0] > 0  # cancelling rows: their logits were recomputed exactly
