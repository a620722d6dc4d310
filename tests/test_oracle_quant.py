"""Pins for the oracle's NVFP4 and FP8_DYNAMIC quantizers.

The pages fix: E2M1 elements, one E4M3 scale per 16 values, one global scale
per tensor (NVFP4 page, "Quantization scheme"); per-row E4M3 with division by
the scale and round-to-nearest (FP8 page, "Quantization scheme"/"method");
0.5625 byte per parameter and ~22 MB per 39.3 M-parameter expert (eurokommerz
page, "Drei Checkpoints und was sie speichern").  The tests below check those
facts and invariants that any correct implementation of the reading has.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import quant as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _rand(shape, seed, scale=1.0, outliers=0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_t(3, size=shape) * 0.5 * scale).astype(np.float32)
    if outliers:
        rows = rng.choice(shape[0], outliers, replace=False)
        x[rows] *= 50
    return _bf16(x)


def test_storage_closed_form_matches_pages():
    facts = {k: v["value"] for k, v in json.load(open(os.path.join(GOLDEN, "storage_facts.json"))).items()
             if not k.startswith("_")}
    x = _rand((32, 256), 0)
    codes, scales, sg = Q.nvfp4_quantize(x)
    bpp = (codes.nbytes + scales.nbytes) / x.size
    assert bpp == facts["bytes_per_param"]
    H, I = facts["hidden"], facts["intermediate"]
    params = 3 * H * I
    assert round(params / 1e6, 1) == facts["expert_params_millions"]
    assert round(params * bpp / 1e6) == facts["expert_bytes_mb"]
    total_params = facts["bf16_checkpoint_gib"] * 2 ** 30 / 2
    expert_params = facts["moe_layers"] * facts["experts_per_layer"] * params
    assert round(100 * expert_params / total_params, 1) == facts["expert_share_percent"]
    nvfp4_bytes = expert_params * bpp + (total_params - expert_params) * 2
    assert round(nvfp4_bytes / 1e9, 1) == facts["nvfp4_checkpoint_gb"]
    assert round(nvfp4_bytes / 2 ** 30) == facts["nvfp4_checkpoint_gib"]


def test_nvfp4_worked_block():
    # one block holding the whole E2M1 grid times 1/8, both signs
    grid = F.E2M1_MAGNITUDES
    blk = np.concatenate([grid, -grid]).astype(np.float32) / 8
    codes, scales, sg = Q.nvfp4_quantize(blk[None, :])
    assert sg == np.float32(np.float32(0.75) / np.float32(2688))
    assert scales[0, 0] == 0x7E  # block max maps to E4M3's 448
    q = Q.unpack_e2m1(codes)[0]
    assert list(q) == list(range(16))
    assert codes[0, 0] == (1 << 4) | 0  # element 0 low nibble, element 1 high nibble


def test_nvfp4_power_of_two_invariance():
    x = _rand((64, 128), 1, outliers=2)
    c0, s0, g0 = Q.nvfp4_quantize(x)
    for k in (-20, -3, 1, 7):
        c1, s1, g1 = Q.nvfp4_quantize(x * np.float32(2.0 ** k))
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
        assert g1 == g0 * np.float32(2.0 ** k)


def test_nvfp4_negation_flips_only_signs():
    x = _rand((16, 64), 2)
    c0, s0, g0 = Q.nvfp4_quantize(x)
    c1, s1, g1 = Q.nvfp4_quantize(-x)
    assert np.array_equal(s0, s1) and g0 == g1
    assert np.array_equal(Q.unpack_e2m1(c0) ^ 0x8, Q.unpack_e2m1(c1))


def test_nvfp4_block_max_encodes_as_six():
    x = _rand((256, 512), 3, outliers=3)
    codes, scales, sg = Q.nvfp4_quantize(x)
    q = Q.unpack_e2m1(codes).reshape(256, 32, 16)
    sb = F.e4m3_decode(scales)
    xb = x.reshape(256, 32, 16)
    arg = np.argmax(np.abs(xb), axis=-1)
    qmax = np.take_along_axis(q, arg[..., None], -1)[..., 0] & 7
    normal = sb >= 2.0 ** -6
    assert normal.sum() > 1000
    # a normal block scale is within 1/16 relative of a_b/(6 S_g): the max lands on 6
    assert np.all(qmax[normal] == 7)


def test_nvfp4_error_bound_and_dequantize():
    x = _rand((128, 256), 4, outliers=2)
    codes, scales, sg = Q.nvfp4_quantize(x)
    xe = Q.nvfp4_dequantize_exact(codes, scales, sg)
    q = Q.unpack_e2m1(codes).reshape(128, 16, 16)
    sb = F.e4m3_decode(scales)
    step = np.where((q & 7) >= 6, 2.0, np.where((q & 7) >= 4, 1.0, 0.5))  # grid spacing around the code
    bound = 0.5 * step * sb[..., None] * float(sg)
    err = np.abs(xe.reshape(128, 16, 16) - x.reshape(128, 16, 16))
    d2 = (sb * np.float32(sg)).astype(np.float32)
    r = np.abs(x.reshape(128, 16, 16)) / d2[..., None]
    unsat = r <= 6.0
    assert np.all(err[unsat] <= bound[unsat] * (1 + 1e-6) + 1e-30)
    xf = Q.nvfp4_dequantize_f32(codes, scales, sg)
    assert np.array_equal(xf, xe.astype(np.float32))


def test_nvfp4_zero_tensor_and_zero_blocks():
    x = np.zeros((4, 32), np.float32)
    x[1, 3] = -0.0
    codes, scales, sg = Q.nvfp4_quantize(x)
    assert sg == 0 and not scales.any() and not (Q.unpack_e2m1(codes) & 7).any()
    y = _rand((4, 32), 5)
    y[2, 16:] = 0
    y[2, 17] = -0.0
    c, s, g = Q.nvfp4_quantize(y)
    assert s[2, 1] == 0 and (Q.unpack_e2m1(c)[2, 17] == 0x8)


def test_nvfp4_static_global_scale():
    x = _rand((8, 64), 6)
    _, _, g = Q.nvfp4_quantize(x)
    c1, s1, g1 = Q.nvfp4_quantize(x, global_scale=g)
    c0, s0, _ = Q.nvfp4_quantize(x)
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1) and g1 == g
    # a too-small static scale saturates block scales at 448 and elements at 6
    c2, s2, _ = Q.nvfp4_quantize(x, global_scale=g / 64)
    assert np.all(s2 == 0x7E)


def test_nvfp4_single_block_recomputed_stepwise():
    """Recompute random blocks one element at a time with Python floats + float32 casts."""
    x = _rand((6, 48), 7, outliers=1)
    codes, scales, sg = Q.nvfp4_quantize(x)
    q = Q.unpack_e2m1(codes)
    f = np.float32
    amax = max(abs(float(v)) for v in x.ravel())
    S = f(f(amax) / f(2688.0))
    assert S == sg
    for r in range(6):
        for b in range(3):
            blk = x[r, 16 * b:16 * b + 16]
            ab = max(abs(float(v)) for v in blk)
            t = f(f(ab) / f(f(6.0) * S))
            sc = F.e4m3_encode_magnitude(t)
            assert sc == scales[r, b]
            d2 = f(f(F.e4m3_decode(sc)) * S)
            for i, v in enumerate(blk):
                ref = F.e2m1_encode(f(f(v) / d2), sign_src=f(v))
                assert ref == q[r, 16 * b + i]


def test_fp8_row_quantize():
    x = _rand((64, 320), 8, outliers=2)
    codes, s = Q.fp8_quantize(x)
    amax = np.abs(x).max(1)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    # the row maximum encodes as +-448
    arg = np.argmax(np.abs(x), axis=1)
    top = codes[np.arange(64), arg]
    assert np.all((top & 0x7F) == 0x7E)
    # elements: RNE of the IEEE float32 quotient (cross-checked with torch's E4M3 cast)
    r = (x / s[:, None]).astype(np.float32)
    ok = np.abs(r) < 464
    ref = torch.from_numpy(r[ok]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[ok], ref)
    # error bound: half an E4M3 ulp of the quotient times the scale
    xe = Q.fp8_dequantize_exact(codes, s)
    e = np.floor(np.log2(np.maximum(np.abs(r.astype(np.float64)), 2.0 ** -6)))
    ulp = 2.0 ** (e - 3)
    assert np.all(np.abs(xe - x) <= 0.5 * ulp * s[:, None] * (1 + 1e-6) + 1e-30)


def test_fp8_zero_row_and_power_of_two():
    x = _rand((4, 64), 9)
    x[1] = 0
    c, s = Q.fp8_quantize(x)
    assert s[1] == 0 and not (c[1] & 0x7F).any()
    c2, s2 = Q.fp8_quantize(x * np.float32(2.0 ** -9))
    assert np.array_equal(c, c2) and np.array_equal(s2, s * np.float32(2.0 ** -9))


def test_nvfp4_subnormal_block_scales():
    # one large element sets the global amax; the other blocks land in E4M3's
    # subnormal range (exponent field 0) and still round-trip within bounds
    rng = np.random.default_rng(10)
    x = _bf16(rng.standard_normal((64, 256)).astype(np.float32) * np.float32(1e-3))
    x[0, 0] = 100.0
    codes, scales, sg = Q.nvfp4_quantize(x)
    sub = (scales & 0x78) == 0
    assert sub.mean() > 0.5 and (scales[sub] != 0).any()
    _check_error_bound(x, codes, scales, sg)


def _check_error_bound(x, codes, scales, sg):
    R, C = x.shape
    xe = Q.nvfp4_dequantize_exact(codes, scales, sg).reshape(R, C // 16, 16)
    q = Q.unpack_e2m1(codes).reshape(R, C // 16, 16) & 7
    sb = F.e4m3_decode(scales)
    step = np.where(q >= 6, 2.0, np.where(q >= 4, 1.0, 0.5))
    bound = 0.5 * step * sb[..., None] * float(sg)
    xb = x.reshape(R, C // 16, 16)
    d2 = (sb * np.float32(sg)).astype(np.float32)
    unsat = (np.abs(xb) / d2[..., None]) <= 6.0
    err = np.abs(xe - xb)
    assert np.all(err[unsat] <= bound[unsat] * (1 + 1e-6) + 1e-30)
    # saturated elements sit at +-6 * s_b * S_g
    assert np.all(np.abs(xe[~unsat]) == 6.0 * (sb[..., None] * float(sg) * np.ones_like(xe))[~unsat])
