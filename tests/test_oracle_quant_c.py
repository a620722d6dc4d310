"""Pins for the oracle's C quantizers (oracle/quant_c.c): bit-identical to oracle/quant.py.

oracle/quant.py is the readable definition, pinned in test_oracle_quant.py to
the formats' value tables, brute force and invariants.  The C loops exist only
so that full-size Beam tensors can be quantized quickly; here they must return
exactly the same codes, scales and global scales as the NumPy code on inputs
chosen to reach every branch: random and heavy-tailed values, every E2M1 and
E4M3 rounding midpoint and its float32 neighbours, zero tensors, blocks and
rows, signed zeros, float32 subnormals (block scales that underflow), static
global scales that saturate, bf16 inputs given as bit patterns.
"""

import numpy as np
import pytest

from oracle import formats as F
from oracle import quant as Q
from oracle import quant_c as QC


def _same_nvfp4(x, gs=None):
    a = Q.nvfp4_quantize(x, gs)
    b = QC.nvfp4_quantize(x, gs)
    assert np.array_equal(a[0], b[0]), "codes differ"
    assert np.array_equal(a[1], b[1]), "scales differ"
    assert a[2].view(np.uint32) == b[2].view(np.uint32), "global scale differs"
    assert np.array_equal(Q.nvfp4_dequantize_exact(*a), QC.nvfp4_dequantize_exact(*b))
    return b


def _same_fp8(x):
    a = Q.fp8_quantize(x)
    b = QC.fp8_quantize(x)
    assert np.array_equal(a[0], b[0]), "codes differ"
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32)), "scales differ"
    assert np.array_equal(Q.fp8_dequantize_exact(*a), QC.fp8_dequantize_exact(*b))
    return b


def _neighbours(v):
    """v and its float32 neighbours below and above."""
    v = np.asarray(v, np.float32)
    return np.concatenate([np.nextafter(v, np.float32(-np.inf)), v, np.nextafter(v, np.float32(np.inf))])


@pytest.mark.parametrize("shape,std", [((64, 256), 1.0), ((33, 48), 0.02), ((1, 16), 3.0), ((7, 5120), 1e-3)])
def test_nvfp4_random(shape, std):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(shape) * std).astype(np.float32)
    _same_nvfp4(x)
    _same_nvfp4(F.bf16_round(x))


def test_nvfp4_heavy_tail_and_subnormal_scales():
    x = (np.random.default_rng(12).standard_t(3, size=(96, 512)) * 0.5).astype(np.float32)
    x[::10] *= np.float32(50.0)  # outlier rows push many block scales into E4M3 subnormals
    _same_nvfp4(x)


def test_nvfp4_every_e2m1_midpoint():
    # static S_g = 1 and a block maximum of 6 give s_b = 1, so each element is encoded as itself
    mids = (F.E2M1_MAGNITUDES[:-1] + F.E2M1_MAGNITUDES[1:]) / 2
    vals = np.concatenate([_neighbours(mids), _neighbours(F.E2M1_MAGNITUDES), [6.5, 7.0, 1e30]]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    n = int(np.ceil(len(vals) / 15))
    blocks = np.zeros((n, 16), np.float32)
    flat = np.zeros(n * 15, np.float32)
    flat[:len(vals)] = vals
    blocks[:, 1:] = flat.reshape(n, 15)
    blocks[:, 0] = 6.0
    x = blocks.reshape(1, -1)
    _same_nvfp4(x, np.float32(1.0))


def test_nvfp4_every_e4m3_scale_midpoint():
    # static S_g = fl32(1/6) makes fl32(6 S_g) = 1, so a block scale encodes the block maximum itself
    gs = np.float32(1.0 / 6.0)
    assert np.float32(np.float32(6.0) * gs) == np.float32(1.0)
    tab = F.E4M3_MAGNITUDES
    mids = (tab[:-1] + tab[1:]) / 2
    amax = np.concatenate([_neighbours(mids[1:]), _neighbours(tab[1:]), [500.0, 1e6]]).astype(np.float32)
    x = np.zeros((len(amax), 16), np.float32)
    x[:, 3] = amax
    x[:, 7] = -amax / np.float32(3.0)
    _same_nvfp4(x, gs)


def test_nvfp4_zeros_signs_and_underflow():
    _same_nvfp4(np.zeros((4, 64), np.float32))
    _same_nvfp4(-np.zeros((2, 32), np.float32))
    x = np.random.default_rng(13).standard_normal((8, 64)).astype(np.float32)
    x[2] = 0.0
    x[3, :16] = -0.0
    _same_nvfp4(x)
    # float32 subnormal inputs: s_b * S_g underflows to 0 for the small blocks (quotients inf or NaN)
    tiny = (np.random.default_rng(14).standard_normal((6, 64)) * 1e-39).astype(np.float32)
    tiny[0, 0] = np.float32(3e-38)
    _same_nvfp4(tiny)
    # a static global scale far too small: every quotient saturates
    _same_nvfp4(x, np.float32(1e-6))


@pytest.mark.parametrize("shape,std", [((64, 256), 1.0), ((5, 37), 0.02), ((1, 4), 5.0), ((3, 5120), 1e-3)])
def test_fp8_random(shape, std):
    rng = np.random.default_rng(21)
    x = (rng.standard_normal(shape) * std).astype(np.float32)
    _same_fp8(x)
    _same_fp8(F.bf16_round(x))


def test_fp8_every_e4m3_midpoint():
    # a row maximum of 448 gives s = 1, so every element is encoded as itself
    tab = F.E4M3_MAGNITUDES
    mids = (tab[:-1] + tab[1:]) / 2
    vals = np.concatenate([_neighbours(mids), _neighbours(tab), [447.9, 448.0]]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    x = np.concatenate([[448.0], vals]).astype(np.float32)[None]
    _same_fp8(x)


def test_fp8_zeros_signs_and_tiny_rows():
    x = np.random.default_rng(22).standard_normal((6, 40)).astype(np.float32)
    x[1] = 0.0
    x[2] = -0.0
    x[4] *= np.float32(1e-40)
    _same_fp8(x)


def test_bf16_bit_patterns():
    x = F.bf16_round(np.random.default_rng(23).standard_normal((16, 128)).astype(np.float32))
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    a, b = QC.nvfp4_quantize(x), QC.nvfp4_quantize(bits)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
    a, b = QC.fp8_quantize(x), QC.fp8_quantize(bits)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
