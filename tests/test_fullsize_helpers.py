"""CPU checks of the full-size comparison helpers (tests/fullsize.py): the near-tie diagnostics.

A difference between two quantizations that comes from a tiny perturbation of h
must be reported as near-ties; a planted large change must not.
"""

import numpy as np

from oracle import quant_c as QC
from tests.fullsize import fp8_flips, nvfp4_flips


def _h(seed, shape=(2048, 512)):
    return (np.random.default_rng(seed).standard_normal(shape) * 0.3).astype(np.float32)


def test_nvfp4_flips_from_rounding_noise_are_near_ties():
    h = _h(1)
    h2 = (h * (1 + 3e-6 * np.random.default_rng(2).uniform(-1, 1, h.shape))).astype(np.float32)
    ns, nc, ok = nvfp4_flips(h, QC.nvfp4_quantize(h), QC.nvfp4_quantize(h2))
    assert ok and ns + nc > 0


def test_nvfp4_flips_catch_a_real_difference():
    h = _h(3)
    h2 = h.copy()
    h2[7, 5] *= np.float32(1.7)  # far from a midpoint change of one element
    q, q2 = QC.nvfp4_quantize(h), QC.nvfp4_quantize(h2)
    assert not np.array_equal(q[0], q2[0]) or not np.array_equal(q[1], q2[1])
    _, _, ok = nvfp4_flips(h, q, q2)
    assert not ok


def test_fp8_flips_from_rounding_noise_are_near_ties():
    h = _h(4)
    h2 = (h * (1 + 3e-6 * np.random.default_rng(5).uniform(-1, 1, h.shape))).astype(np.float32)
    _, nc, ok = fp8_flips(h, QC.fp8_quantize(h), QC.fp8_quantize(h2))
    assert ok and nc > 0


def test_fp8_flips_catch_a_real_difference():
    h = _h(6)
    h2 = h.copy()
    h2[3, 9] = h2[3, 9] * np.float32(1.3) + np.float32(0.01)
    _, nc, ok = fp8_flips(h, QC.fp8_quantize(h), QC.fp8_quantize(h2))
    assert nc > 0 and not ok
