"""CPU checks of the full-size comparison helpers (tests/fullsize.py): the near-tie diagnostic.

Code differences that come from a perturbation of h at the FP32 accumulation
level must be reported as near-ties; a planted large change must not.
"""

import numpy as np
import pytest

from oracle import quant_c as QC
from tests.fullsize import TIE_TOL, code_flips


def _h(seed, shape=(2048, 512)):
    return (np.random.default_rng(seed).standard_normal(shape) * 0.3).astype(np.float32)


def _q(fmt, h):
    return QC.nvfp4_quantize(h) if fmt == "nvfp4" else QC.fp8_quantize(h)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_flips_from_rounding_noise_are_near_ties(fmt):
    h = _h(1)
    rms = np.sqrt(np.mean(h.astype(np.float64) ** 2, axis=1, keepdims=True))
    noise = np.random.default_rng(2).uniform(-1, 1, h.shape) * 3e-6 * rms
    h2 = (h + noise).astype(np.float32)
    ns, nc, worst = code_flips(fmt, h, h2, _q(fmt, h), _q(fmt, h2))
    assert nc > 0 and worst <= TIE_TOL


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_flips_catch_a_real_difference(fmt):
    h = _h(3)
    h2 = h.copy()
    h2[7, 5] = h2[7, 5] * np.float32(1.7) + np.float32(0.05)
    q, q2 = _q(fmt, h), _q(fmt, h2)
    _, nc, worst = code_flips(fmt, h, h2, q, q2)
    assert nc > 0 and worst > TIE_TOL
