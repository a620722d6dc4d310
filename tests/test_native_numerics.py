"""The HIP library's scalar numerics (bsm_numerics.h, compiled for the host) against the oracle.

These are the encoders and exact-rounding routines the gfx950 kernels run; a
g++ build of the same header lets the CPU suite check them without a GPU.
"""

import ctypes
import os

import numpy as np
import pytest

from oracle import formats as F
from oracle import route as R

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def hc():
    path = os.path.join(HERE, "native", "libbsm_host_checks.so")
    if not os.path.exists(path):
        from tests.native.build_host_checks import build
        build()
    lib = ctypes.CDLL(path)
    P = np.ctypeslib.ndpointer
    lib.hc_e4m3_code.argtypes = [P(np.float32), ctypes.c_int64, P(np.uint8)]
    lib.hc_e2m1_code.argtypes = [P(np.float32), ctypes.c_int64, P(np.uint8)]
    lib.hc_e4m3_value.argtypes = [P(np.uint8), ctypes.c_int64, P(np.float32)]
    lib.hc_e2m1_value.argtypes = [P(np.uint8), ctypes.c_int64, P(np.float32)]
    lib.hc_exact_dot.argtypes = [P(np.float32), P(np.float32), ctypes.c_int64, ctypes.c_int64, P(np.float32)]
    lib.hc_window_dot.argtypes = [P(np.float32), P(np.float32), ctypes.c_int64, ctypes.c_int64, P(np.float32),
                                  P(np.int32)]
    lib.hc_sigmoid.argtypes = [P(np.float32), ctypes.c_int64, P(np.float32), P(np.int32)]
    lib.hc_sigmoid_dd.argtypes = [P(np.float32), ctypes.c_int64, P(np.float32)]
    lib.hc_lsb_exp.argtypes = [ctypes.c_float]
    lib.hc_lsb_exp.restype = ctypes.c_int
    return lib


def _probe(table, rng, n):
    t = np.asarray(table, np.float64)
    mids = ((t[1:] + t[:-1]) / 2).astype(np.float32)
    parts = [mids, np.nextafter(mids, np.float32(1e30)), np.nextafter(mids, np.float32(0)), t.astype(np.float32),
             rng.uniform(0, float(t[-1]) * 1.3, n).astype(np.float32),
             (rng.uniform(0, 1, n) * 2.0 ** rng.integers(-40, 10, n)).astype(np.float32),
             np.float32([0.0, np.inf, 1e30, 2.0 ** -149, 2.0 ** -126])]
    return np.concatenate(parts).astype(np.float32)


def test_e4m3_encoder_matches_oracle(hc):
    rng = np.random.default_rng(0)
    a = _probe(F.E4M3_MAGNITUDES, rng, 200000)
    out = np.empty(a.size, np.uint8)
    hc.hc_e4m3_code(a, a.size, out)
    assert np.array_equal(out, F.e4m3_encode_magnitude(a))
    codes = np.arange(127, dtype=np.uint8)
    v = np.empty(127, np.float32)
    hc.hc_e4m3_value(codes, 127, v)
    assert np.array_equal(v, F.E4M3_MAGNITUDES.astype(np.float32))


def test_e2m1_encoder_matches_oracle(hc):
    rng = np.random.default_rng(1)
    a = _probe(F.E2M1_MAGNITUDES, rng, 200000)
    a = np.concatenate([a, np.float32([np.nan])])
    out = np.empty(a.size, np.uint8)
    hc.hc_e2m1_code(a, a.size, out)
    assert np.array_equal(out, F.e2m1_encode_magnitude(a))
    codes = np.arange(8, dtype=np.uint8)
    v = np.empty(8, np.float32)
    hc.hc_e2m1_value(codes, 8, v)
    assert np.array_equal(v, F.E2M1_MAGNITUDES.astype(np.float32))


def test_superaccumulator_exact_dot(hc):
    rng = np.random.default_rng(2)
    rows, n = 300, 512
    x = rng.standard_normal((rows, n)).astype(np.float32)
    w = (rng.standard_normal((rows, n)) * 0.05).astype(np.float32)
    # adversarial rows: huge cancellation, ties at float32 midpoints, tiny and subnormal products
    x[0, :3] = [2.0 ** 30, 1.0, -2.0 ** 30]
    w[0, :3] = [1.0, 2.0 ** -40, 1.0]
    x[0, 3:] = 0
    x[1, :2] = [1.0, 2.0 ** -24]
    w[1, :2] = [1.0, 1.0]
    x[1, 2:] = 0
    x[2] = np.float32(2.0 ** -120)
    w[2] = np.float32(2.0 ** -100)
    x[3] = -x[4]
    w[3] = w[4]
    x[5, :] = np.float32(3e38) * np.sign(rng.standard_normal(n)).astype(np.float32)
    w[5, :] = np.float32(1e-38)
    out = np.empty(rows, np.float32)
    hc.hc_exact_dot(x, w, rows, n, out)
    ref = np.array([R.logits_exact_f32(x[r:r + 1], w[r:r + 1])[0][0, 0] for r in range(rows)], np.float32)
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    assert out[0] == np.float32(2.0 ** -40) and out[1] == 1.0


def test_window_exact_dot(hc):
    rng = np.random.default_rng(21)
    rows, n = 400, 640
    x = W_bf16(rng.standard_normal((rows, n)))
    w = W_bf16(rng.standard_normal((rows, n)) * 0.05)
    # exact ties, cancellation, carries across digit boundaries, negative totals, zero rows
    x[0, :2] = [1.0, 2.0 ** -24]
    w[0, :2] = [1.0, 1.0]
    x[0, 2:] = 0
    x[1] = -x[2]
    w[1] = w[2]
    x[3, :] = 0
    x[4, ::2] = 3.0
    x[4, 1::2] = -3.0
    w[4, :] = 0.5
    x[5, 0] = 1.0
    w[5, 0] = 1.0
    x[5, 1:] = 2.0 ** -40
    w[5, 1:] = -1.0
    xf = rng.standard_normal((rows, n)).astype(np.float32)  # full binary32 inputs too
    for xa, wa in ((x, w), (xf, w)):
        out = np.empty(rows, np.float32)
        ok = np.empty(rows, np.int32)
        hc.hc_window_dot(np.ascontiguousarray(xa), np.ascontiguousarray(wa), rows, n, out, ok)
        ref = np.array([R.logits_exact_f32(xa[r:r + 1], wa[r:r + 1])[0][0, 0] for r in range(rows)], np.float32)
        assert ok.all()
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    # a product 2^-130 below the largest falls outside the window and is reported
    x2 = np.zeros((1, 4), np.float32)
    w2 = np.zeros((1, 4), np.float32)
    x2[0, :2] = [1.0, 2.0 ** -70]
    w2[0, :2] = [1.0, 2.0 ** -70]
    out = np.empty(1, np.float32)
    ok = np.empty(1, np.int32)
    hc.hc_window_dot(x2, w2, 1, 4, out, ok)
    assert ok[0] == 0


def W_bf16(a):
    import torch
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def test_sigmoid_fast_path_and_dd_path_match_oracle(hc):
    rng = np.random.default_rng(3)
    l = np.concatenate([rng.standard_normal(200000) * 4, rng.uniform(-110, 30, 100000),
                        np.float32([0, -0.0, 16, 17, 17.33, 17.4, 88, -87, -103, -104, -200, 800, -800])]).astype(np.float32)
    ref, _ = R.sigmoid_exact_f32(l)
    out = np.empty(l.size, np.float32)
    fast = np.empty(l.size, np.int32)
    hc.hc_sigmoid(l, l.size, out, fast)
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    # the double-double path alone must also be exactly rounded
    sub = l[(l > -100) & (l < 25)][:20000]
    dd = np.empty(sub.size, np.float32)
    hc.hc_sigmoid_dd(sub, sub.size, dd)
    ref2, _ = R.sigmoid_exact_f32(sub)
    assert np.array_equal(dd.view(np.uint32), ref2.view(np.uint32))


def test_lsb_exponent(hc):
    assert hc.hc_lsb_exp(1.0) == 0
    assert hc.hc_lsb_exp(1.5) == -1
    assert hc.hc_lsb_exp(2.0 ** -149) == -149
    assert hc.hc_lsb_exp(3.0 * 2.0 ** -140) == -140
    assert hc.hc_lsb_exp(-6.0) == 1


def test_exact_dot_nonfinite_inputs_stay_in_range(hc):
    # non-finite inputs give unspecified logits; the accumulators must not index out of range
    x = np.ones((3, 64), np.float32)
    w = np.ones((3, 64), np.float32)
    x[0, 5] = np.inf
    x[1, 7] = np.nan
    w[2, 0] = -np.inf
    out = np.empty(3, np.float32)
    ok = np.empty(3, np.int32)
    hc.hc_exact_dot(x, w, 3, 64, out)
    hc.hc_window_dot(x, w, 3, 64, out, ok)


def test_e2m1_thresholds_equal_the_divided_encoding(hc):
    """The gfx950 encoder's division-free E2M1 codes: a compared with e2m1_threshold(d2, i) must give the
    oracle's code of the correctly rounded float32 quotient a / d2, for every block-scale value times
    global scales across the range (subnormal, tiny and huge d2) and at every rounding midpoint of the
    quotient, its float32 neighbours and random values."""
    hc.hc_e2m1_code_thr.argtypes = [np.ctypeslib.ndpointer(np.float32), np.ctypeslib.ndpointer(np.float32),
                                    ctypes.c_int64, np.ctypeslib.ndpointer(np.uint8)]
    rng = np.random.default_rng(7)
    sv = F.E4M3_MAGNITUDES[1:].astype(np.float32)
    gs = np.float32([1.0, 1.0 / 6.0, 2.0 ** -20, 3.7e-3, 1.234567e-5, 2.0 ** -130, 1e-38, 5e30,
                     3.4028235e38 / 448.0, *rng.uniform(1e-6, 1.0, 12)])
    d2 = (sv[None, :] * gs[:, None]).astype(np.float32).ravel()
    d2 = d2[(d2 > 0) & np.isfinite(d2)]
    mids = np.float64([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    a_list, d_list = [], []
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        for d in d2:
            b = (mids * np.float64(d)).astype(np.float32)  # the E2M1 decision points times d2, then +-2 ulps
            near, up, lo = [b], b, b
            for _ in range(2):
                up, lo = np.nextafter(up, np.float32(np.inf)), np.nextafter(lo, np.float32(0))
                near += [up, lo]
            near.append(np.float32(rng.uniform(0, 7, 8) * d))
            near.append(np.float32([0.0, np.inf, np.nan, 3.4028235e38, 2.0 ** -149]))
            a = np.concatenate(near).astype(np.float32)
            a_list.append(a)
            d_list.append(np.full(a.size, d, np.float32))
        a = np.concatenate(a_list)
        dd = np.concatenate(d_list)
        expect = F.e2m1_encode_magnitude((a / dd).astype(np.float32))
    out = np.empty(a.size, np.uint8)
    hc.hc_e2m1_code_thr(a, dd, a.size, out)
    bad = np.nonzero(out != expect)[0]
    assert bad.size == 0, [(float(a[i]), float(dd[i]), int(out[i]), int(expect[i])) for i in bad[:8]]
