"""Pins for the oracle's element codecs (E2M1, OCP E4M3FN) and exact-rounding helpers."""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _grid():
    out = {}
    for line in open(os.path.join(GOLDEN, "e2m1_grid.txt")):
        line = line.split("#")[0].strip()
        if line:
            c, v = line.split()
            out[int(c, 16)] = float(v)
    return out


def test_e2m1_decode_matches_format_grid():
    grid = _grid()
    assert len(grid) == 16
    dec = F.e2m1_decode(np.arange(16))
    for c, v in grid.items():
        assert dec[c] == v and np.signbit(dec[c]) == np.signbit(v), c


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    dec = F.e4m3_decode(codes)
    both_nan = np.isnan(ref) & np.isnan(dec)
    assert np.array_equal(both_nan, np.isnan(ref))
    assert np.array_equal(dec[~both_nan], ref[~both_nan])
    assert F.E4M3_MAX == 448.0 and F.e4m3_decode(1) == 2.0 ** -9 and F.e4m3_decode(8) == 2.0 ** -6


def _brute_nearest(a, table):
    """argmin_i |a - table[i]| with exact rationals; ties -> even index."""
    out = []
    for v in a:
        fv = Fraction(float(v))
        d = [abs(fv - Fraction(float(t))) for t in table]
        m = min(d)
        idx = [i for i, di in enumerate(d) if di == m]
        even = [i for i in idx if i % 2 == 0]
        out.append(even[0] if even else idx[0])
    return np.array(out)


def _probe_values(table, rng, n_random):
    """Every midpoint of the table and its float32 neighbours, the grid itself, and random values."""
    t = np.asarray(table, np.float64)
    mids = ((t[1:] + t[:-1]) / 2).astype(np.float32)
    pts = [mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf)),
           t.astype(np.float32), np.nextafter(t.astype(np.float32), np.float32(np.inf))]
    hi = float(t[-1]) * 1.5
    pts.append(rng.uniform(0, hi, n_random).astype(np.float32))
    pts.append(np.float32([hi, 1e30, 3.4e38]))
    return np.concatenate(pts).astype(np.float32)


def test_e2m1_encode_is_nearest_ties_even_saturating():
    rng = np.random.default_rng(1)
    a = _probe_values(F.E2M1_MAGNITUDES, rng, 4000)
    got = F.e2m1_encode_magnitude(a)
    exp = _brute_nearest(a, F.E2M1_MAGNITUDES)
    assert np.array_equal(got, exp)
    # thresholds of the round-to-nearest-even grid
    cases = {0.25: 0, 0.2500001: 1, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 5.0000005: 7, 1e9: 7}
    for v, c in cases.items():
        assert F.e2m1_encode_magnitude(np.float32(v)) == c, v


def test_e2m1_encode_sign_bit():
    assert F.e2m1_encode(np.float32(-0.0)) == 0x8
    assert F.e2m1_encode(np.float32(-0.1)) == 0x8
    assert F.e2m1_encode(np.float32(-6.0)) == 0xF
    assert F.e2m1_encode(np.float32(0.3), sign_src=np.float32(-1)) == 0x9


def test_e4m3_encode_is_nearest_ties_even_saturating():
    rng = np.random.default_rng(2)
    a = _probe_values(F.E4M3_MAGNITUDES, rng, 3000)
    got = F.e4m3_encode_magnitude(a)
    exp = _brute_nearest(a, F.E4M3_MAGNITUDES)
    assert np.array_equal(got, exp)


def test_e4m3_encode_matches_torch_rne_below_saturation():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(50),
        (rng.standard_normal(200000) * 1e-3).astype(np.float32),
        np.float32([447.9, 448.0, 463.99, -463.99, 2.0 ** -10, 2.0 ** -10 * 1.0000001, 0.0, -0.0]),
    ]).astype(np.float32)
    x = x[np.abs(x) < 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(x)
    assert np.array_equal(got, ref)


def test_e4m3_saturates_instead_of_nan():
    assert F.e4m3_encode_magnitude(np.float32(464.0)) == 0x7E
    assert F.e4m3_encode_magnitude(np.float32(1e30)) == 0x7E
    assert F.e4m3_encode(np.float32(-1e30)) == 0xFE


def test_round_fraction_to_f32_and_certification():
    rng = np.random.default_rng(4)
    for _ in range(300):
        a = np.float32(rng.standard_normal() * 10.0 ** float(rng.integers(-30, 30)))
        b = np.nextafter(a, np.float32(np.inf))
        mid = (Fraction(float(a)) + Fraction(float(b))) / 2
        even = a if (int(np.array(a).view(np.uint32)) & 1) == 0 else b
        assert F.round_fraction_to_f32(mid) == even
        assert F.round_fraction_to_f32(mid + Fraction(1, 10 ** 60)) == b
        assert F.round_fraction_to_f32(Fraction(float(a))) == a
    v = np.array([1.0 + 2.0 ** -24, 1.0 + 2.0 ** -23])
    r, ok = F.f32_rounding_certified(v, np.array([0.0, 0.0]))
    assert not ok[0] and ok[1]
    r, ok = F.f32_rounding_certified(np.array([1.0 + 2.0 ** -25]), np.array([2.0 ** -27]))
    assert ok[0] and r[0] == 1.0
    r, ok = F.f32_rounding_certified(np.array([1.0 + 2.0 ** -25]), np.array([2.0 ** -24]))
    assert not ok[0]


@pytest.mark.parametrize("sign", [1, -1])
def test_round_fraction_sign_symmetry(sign):
    q = Fraction(sign * 7, 3)
    assert F.round_fraction_to_f32(q) == sign * np.float32(7.0 / 3.0)


def test_bf16_round_matches_torch_and_ties_to_even():
    import torch
    rng = np.random.default_rng(5)
    a = np.concatenate([rng.standard_normal(50000) * 1e3, rng.standard_normal(50000) * 1e-30,
                        rng.uniform(-7, 7, 50000)]).astype(np.float32)
    # exact ties: low 16 bits 0x8000 with even and odd kept LSB
    base = rng.integers(0, 0x7F00, 1000, dtype=np.uint32) << 16
    ties = np.concatenate([base | 0x8000, (base | 0x10000) | 0x8000]).view(np.float32)
    for v in (a, ties):
        got = F.bf16_round(v)
        ref = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # tie cases by hand: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> the even 1.0
    assert F.bf16_round(np.float32([1 + 2.0 ** -8]))[0] == 1.0
    assert F.bf16_round(np.float32([1 + 3 * 2.0 ** -8]))[0] == np.float32(1 + 2 * 2.0 ** -7)


def test_bf16_round_exact_is_the_nearest_bf16():
    """Brute force: every BF16 value between 1/4 and 4 and near the subnormal floor, each exact midpoint
    between neighbours (ties to the even significand), and points just off the midpoints."""
    ranges = [np.arange(0x3E80, 0x4081), np.arange(0x0000, 0x0100)]  # [1/4, 4] and the subnormal floor
    tables = [(r.astype(np.uint32) << 16).view(np.float32).astype(np.float64) for r in ranges]
    vals = np.concatenate(tables)
    mids = np.concatenate([(t[:-1] + t[1:]) / 2 for t in tables])  # midpoints inside each range only
    off = np.concatenate([mids * (1 + 2.0 ** -40), mids * (1 - 2.0 ** -40)])
    off = off[off > 0]
    for v in (vals, mids, off, -mids):
        got = F.bf16_round_exact(v)
        # nearest table entry by brute force, ties to the even bit pattern
        a = np.abs(v)[:, None]
        d = np.abs(a - vals[None, :])
        best = d.min(axis=1, keepdims=True)
        cand = np.where(d == best, vals[None, :], np.nan)
        lo, hi = np.nanmin(cand, axis=1), np.nanmax(cand, axis=1)
        even_lo = ((lo.astype(np.float32).view(np.uint32) >> 16) & 1) == 0
        want = np.where(lo == hi, lo, np.where(even_lo, lo, hi)) * np.sign(v)
        assert np.array_equal(got, want)
    # on float32-exact inputs it is the pinned binary32 -> BF16 rounding
    x = np.random.default_rng(5).standard_normal(100000).astype(np.float32)
    assert np.array_equal(F.bf16_round_exact(x.astype(np.float64)), F.bf16_round(x).astype(np.float64))
