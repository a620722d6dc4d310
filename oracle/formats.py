"""Element formats (E2M1, OCP E4M3FN) and exact FP32 rounding helpers.

TEST INFRASTRUCTURE ONLY -- part of the CPU oracle; never used by the product path.

Sources:
* "NVFP4 quantization" page, "Quantization scheme": elements are 4-bit E2M1,
  block scales are FP8 E4M3.
* "FP8 quantization" page, "Quantization scheme" / "Quantization method": E4M3
  elements; a scaled value becomes the closest E4M3 value.

The pages name the formats but print neither value grid.  The grids below are
the formats' own definitions:
* E2M1: sign | 2 exponent bits | 1 mantissa bit, bias 1, no Inf/NaN.
  Magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* E4M3 (OCP "E4M3FN"): sign | 4 exponent bits | 3 mantissa bits, bias 7,
  codes 0x7F/0xFF are NaN, largest finite 448, smallest subnormal 2^-9.

Rounding reading (the pages only say "round to nearest"): nearest representable
value, ties to the even code (mantissa LSB 0), values beyond the largest finite
magnitude saturate to it.  Encoders here are written as "nearest entry of the
value table", which makes that reading explicit; tests pin them against a
brute-force argmin over the whole table.

* BF16 (weight-only path's activations): the upper 16 bits of binary32;
  rounding binary32 -> BF16 is round to nearest, ties to even.

Parity: pinned (exhaustive decode vs. the bit-level definition, brute-force
nearest encode over all midpoints +-1 ulp and random inputs; BF16 rounding
against torch's conversion and constructed ties).
"""

from fractions import Fraction

import numpy as np

# --------------------------------------------------------------------------
# E2M1
# --------------------------------------------------------------------------


def e2m1_decode(codes):
    """Decode 4-bit E2M1 codes (bit 3 = sign) to float64 values."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    mag = c & 7
    e = mag >> 1
    m = mag & 1
    val = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(c & 8, -val, val)


E2M1_MAGNITUDES = e2m1_decode(np.arange(8))  # [0, .5, 1, 1.5, 2, 3, 4, 6]

# --------------------------------------------------------------------------
# E4M3 (OCP E4M3FN)
# --------------------------------------------------------------------------


def e4m3_decode(codes):
    """Decode 8-bit OCP E4M3FN codes to float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    e = (c >> 3) & 0xF
    m = c & 7
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return np.where(c & 0x80, -val, val)


E4M3_MAGNITUDES = e4m3_decode(np.arange(0x7F))  # codes 0..126, strictly increasing
E4M3_MAX = float(E4M3_MAGNITUDES[-1])  # 448
E2M1_MAX = float(E2M1_MAGNITUDES[-1])  # 6


def _nearest_code(a, table):
    """Index of the nearest table entry to each non-negative a.

    ``table`` is strictly increasing and starts at 0.  Ties go to the even
    index (the even code); a >= table[-1] gives the last index (saturation).
    NaN maps to code 0.  Differences are exact in float64 because a is a
    float32 value lying between two neighbouring table entries.
    """
    a = np.asarray(a, dtype=np.float64)
    n = len(table)
    hi = np.searchsorted(table, a, side="left")
    hi = np.clip(hi, 0, n - 1)
    lo = np.clip(hi - 1, 0, n - 1)
    dlo = a - table[lo]
    dhi = table[hi] - a
    pick_hi = dhi < dlo
    tie = dhi == dlo
    even_hi = (hi & 1) == 0
    idx = np.where(pick_hi | (tie & even_hi), hi, lo)
    idx = np.where(a >= table[-1], n - 1, idx)
    idx = np.where(np.isnan(a), 0, idx)
    return idx.astype(np.uint8)


def e2m1_encode_magnitude(a):
    """3-bit E2M1 magnitude code of |value| (nearest, ties-to-even, saturating)."""
    return _nearest_code(np.abs(np.asarray(a, dtype=np.float64)), E2M1_MAGNITUDES)


def e4m3_encode_magnitude(a):
    """7-bit E4M3 magnitude code of |value| (nearest, ties-to-even, saturating at 448)."""
    return _nearest_code(np.abs(np.asarray(a, dtype=np.float64)), E4M3_MAGNITUDES)


def e2m1_encode(r, sign_src=None):
    """Signed E2M1 code: sign bit from ``sign_src`` (default r), magnitude from |r|."""
    r = np.asarray(r)
    s = np.signbit(r if sign_src is None else np.asarray(sign_src))
    return (e2m1_encode_magnitude(r) | (s.astype(np.uint8) << 3)).astype(np.uint8)


def e4m3_encode(r, sign_src=None):
    """Signed E4M3 code: sign bit from ``sign_src`` (default r), magnitude from |r|."""
    r = np.asarray(r)
    s = np.signbit(r if sign_src is None else np.asarray(sign_src))
    return (e4m3_encode_magnitude(r) | (s.astype(np.uint8) << 7)).astype(np.uint8)


# --------------------------------------------------------------------------
# Exact rounding to float32
# --------------------------------------------------------------------------


def round_fraction_to_f32(q: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32, ties to even significand."""
    if q == 0:
        return np.float32(0.0)
    c = np.float32(float(q))
    cands = [c, np.nextafter(c, np.float32(-np.inf)), np.nextafter(c, np.float32(np.inf))]
    best = None
    for x in cands:
        if not np.isfinite(x):
            continue
        d = abs(Fraction(float(x)) - q)
        key = (d, int(np.array(x, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, x)
    return np.float32(best[1])


def f32_rounding_certified(v, err):
    """Round float64 estimates ``v`` to float32 and say where that is provably exact.

    ``err`` bounds |exact - v|.  The float32 result is the correctly rounded
    value of the exact quantity whenever no float32 rounding boundary (a
    midpoint between neighbouring float32 values) lies within [v-err, v+err].
    Returns (rounded float32 array, bool mask of certified entries).
    """
    v = np.asarray(v, dtype=np.float64)
    err = np.asarray(err, dtype=np.float64)
    r = v.astype(np.float32)
    lo = np.nextafter(r, np.float32(-np.inf)).astype(np.float64)
    hi = np.nextafter(r, np.float32(np.inf)).astype(np.float64)
    r64 = r.astype(np.float64)
    mlo = (r64 + lo) / 2.0
    mhi = (r64 + hi) / 2.0
    ok = (v - err > mlo) & (v + err < mhi) & np.isfinite(r64)
    return r, ok


def bf16_round(a):
    """binary32 -> nearest BF16 value (ties to even), returned as float32.

    BF16 keeps the sign, the 8 exponent bits and the top 7 mantissa bits of
    binary32; the dropped 16 bits round to nearest, ties to the even kept
    mantissa.  Finite inputs only (the callers' values are finite).
    """
    b = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + keep_lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def bf16_round_exact(v):
    """float64 values -> nearest BF16 value (ties to even), rounded once, returned as float64.

    BF16 has 8 significant bits and binary32's exponent range (smallest subnormal
    2^-133).  v = m * 2^e with m in [0.5, 1): the BF16 neighbours of v are the
    multiples of 2^(e-8) (of 2^-133 below the normal range), so v / 2^q rounded
    to the nearest integer with ties to even (numpy's rint) times 2^q is the
    answer; both scalings are exact.  Finite inputs of BF16 range only.
    """
    v = np.asarray(v, np.float64)
    _, e = np.frexp(v)
    q = np.maximum(e - 8, -133)
    return np.ldexp(np.rint(np.ldexp(v, -q)), q)
