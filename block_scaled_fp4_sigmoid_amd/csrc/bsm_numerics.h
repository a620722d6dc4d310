// bsm_numerics.h -- scalar numerics shared by the gfx950 kernels.
//
// Every function here is __host__ __device__ so the same code can be unit
// tested on the host.  All arithmetic is IEEE binary32/binary64 with
// round-to-nearest-even; the library is built with -ffp-contract=off, so an
// expression rounds exactly where it is written and FMAs appear only where
// fma()/fmaf() is called.
//
// Contents
//   * E2M1 / E4M3 (OCP E4M3FN) encoders and decoders: nearest value, ties to
//     the even code, saturating at 6 / 448 -- the element and block-scale
//     formats of NVFP4 ("NVFP4 quantization" page, "Quantization scheme") and
//     of FP8_DYNAMIC ("FP8 quantization" page, "Quantization scheme").
//   * exact rounding helpers used by the router, whose logits and sigmoid
//     scores are defined as exactly rounded binary32 values ("Reflection
//     releases Beam" news page, "Residual stream and numerical decisions":
//     the router runs in FP32):
//       - f32_certified(): binary64 estimate + error bound -> binary32 result
//         when provably correctly rounded;
//       - a signed fixed-point superaccumulator that sums binary64 products
//         exactly and rounds once to binary32;
//       - a double-double evaluation of 1/(1+exp(-l)) for the rare scores the
//         binary64 estimate cannot decide.
#pragma once

#include <stdint.h>
#include <math.h>

#if !defined(__HIPCC__)
#ifndef __host__
#define __host__
#endif
#ifndef __device__
#define __device__
#endif
#endif

#define BSM_HD __host__ __device__ inline

namespace bsm {

BSM_HD uint32_t f2u(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  return v.u;
}
BSM_HD float u2f(uint32_t u) {
  union { float f; uint32_t u; } v;
  v.u = u;
  return v.f;
}
BSM_HD uint64_t d2u(double f) {
  union { double f; uint64_t u; } v;
  v.f = f;
  return v.u;
}
BSM_HD double u2d(uint64_t u) {
  union { double f; uint64_t u; } v;
  v.u = u;
  return v.f;
}
BSM_HD float bf16_to_f32(uint16_t b) { return u2f(((uint32_t)b) << 16); }

// ---------------------------------------------------------------------------
// E2M1: magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.  Round-to-nearest-even
// thresholds: ties at .25, 1.25, 2.5, 5 go down (to the even code), ties at
// .75, 1.75, 3.5 go up.  NaN -> 0, beyond 5 -> 6 (saturation).
// ---------------------------------------------------------------------------
BSM_HD uint32_t e2m1_code_mag(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
         (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
}
BSM_HD float e2m1_value_mag(uint32_t c) {
  // c in 0..7: e = c>>1, m = c&1 ; e==0 -> m/2 ; else (1+m/2) * 2^(e-1)
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  return e == 0 ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * (float)(1u << (e - 1));
}

// ---------------------------------------------------------------------------
// E4M3 (OCP E4M3FN): bias 7, subnormal quantum 2^-9, max finite 448 (0x7E).
// ---------------------------------------------------------------------------
BSM_HD float e4m3_value_mag(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9
  return u2f(((e + 120u) << 23) | (m << 20));   // (1+m/8) * 2^(e-7)
}
// Nearest E4M3 magnitude code of a >= 0 (ties to even code, saturate at 448, NaN -> 0).
BSM_HD uint32_t e4m3_code_mag(float a) {
  if (!(a == a)) return 0u;
  if (a >= 448.0f) return 0x7Eu;
  if (a < 0.015625f) {                    // below 2^-6: subnormal grid m * 2^-9
    const float q = a * 512.0f;           // exact scaling
    return (uint32_t)rintf(q);            // 0..8 (8 == code of 2^-6)
  }
  const uint32_t b = f2u(a);
  const uint32_t lsb = (b >> 20) & 1u;
  const uint32_t r = b + 0x7FFFFu + lsb;  // round the low 20 mantissa bits, ties to even
  const uint32_t e = (r >> 23) - 120u;    // E4M3 exponent field (>= 1 here)
  uint32_t code = (e << 3) | ((r >> 20) & 7u);
  return code > 0x7Eu ? 0x7Eu : code;
}

// The E2M1 code of fl32(a / d2) as comparisons of a.  e2m1_code_mag counts seven tests on the binary32
// quotient q = fl32(a / d2): q > 0.25, q >= 0.75, q > 1.25, q >= 1.75, q > 2.5, q >= 3.5, q > 5.  Each
// threshold t has an even last significand bit, so with ties to even a test on q is a test on the exact
// quotient against the midpoint next to t: a / d2 > t + u/2 (the strict tests, i even) or a / d2 >= t - u/2
// (i odd), u being the spacing of binary32 values at t (only 0.25, a strict one, is a power of two).  For
// 0 < d2 <= FLT_MAX that is a > M d2 or a >= M d2, and M d2 is exact in binary64 (25 + 24 significant
// bits).  e2m1_threshold(d2, i) is the smallest binary32 T with that property, so test i holds exactly
// when a >= T (NaN a fails every test, as in e2m1_code_mag).  (M d2 itself is never a binary32 value: M's
// significand has 25 bits ending in 1, so the strict and the other tests differ only in principle.)
BSM_HD float e2m1_threshold(float d2, int i) {
  const double M = i == 0 ? 0.25 + 0x1p-26 : i == 1 ? 0.75 - 0x1p-25 : i == 2 ? 1.25 + 0x1p-24
                 : i == 3 ? 1.75 - 0x1p-24 : i == 4 ? 2.5 + 0x1p-23  : i == 5 ? 3.5 - 0x1p-23
                 : 5.0 + 0x1p-22;
  const double B = M * (double)d2;
  float t = (float)B;
  const bool bump = (i & 1) ? (double)t < B : (double)t <= B;
  if (bump && t != __builtin_huge_valf()) t = u2f(f2u(t) + 1u);
  return t;
}

// ---------------------------------------------------------------------------
// binary64 -> binary32 rounding with a proof obligation.
// Returns true when every real in [v - err, v + err] rounds to the same
// binary32 value as v (written to *out).
// ---------------------------------------------------------------------------
BSM_HD bool f32_certified(double v, double err, float* out) {
  const float r = (float)v;
  *out = r;
  if (!(r - r == 0.0f)) return false;  // inf / nan
  const double rd = (double)r;
  const double lo = (double)nextafterf(r, -INFINITY);
  const double hi = (double)nextafterf(r, INFINITY);
  const double mlo = 0.5 * (rd + lo), mhi = 0.5 * (rd + hi);
  return (v - err > mlo) && (v + err < mhi);
}

// Lowest set-bit exponent of a nonzero binary32 value (value = odd * 2^lsb).
BSM_HD int f32_lsb_exp(float f) {
  const uint32_t b = f2u(f) & 0x7FFFFFFFu;
  const uint32_t ef = b >> 23;
  uint32_t sig = b & 0x7FFFFFu;
  int e0;
  if (ef == 0) {
    e0 = -149;
  } else {
    sig |= 0x800000u;
    e0 = (int)ef - 150;
  }
  return e0 + __builtin_ctz(sig);  // f != 0, so sig != 0
}

// ---------------------------------------------------------------------------
// Exact sum of binary64 values that are products of two binary32 values
// (|p| in [2^-298, 2^256)).  Fixed point with base 2^BASE, NDIG signed 64-bit
// digits of 32 bits each; every add touches 3 digits.  Up to 2^30 terms per
// digit array before any digit can overflow.
// ---------------------------------------------------------------------------
constexpr int SA_BASE = -352;
constexpr int SA_NDIG = 22;

BSM_HD void sa_add(int64_t* dig, double p) {
  if (p == 0.0) return;
  const uint64_t b = d2u(p);
  const int ef = (int)((b >> 52) & 0x7FF);
  if (ef == 0x7FF) return;  // Inf/NaN input: the result is unspecified, the digit index must stay in range
  uint64_t m = b & 0xFFFFFFFFFFFFFull;
  int e;
  if (ef == 0) {
    e = -1074;
  } else {
    m |= 1ull << 52;
    e = ef - 1075;
  }
  const int pos = e - SA_BASE;  // >= 0 for products of binary32 values
  const int d = pos >> 5, o = pos & 31;
  const uint64_t lo = m << o;
  const uint64_t hi = o ? (m >> (64 - o)) : 0ull;
  const int64_t c0 = (int64_t)(lo & 0xFFFFFFFFull), c1 = (int64_t)(lo >> 32), c2 = (int64_t)hi;
  if (b >> 63) {
    dig[d] -= c0;
    dig[d + 1] -= c1;
    dig[d + 2] -= c2;
  } else {
    dig[d] += c0;
    dig[d + 1] += c1;
    dig[d + 2] += c2;
  }
}

// Round (W + tail) * 2^wexp, 0 <= tail < 1 (sticky = tail > 0), to binary32 (RNE).
BSM_HD float round_u64_to_f32(uint64_t W, bool sticky, int wexp, bool neg) {
  if (W == 0) return neg ? -0.0f : 0.0f;  // tail < 2^wexp is far below 2^-149 here
  int lb = 63;
  while (((W >> lb) & 1ull) == 0ull) --lb;
  int lsb_e = lb + wexp - 23;
  if (lsb_e < -149) lsb_e = -149;
  const int shift = lsb_e - wexp;
  uint64_t mant;
  if (shift <= 0) {
    mant = W << (-shift);  // exact (value has at most 24 bits and no tail)
  } else if (shift >= 64) {
    // everything is below the last binary32 place: only half-way matters
    const bool above_half = (shift == 64) && ((W >> 63) & 1ull) && (((W << 1) != 0ull) || sticky);
    mant = above_half ? 1ull : 0ull;
  } else {
    mant = W >> shift;
    const uint64_t rem = W & ((1ull << shift) - 1ull);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (sticky || (mant & 1ull)))) ++mant;
  }
  const float v = ldexpf((float)mant, lsb_e);  // mant <= 2^24: exact
  return neg ? -v : v;
}

// Finish a digit array: propagate carries, take the sign, round once to binary32.
BSM_HD float sa_round_f32(int64_t* dig) {
  for (int d = 0; d < SA_NDIG - 1; ++d) {
    const int64_t c = dig[d] >> 32;  // floor division by 2^32
    dig[d] -= c * 4294967296ll;
    dig[d + 1] += c;
  }
  bool neg = dig[SA_NDIG - 1] < 0;
  if (neg) {
    for (int d = 0; d < SA_NDIG; ++d) dig[d] = -dig[d];
    for (int d = 0; d < SA_NDIG - 1; ++d) {
      const int64_t c = dig[d] >> 32;
      dig[d] -= c * 4294967296ll;
      dig[d + 1] += c;
    }
  }
  int h = SA_NDIG - 1;
  while (h > 0 && dig[h] == 0) --h;
  uint64_t W;
  bool sticky = false;
  int wexp;
  if (h == 0) {
    W = (uint64_t)dig[0];
    wexp = SA_BASE;
  } else {
    W = ((uint64_t)dig[h] << 32) | (uint64_t)dig[h - 1];
    wexp = SA_BASE + 32 * (h - 1);
    for (int d = 0; d < h - 1; ++d) sticky |= dig[d] != 0;
    // dig[h] < 2^31 here, so W keeps every bit of the top two digits
  }
  return round_u64_to_f32(W, sticky, wexp, neg);
}

// ---------------------------------------------------------------------------
// Fixed-point window for the exact sum of binary64 products (fast path).
// Five signed digits of 48 bits; bit 0 of digit 0 has weight 2^base.  With
// base = (lsb of the largest product) - 120 every product whose lowest bit is
// >= 2^base lands in digits 0..4 and a sum of up to 2^10 * 4 (thread) terms
// cannot overflow a digit.  win_add returns false for a product below the
// window (the caller then uses the general superaccumulator).
// ---------------------------------------------------------------------------
constexpr int WIN_DIGITS = 5;

BSM_HD int win_base(int emax_biased) { return emax_biased - 1075 - 120; }

BSM_HD bool win_add(int64_t* dig, double p, int base) {
  if (p == 0.0) return true;
  const uint64_t b = d2u(p);
  const int ef = (int)((b >> 52) & 0x7FF);
  if (ef == 0x7FF) return true;  // Inf/NaN input: ignored, the result is unspecified
  const uint64_t M = (b & 0xFFFFFFFFFFFFFull) | (ef ? (1ull << 52) : 0ull);
  const int lsb = (ef ? ef : 1) - 1075;
  const int shift = lsb - base;
  if (shift < 0 || shift > 120) return false;
  const int d = shift / 48, r = shift % 48;
  const uint64_t lo = M << r;
  const uint64_t hi = r ? (M >> (64 - r)) : 0ull;
  const uint64_t mask = (1ull << 48) - 1;
  const int64_t c0 = (int64_t)(lo & mask);
  const int64_t c1 = (int64_t)(((lo >> 48) | (hi << 16)) & mask);
  const int64_t c2 = (int64_t)(hi >> 32);
  const int64_t sg = (b >> 63) ? -1 : 1;
  dig[0] += sg * (d == 0 ? c0 : 0);
  dig[1] += sg * (d == 0 ? c1 : (d == 1 ? c0 : 0));
  dig[2] += sg * (d == 0 ? c2 : (d == 1 ? c1 : c0));
  dig[3] += sg * (d == 1 ? c2 : (d == 2 ? c1 : 0));
  dig[4] += sg * (d == 2 ? c2 : 0);
  return true;
}

// Round the window value sum_q D[q] * 2^(base + 48 q) to binary32 (D is modified).
BSM_HD float win_round_f32(int64_t* D, int base) {
  for (int q = 0; q < WIN_DIGITS - 1; ++q) {
    const int64_t c = D[q] >> 48;  // floor division by 2^48
    D[q] -= c * (int64_t)(1ll << 48);
    D[q + 1] += c;
  }
  const bool neg = D[WIN_DIGITS - 1] < 0;
  if (neg) {
    for (int q = 0; q < WIN_DIGITS; ++q) D[q] = -D[q];
    for (int q = 0; q < WIN_DIGITS - 1; ++q) {
      const int64_t c = D[q] >> 48;
      D[q] -= c * (int64_t)(1ll << 48);
      D[q + 1] += c;
    }
  }
  int h = WIN_DIGITS - 1;
  while (h > 0 && D[h] == 0) --h;
  uint64_t W;
  bool sticky = false;
  int wexp;
  if (h == 0) {
    W = (uint64_t)D[0];
    wexp = base;
  } else {
    // W keeps at least 33 leading bits exactly: enough to round to 24 bits
    const uint64_t dh = (uint64_t)D[h], dl = (uint64_t)D[h - 1];  // dh < 2^48 except in the top digit
    for (int q = 0; q < h - 1; ++q) sticky |= D[q] != 0;
    if (dh < (1ull << 16)) {
      W = (dh << 48) | dl;
      wexp = base + 48 * (h - 1);
    } else if (dh < (1ull << 48)) {
      W = (dh << 16) | (dl >> 32);
      sticky |= (dl & 0xFFFFFFFFull) != 0;
      wexp = base + 48 * (h - 1) + 32;
    } else {  // top digit beyond 48 bits (only possible in digit 4)
      W = dh;
      sticky |= dl != 0;
      wexp = base + 48 * h;
    }
  }
  return round_u64_to_f32(W, sticky, wexp, neg);
}

// ---------------------------------------------------------------------------
// double-double arithmetic (error-free transforms, Dekker / Knuth)
// ---------------------------------------------------------------------------
struct dd {
  double hi, lo;
};
BSM_HD dd two_sum(double a, double b) {
  const double s = a + b;
  const double bb = s - a;
  const double e = (a - (s - bb)) + (b - bb);
  return {s, e};
}
BSM_HD dd quick_two_sum(double a, double b) {
  const double s = a + b;
  return {s, b - (s - a)};
}
BSM_HD dd two_prod(double a, double b) {
  const double p = a * b;
  return {p, fma(a, b, -p)};
}
BSM_HD dd dd_add(dd a, dd b) {
  dd s = two_sum(a.hi, b.hi);
  dd t = two_sum(a.lo, b.lo);
  s.lo += t.hi;
  s = quick_two_sum(s.hi, s.lo);
  s.lo += t.lo;
  return quick_two_sum(s.hi, s.lo);
}
BSM_HD dd dd_mul(dd a, dd b) {
  dd p = two_prod(a.hi, b.hi);
  p.lo += a.hi * b.lo + a.lo * b.hi;
  return quick_two_sum(p.hi, p.lo);
}
BSM_HD dd dd_mul_d(dd a, double b) {
  dd p = two_prod(a.hi, b);
  p.lo += a.lo * b;
  return quick_two_sum(p.hi, p.lo);
}
BSM_HD dd dd_div(dd a, dd b) {
  const double q1 = a.hi / b.hi;
  dd r = dd_add(a, dd_mul_d(b, -q1));
  const double q2 = r.hi / b.hi;
  r = dd_add(r, dd_mul_d(b, -q2));
  const double q3 = r.hi / b.hi;
  dd q = quick_two_sum(q1, q2);
  return dd_add(q, dd{q3, 0.0});
}

// exp(x) in double-double for |x| <= 745 (Cody-Waite reduction by ln 2 split
// into three binary64 parts, Taylor series of degree 27 in Horner form).
BSM_HD dd dd_exp(double x) {
  const double LN2_HI = 0x1.62e42fee00000p-1;  // 32 significant bits: k*LN2_HI is exact
  const double LN2_MID = 0x1.a39ef35793c76p-33;
  const double LN2_LO = 0x1.cc01f97b57a08p-87;
  const double k = rint(x * 0x1.71547652b82fep+0);
  dd r = two_sum(x, -k * LN2_HI);
  r = dd_add(r, two_prod(-k, LN2_MID));
  r = dd_add(r, dd{-k * LN2_LO, 0.0});
  dd t = {1.0, 0.0};
#pragma unroll 1
  for (int n = 27; n >= 1; --n) {
    t = dd_mul(t, r);
    t = dd_div(t, dd{(double)n, 0.0});
    t = dd_add(t, dd{1.0, 0.0});
  }
  const int ki = (int)k;
  return {ldexp(t.hi, ki), ldexp(t.lo, ki)};
}

// binary32 rounding of hi + lo (|lo| <= ulp(hi)/2).
BSM_HD float dd_to_f32(dd v) {
  const float r = (float)v.hi;
  const double rd = (double)r;
  if (rd == v.hi || v.lo == 0.0) return r;
  const float other = (v.hi > rd) ? nextafterf(r, INFINITY) : nextafterf(r, -INFINITY);
  const double mid = 0.5 * (rd + (double)other);
  if (v.hi != mid) return r;  // not on a binary32 rounding boundary
  // hi sits exactly on the boundary: lo decides
  if ((v.lo > 0.0) == (v.hi > rd)) return other;
  return r;
}

// 1 / (1 + exp(-l)) exactly rounded to binary32.  fast_ok: the binary64 path
// was certified (otherwise the double-double path was taken).
BSM_HD float sigmoid_f32_exact(float l, bool* fast_ok) {
  const double x = -(double)l;
  const double e = exp(x);
  const double s = 1.0 / (1.0 + e);
  float r;
  // binary64 exp is accurate to a few ulp; 2^-47 relative covers it with margin
  if (f32_certified(s, s * 0x1p-47, &r)) {
    *fast_ok = true;
    return r;
  }
  *fast_ok = false;
  if (x > 700.0) return 0.0f;  // sigmoid < 2^-1000 (never reached: certified above)
  const dd E = dd_exp(x);
  const dd den = dd_add(dd{1.0, 0.0}, E);
  return dd_to_f32(dd_div(dd{1.0, 0.0}, den));
}

}  // namespace bsm
