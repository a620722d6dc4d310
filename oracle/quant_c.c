/* quant_c.c -- the oracle's NVFP4 and FP8_DYNAMIC quantizers as plain C loops.
 *
 * TEST INFRASTRUCTURE ONLY -- part of the CPU oracle; never linked into or
 * called by the product library.  Built by oracle/build_c.py with gcc
 * (-O2 -fno-fast-math -ffp-contract=off, OpenMP over rows).
 *
 * The same definitions as oracle/quant.py, one element at a time, so that
 * full-size tensors (a Beam expert is 39.3 M weights) can be quantized in
 * seconds.  tests/test_oracle_quant_c.py pins this file bit-exactly against
 * oracle/quant.py on random, heavy-tailed, zero, subnormal-scale and
 * underflowing inputs.
 *
 * Sources: "NVFP4 quantization" page, "Quantization scheme" (E2M1 elements,
 * one E4M3 scale per block of 16 values, one more global scale per tensor);
 * "FP8 quantization" page, "Quantization scheme" and "Quantization method"
 * (E4M3 values, one scale per row; each quotient value / scale becomes the
 * closest E4M3 value).
 *
 * Readings (the same as oracle/quant.py):
 *   S_g = fl32(amax / 2688); s_b = E4M3(fl32(a_b / fl32(6 S_g)));
 *   q = E2M1(fl32(x / fl32(s_b S_g))); a zero block scale gives +-0 codes;
 *   the sign bit is the sign of x; element 2j in the low nibble of byte j;
 *   FP8 row scale s = fl32(amax / 448), q = E4M3(fl32(x / s)).
 *   Encoding = nearest entry of the format's value table, ties to the even
 *   code, saturating at the largest finite value; NaN encodes as 0 (the
 *   tables are built from the formats' bit-level definitions; the encoders
 *   find the nearest entry by midpoint counts (E2M1) and by the even spacing
 *   of the entries inside a binade (E4M3)).
 * Every float operation below is one IEEE binary32 operation (SSE, no
 * contraction), in the order the readings write them.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---- formats, from their bit-level definitions ------------------------ */

/* E2M1 magnitude of code c (0..7): exponent e = c >> 1, mantissa m = c & 1, bias 1. */
static double e2m1_mag(int c) {
  const int e = c >> 1, m = c & 1;
  return e == 0 ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
}

/* OCP E4M3FN magnitude of code c (0..126): exponent 4 bits, mantissa 3, bias 7. */
static double e4m3_mag(int c) {
  const int e = (c >> 3) & 15, m = c & 7;
  return e == 0 ? (m / 8.0) * ldexp(1.0, -6) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
}

static double E2M1[8];
static double E4M3[127];
static double E2M1_MID[7]; /* midpoints between neighbouring E2M1 magnitudes */
static int tables_ready = 0;

static void init_tables(void) {
  if (tables_ready) return;
  for (int c = 0; c < 8; ++c) E2M1[c] = e2m1_mag(c);
  for (int c = 0; c < 127; ++c) E4M3[c] = e4m3_mag(c);
  for (int i = 0; i < 7; ++i) E2M1_MID[i] = 0.5 * (E2M1[i] + E2M1[i + 1]);
  tables_ready = 1;
}

/* Nearest-value encoders, ties to the even code, saturating at the largest finite magnitude, NaN -> 0.
 *
 * E2M1: the codes are the table indices and the table is increasing, so the nearest index is the
 * number of midpoints between neighbouring entries that a lies above; at a midpoint exactly, the even
 * one of the two neighbours.  Saturation falls out (a above every midpoint gives 7), and every
 * comparison with NaN is false (code 0).  Midpoints are exact in binary64. */
static int e2m1_nearest(double a) {
  int code = 0;
  for (int i = 0; i < 7; ++i) code += (a > E2M1_MID[i]) | ((a == E2M1_MID[i]) & ((i + 1) % 2 == 0));
  return code;
}

/* E4M3: inside the binade [2^k, 2^(k+1)) (k >= -6) the entries are 2^k (1 + j/8), evenly spaced,
 * and below 2^-6 they are j 2^-9; code = 8 (k + 7) + j (subnormals: j).  So a 2^(3-k) (exact: a
 * power-of-two scaling) rounded to the nearest integer, ties to even (rint in the default rounding
 * mode), is 8 + j, or 16 when a rounds up to the next binade's first entry, which the same formula
 * encodes.  The code's parity is the integer's, so ties go to the even code.  At or above 448 (code
 * 126) it saturates. */
static int e4m3_nearest(double a) {
  if (a != a) return 0;
  if (a >= 448.0) return 126;
  if (a < 0x1p-6) return (int)rint(a * 0x1p9);  /* 0..8; 8 is the first normal entry, 2^-6 */
  int k;
  frexp(a, &k);
  k -= 1; /* a in [2^k, 2^(k+1)) */
  const int t = (int)rint(ldexp(a, 3 - k)); /* 8..16 */
  const int code = 8 * (k + 7) + (t - 8);
  return code > 126 ? 126 : code;
}

static float load_value(const void* x, int bf16, int64_t i) {
  if (bf16) {
    const uint32_t b = (uint32_t)((const uint16_t*)x)[i] << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
  }
  return ((const float*)x)[i];
}

static int sign_bit(float v) { return signbit(v) ? 1 : 0; }

/* ---- NVFP4 -------------------------------------------------------------- */

void orq_nvfp4_quantize(const void* x, int bf16, int64_t R, int64_t C, int static_gs, float gs_in,
                        uint8_t* codes, uint8_t* scales, float* gs_out) {
  init_tables();
  const int64_t n = R * C, nb = C / 16;
  float amax = 0.0f;
  if (!static_gs) {
#pragma omp parallel for reduction(max : amax) schedule(static)
    for (int64_t i = 0; i < n; ++i) {
      const float a = fabsf(load_value(x, bf16, i));
      if (a > amax) amax = a;
    }
  }
  const float sg = static_gs ? gs_in : amax / 2688.0f;
  const float d1 = 6.0f * sg;
  *gs_out = sg;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const int64_t base = r * C + 16 * b;
      float v[16], ab = 0.0f;
      for (int k = 0; k < 16; ++k) {
        v[k] = load_value(x, bf16, base + k);
        const float a = fabsf(v[k]);
        if (a > ab) ab = a;
      }
      int sc = 0;
      if (sg != 0.0f) {
        const float q = ab / d1;
        sc = e4m3_nearest(fabs((double)q));
      }
      scales[r * nb + b] = (uint8_t)sc;
      const float sb = (float)E4M3[sc]; /* exact: 4 significant bits */
      const float d2 = sb * sg;
      uint8_t nib[16];
      for (int k = 0; k < 16; ++k) {
        int code;
        if (sb == 0.0f) {
          code = 0;
        } else {
          const float q = v[k] / d2;
          code = e2m1_nearest(fabs((double)q));
        }
        nib[k] = (uint8_t)(code | (sign_bit(v[k]) << 3));
      }
      for (int j = 0; j < 8; ++j) codes[(base >> 1) + j] = (uint8_t)(nib[2 * j] | (nib[2 * j + 1] << 4));
    }
  }
}

/* Exact decoded values q * s_b * S_g in binary64 (<= 30 significant bits). */
void orq_nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, float sg, int64_t R, int64_t C,
                          double* out) {
  init_tables();
  const int64_t nb = C / 16;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t i = 0; i < C; ++i) {
      const int byte = codes[(r * C + i) >> 1];
      const int c = (i & 1) ? (byte >> 4) : (byte & 15);
      const double q = (c & 8) ? -E2M1[c & 7] : E2M1[c & 7];
      const int s = scales[r * nb + i / 16];
      const double sb = (s & 0x80) ? -E4M3[s & 0x7F] : E4M3[s & 0x7F];
      out[r * C + i] = (q * sb) * (double)sg;
    }
  }
}

/* ---- FP8_DYNAMIC (per row) --------------------------------------------- */

void orq_fp8_quantize(const void* x, int bf16, int64_t R, int64_t C, uint8_t* codes, float* scales) {
  init_tables();
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    float amax = 0.0f;
    for (int64_t i = 0; i < C; ++i) {
      const float a = fabsf(load_value(x, bf16, r * C + i));
      if (a > amax) amax = a;
    }
    const float s = amax / 448.0f;
    scales[r] = s;
    for (int64_t i = 0; i < C; ++i) {
      const float v = load_value(x, bf16, r * C + i);
      int code = 0;
      if (s != 0.0f) {
        const float q = v / s;
        code = e4m3_nearest(fabs((double)q));
      }
      codes[r * C + i] = (uint8_t)(code | (sign_bit(v) << 7));
    }
  }
}

/* Exact decoded values q * s in binary64 (4 + 24 significant bits). */
void orq_fp8_dequantize(const uint8_t* codes, const float* scales, int64_t R, int64_t C, double* out) {
  init_tables();
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    const double s = (double)scales[r];
    for (int64_t i = 0; i < C; ++i) {
      const int c = codes[r * C + i];
      const double q = (c & 0x80) ? -E4M3[c & 0x7F] : E4M3[c & 0x7F];
      out[r * C + i] = q * s;
    }
  }
}
