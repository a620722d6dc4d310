// Host build of the library's scalar numerics (bsm_numerics.h) for CPU tests:
// the same source the gfx950 kernels use, compiled by g++ and called through
// ctypes so the oracle can check it without a GPU.
#include "../../block_scaled_fp4_sigmoid_amd/csrc/bsm_numerics.h"

extern "C" {

void hc_e4m3_code(const float* a, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)bsm::e4m3_code_mag(a[i]);
}
void hc_e2m1_code(const float* a, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)bsm::e2m1_code_mag(a[i]);
}

// E2M1 magnitude code of fl32(a / d2) from the thresholds (0 < d2 <= FLT_MAX)
void hc_e2m1_code_thr(const float* a, const float* d2, int64_t n, uint8_t* out) {
  for (int64_t k = 0; k < n; ++k) {
    uint32_t c = 0;
    for (int i = 0; i < 7; ++i) c += (uint32_t)(a[k] >= bsm::e2m1_threshold(d2[k], i));
    out[k] = (uint8_t)c;
  }
}
void hc_e4m3_value(const uint8_t* c, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bsm::e4m3_value_mag(c[i]);
}
void hc_e2m1_value(const uint8_t* c, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bsm::e2m1_value_mag(c[i]);
}
// exact dot products of float32 rows through the superaccumulator
void hc_exact_dot(const float* x, const float* w, int64_t rows, int64_t n, float* out) {
  for (int64_t r = 0; r < rows; ++r) {
    int64_t dig[bsm::SA_NDIG] = {0};
    for (int64_t k = 0; k < n; ++k) bsm::sa_add(dig, (double)x[r * n + k] * (double)w[r * n + k]);
    out[r] = bsm::sa_round_f32(dig);
  }
}
// exact dot products through the fixed-point window (returns -1 in ok[r] when a product fell below it)
void hc_window_dot(const float* x, const float* w, int64_t rows, int64_t n, float* out, int32_t* ok) {
  for (int64_t r = 0; r < rows; ++r) {
    int emax = 0;
    for (int64_t k = 0; k < n; ++k) {
      const double p = (double)x[r * n + k] * (double)w[r * n + k];
      const int ex = (int)((bsm::d2u(p) >> 52) & 0x7FF);
      emax = ex > emax ? ex : emax;
    }
    const int base = bsm::win_base(emax);
    int64_t dig[bsm::WIN_DIGITS] = {0, 0, 0, 0, 0};
    bool good = true;
    for (int64_t k = 0; k < n; ++k) good &= bsm::win_add(dig, (double)x[r * n + k] * (double)w[r * n + k], base);
    ok[r] = good ? 1 : 0;
    out[r] = good ? bsm::win_round_f32(dig, base) : 0.0f;
  }
}
void hc_sigmoid(const float* l, int64_t n, float* out, int32_t* fast) {
  for (int64_t i = 0; i < n; ++i) {
    bool f;
    out[i] = bsm::sigmoid_f32_exact(l[i], &f);
    fast[i] = f ? 1 : 0;
  }
}
void hc_sigmoid_dd(const float* l, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) {
    const double x = -(double)l[i];
    if (x > 700.0) {
      out[i] = 0.0f;
      continue;
    }
    const bsm::dd E = bsm::dd_exp(x);
    out[i] = bsm::dd_to_f32(bsm::dd_div(bsm::dd{1.0, 0.0}, bsm::dd_add(bsm::dd{1.0, 0.0}, E)));
  }
}
int hc_f32_certified(double v, double err, float* out) { return bsm::f32_certified(v, err, out) ? 1 : 0; }
int hc_lsb_exp(float f) { return bsm::f32_lsb_exp(f); }
}
