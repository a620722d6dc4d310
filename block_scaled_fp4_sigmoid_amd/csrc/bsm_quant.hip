// bsm_quant.hip -- NVFP4 and FP8_DYNAMIC quantization kernels for gfx950.
//
// NVFP4 ("NVFP4 quantization" page, "Quantization scheme"): E2M1 elements,
// one E4M3 scale per 16 consecutive values, one global scale per tensor.
// FP8_DYNAMIC ("FP8 quantization" page, "Quantization scheme" and
// "Quantization method"): one scale per row; each quotient value / scale
// becomes the closest E4M3 value.
//
// Arithmetic per tensor (binary32, round to nearest even, in this order):
//   S_g = amax / 2688 ; s_b = E4M3(a_b / (6*S_g)) ; q = E2M1(x / (s_b*S_g))
// FP8 row: s = amax / 448 ; q = E4M3(x / s).
//
// Layout: a tensor [R, C] with C % 16 == 0 is a flat sequence of 16-value
// blocks; block f covers elements 16f..16f+15, its codes are bytes 8f..8f+7
// (low nibble = even element) and its scale is byte f.  One thread handles one
// block per iteration, so a wave reads 2 KB (bf16) / 4 KB (f32) contiguous and
// writes 512 B of codes and 64 B of scales contiguous.
//
// The dynamic global scale needs max|x| of the whole tensor before any block
// can be encoded: pass 1 writes one partial maximum per workgroup, pass 2
// reduces those (max is order independent, so the result is deterministic)
// and encodes.  Pass 2 walks the tensor from the end so that the blocks pass 1
// touched last are still in the last-level cache.

#include "bsm_internal.h"

namespace bsm {

namespace {

constexpr int kThreads = 256;

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ inline float block_max(float v, float* lds) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) lds[wid] = v;
  __syncthreads();
  float r = lds[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = fmaxf(r, lds[i]);
  __syncthreads();
  return r;
}

// Load 16 consecutive elements of block f as floats.
template <bool BF16>
__device__ inline void load16(const void* x, int64_t f, float* v) {
  if (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + f * 16);
    const uint4 a = p[0], b = p[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = u2f(w[i] << 16);
      v[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + f * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 q = p[i];
      v[4 * i] = q.x;
      v[4 * i + 1] = q.y;
      v[4 * i + 2] = q.z;
      v[4 * i + 3] = q.w;
    }
  }
}

typedef unsigned int u4v __attribute__((ext_vector_type(4)));
constexpr int kAmaxUnroll = 4;  // 16-byte pieces per lane and iteration

// Pass 1 needs no block structure: consecutive lanes read consecutive 16-byte pieces, non-temporal, so
// each load instruction covers 8 whole 128-byte lines.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_amax_parts(const void* __restrict__ x, int64_t n_blk,
                                                          float* __restrict__ parts, int nparts) {
  __shared__ float lds[kThreads / 64];
  const int b = blockIdx.y;
  const u4v* xb = reinterpret_cast<const u4v*>(BF16 ? (const void*)((const uint16_t*)x + (int64_t)b * n_blk * 16)
                                                    : (const void*)((const float*)x + (int64_t)b * n_blk * 16));
  const int64_t np = n_blk * (BF16 ? 2 : 4);
  float m = 0.0f;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kAmaxUnroll + threadIdx.x; base < np;
       base += (int64_t)nparts * kThreads * kAmaxUnroll) {
    u4v v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kThreads;
      v[u] = i < np ? __builtin_nontemporal_load(xb + i) : u4v{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (BF16) {
          m = fmaxf(m, fabsf(u2f(v[u][i] << 16)));
          m = fmaxf(m, fabsf(u2f(v[u][i] & 0xFFFF0000u)));
        } else {
          m = fmaxf(m, fabsf(u2f(v[u][i])));
        }
      }
    }
  }
  m = block_max(m, lds);
  if (threadIdx.x == 0) parts[(int64_t)b * kAmaxMaxParts + blockIdx.x] = m;
}

// The E2M1 codes of a block without dividing (e2m1_threshold): the thresholds depend on the block scale
// code only (d2 = fl32(E4M3(sc) * S)), so one table per tensor serves every block.  Row sc holds the 7
// thresholds and, in [7], a flag for a d2 of 0 or inf, where the block divides instead.  The division costs
// about ten instructions per element; the table, seven compares.
__device__ inline void build_e2m1_thresholds(float S, float (*thr)[8]) {
  for (int k = threadIdx.x; k < 127 * 8; k += kThreads) {
    const int sc = k >> 3, i = k & 7;
    const float d2 = e4m3_value_mag((uint32_t)sc) * S;
    const bool ok = d2 > 0.0f && d2 <= 3.4028234663852886e38f;
    thr[sc][i] = i == 7 ? (ok ? 0.0f : 1.0f) : ok ? e2m1_threshold(d2, i) : 0.0f;
  }
}

// Encode one 16-value block with global scale S (S > 0, or S == 0 -> zero scales); thr from
// build_e2m1_thresholds(S).
__device__ inline void encode_block(const float* v, float S, float d1, const float (*thr)[8], uint8_t* codes_f,
                                    uint8_t* scale_f, _Float16* dec_f) {
  float ab = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) ab = fmaxf(ab, fabsf(v[i]));
  uint32_t sc = 0;
  if (S != 0.0f) sc = e4m3_code_mag(ab / d1);
  const float sv = e4m3_value_mag(sc);
  const float d2 = sv * S;
  const float4 t03 = *reinterpret_cast<const float4*>(&thr[sc][0]);
  const float4 t47 = *reinterpret_cast<const float4*>(&thr[sc][4]);
  uint32_t q[16];
  if (sv == 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = (f2u(v[i]) >> 31) << 3;
  } else if (t47.w != 0.0f) {  // d2 of 0 or inf: divide
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = ((f2u(v[i]) >> 31) << 3) | e2m1_code_mag(fabsf(v[i]) / d2);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // the number of thresholds at or below a, by binary search over the sorted T_0 <= ... <= T_6
      const float a = fabsf(v[i]);
      const bool hi = a >= t03.w;
      const bool mid = a >= (hi ? t47.y : t03.y);
      const bool lo = a >= (hi ? (mid ? t47.z : t47.x) : (mid ? t03.z : t03.x));
      q[i] = ((f2u(v[i]) >> 31) << 3) | (hi ? 4u : 0u) | (mid ? 2u : 0u) | (lo ? 1u : 0u);
    }
  }
  uint2 packed;
  packed.x = q[0] | (q[1] << 4) | (q[2] << 8) | (q[3] << 12) | (q[4] << 16) | (q[5] << 20) | (q[6] << 24) |
             (q[7] << 28);
  packed.y = q[8] | (q[9] << 4) | (q[10] << 8) | (q[11] << 12) | (q[12] << 16) | (q[13] << 20) |
             (q[14] << 24) | (q[15] << 28);
  *reinterpret_cast<uint2*>(codes_f) = packed;
  *scale_f = (uint8_t)sc;
  if (dec_f) {
    // exact FP16 of q * s_b (at most 6 significant bits, within [2^-10, 2688]): the hardware E2M1 -> FP16
    // converter (unit scale) and one packed multiply by s_b, which FP16 holds exactly
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 s2 = {(_Float16)sv, (_Float16)sv};
#define BSM_DEC2(W, K) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(W, 1.0f, K) * s2)
    uint4* dp = reinterpret_cast<uint4*>(dec_f);
    dp[0] = make_uint4(BSM_DEC2(packed.x, 0), BSM_DEC2(packed.x, 1), BSM_DEC2(packed.x, 2), BSM_DEC2(packed.x, 3));
    dp[1] = make_uint4(BSM_DEC2(packed.y, 0), BSM_DEC2(packed.y, 1), BSM_DEC2(packed.y, 2), BSM_DEC2(packed.y, 3));
#undef BSM_DEC2
  }
}

// mode 0: dynamic from partial maxima; mode 1: static (gs read); mode 2: amax bits given
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_nvfp4_encode(const void* __restrict__ x, int64_t n_blk,
                                                            uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                            float* __restrict__ gs, const float* __restrict__ parts,
                                                            int nparts1, const uint32_t* __restrict__ amax_bits,
                                                            const float* __restrict__ static_gs, int mode,
                                                            int nparts2, _Float16* __restrict__ dec16) {
  __shared__ float lds[kThreads / 64];
  const int b = blockIdx.y;
  float S;
  if (mode == 0) {
    float m = 0.0f;
    for (int i = threadIdx.x; i < nparts1; i += kThreads) m = fmaxf(m, parts[(int64_t)b * kAmaxMaxParts + i]);
    m = block_max(m, lds);
    S = m / 2688.0f;
  } else if (mode == 1) {
    S = static_gs[b];
  } else {
    S = static_gs ? static_gs[b] : u2f(amax_bits[b]) / 2688.0f;
  }
  if (gs && mode != 1 && blockIdx.x == 0 && threadIdx.x == 0) gs[b] = S;
  const float d1 = 6.0f * S;
  __shared__ __attribute__((aligned(16))) float thr[128][8];
  build_e2m1_thresholds(S, thr);
  __syncthreads();
  const void* xb = BF16 ? (const void*)((const uint16_t*)x + (int64_t)b * n_blk * 16)
                        : (const void*)((const float*)x + (int64_t)b * n_blk * 16);
  uint8_t* cb = codes + (int64_t)b * n_blk * 8;
  uint8_t* sb = scales + (int64_t)b * n_blk;
  // walk from the end of the tensor (the blocks pass 1 read last come first)
  const int64_t start = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (int64_t g = start; g < n_blk; g += (int64_t)nparts2 * kThreads) {
    const int64_t f = n_blk - 1 - g;
    float v[16];
    load16<BF16>(xb, f, v);
    encode_block(v, S, d1, thr, cb + f * 8, sb + f, dec16 ? dec16 + (int64_t)b * n_blk * 16 + f * 16 : nullptr);
  }
}

// out = the exact q * s_b * S_g rounded once: to binary32 (fl32 of an exact product: q * s_b is exact in
// binary32) or to BF16 (from the exact binary64 product: rounded to odd at binary32, whose 24 bits leave
// room for the single correct round to nearest even at BF16's 8 bits).
template <bool BF16_OUT>
__global__ __launch_bounds__(kThreads) void k_nvfp4_decode(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           const float* __restrict__ gs, int64_t n_blk,
                                                           void* __restrict__ out) {
  const int b = blockIdx.y;
  const float S = gs[b];
  const uint8_t* cb = codes + (int64_t)b * n_blk * 8;
  const uint8_t* sb = scales + (int64_t)b * n_blk;
  for (int64_t f = (int64_t)blockIdx.x * kThreads + threadIdx.x; f < n_blk; f += (int64_t)gridDim.x * kThreads) {
    const uint2 c = *reinterpret_cast<const uint2*>(cb + f * 8);
    const float sv = e4m3_value_mag(sb[f]);
    if constexpr (BF16_OUT) {
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        uint32_t h2 = 0;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint32_t w = i + k < 8 ? c.x : c.y;
          const uint32_t q = (w >> (4 * ((i + k) & 7))) & 15u;
          const double d = (double)(e2m1_value_mag(q & 7u) * sv) * (double)S;  // exact: <= 30 significant bits
          const float t = __double2float_rz(d);
          const uint32_t u = f2u(t) | ((double)t != d ? 1u : 0u);  // round to odd at binary32
          const uint32_t hb = ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16) | ((q & 8u) ? 0x8000u : 0u);
          h2 |= hb << (16 * k);
        }
        o[i / 2] = h2;
      }
      uint4* op = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + ((int64_t)b * n_blk + f) * 16);
      op[0] = make_uint4(o[0], o[1], o[2], o[3]);
      op[1] = make_uint4(o[4], o[5], o[6], o[7]);
    } else {
      float o[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t w = i < 8 ? c.x : c.y;
        const uint32_t q = (w >> (4 * (i & 7))) & 15u;
        const float e = e2m1_value_mag(q & 7u) * sv;  // exact: <= 6 significant bits
        const float r = e * S;
        o[i] = (q & 8u) ? -r : r;
      }
      float4* op = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + ((int64_t)b * n_blk + f) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) op[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_fp8_rows(const void* __restrict__ x, int64_t C,
                                                        uint8_t* __restrict__ codes, float* __restrict__ scales,
                                                        _Float16* __restrict__ dec16) {
  __shared__ float lds[kThreads / 64];
  const int64_t r = blockIdx.x;
  const int64_t n4 = C / 4;
  auto load4 = [&](int64_t j, float* v) {
    if (BF16) {
      const uint2 w = *reinterpret_cast<const uint2*>((const uint16_t*)x + r * C + 4 * j);
      v[0] = u2f(w.x << 16);
      v[1] = u2f(w.x & 0xFFFF0000u);
      v[2] = u2f(w.y << 16);
      v[3] = u2f(w.y & 0xFFFF0000u);
    } else {
      const float4 q = *reinterpret_cast<const float4*>((const float*)x + r * C + 4 * j);
      v[0] = q.x;
      v[1] = q.y;
      v[2] = q.z;
      v[3] = q.w;
    }
  };
  // rows of up to kCache * 4 * kThreads values stay in registers between the amax and the encode pass
  constexpr int kCache = 8;
  const bool cached = n4 <= (int64_t)kCache * kThreads;
  float cv[kCache][4];
  float m = 0.0f;
  if (cached) {
#pragma unroll
    for (int q = 0; q < kCache; ++q) {
      const int64_t j = threadIdx.x + (int64_t)q * kThreads;
      if (j < n4) {
        load4(j, cv[q]);
        m = fmaxf(m, fmaxf(fmaxf(fabsf(cv[q][0]), fabsf(cv[q][1])), fmaxf(fabsf(cv[q][2]), fabsf(cv[q][3]))));
      }
    }
  } else {
    for (int64_t j = threadIdx.x; j < n4; j += kThreads) {
      float v[4];
      load4(j, v);
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    }
  }
  m = block_max(m, lds);
  const float s = m / 448.0f;
  if (threadIdx.x == 0) scales[r] = s;
  for (int64_t j = threadIdx.x, q = 0; j < n4; j += kThreads, ++q) {
    float v[4];
    if (cached) {
#pragma unroll
      for (int qq = 0; qq < kCache; ++qq)
        if (qq == q) {
          v[0] = cv[qq][0];
          v[1] = cv[qq][1];
          v[2] = cv[qq][2];
          v[3] = cv[qq][3];
        }
    } else {
      load4(j, v);
    }
    uint32_t word = 0;
    _Float16 d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t sgn = (f2u(v[i]) >> 31) << 7;
      const uint32_t mag = (s == 0.0f) ? 0u : e4m3_code_mag(fabsf(v[i]) / s);
      word |= (sgn | mag) << (8 * i);
      const float dv = e4m3_value_mag(mag);
      d[i] = (_Float16)(sgn ? -dv : dv);
    }
    *reinterpret_cast<uint32_t*>(codes + r * C + 4 * j) = word;
    if (dec16) *reinterpret_cast<uint2*>(dec16 + r * C + 4 * j) = __builtin_bit_cast(uint2, d);
  }
}

// Local Hessian blocks of the inputs x [N, C]: out[b][i][j] = sum_t x[t, 16b+i] x[t, 16b+j]
// (binary64, t ascending).  One thread per (b, i, j).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_local_hessian(const void* __restrict__ x, int64_t N, int64_t C,
                                                             double* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= (C / 16) * 256) return;
  const int64_t b = gid >> 8;
  const int i = (int)((gid >> 4) & 15), j = (int)(gid & 15);
  const int64_t ci = 16 * b + i, cj = 16 * b + j;
  double acc = 0.0;
  for (int64_t t = 0; t < N; ++t) {
    float a, c;
    if (BF16) {
      a = u2f((uint32_t)reinterpret_cast<const uint16_t*>(x)[t * C + ci] << 16);
      c = u2f((uint32_t)reinterpret_cast<const uint16_t*>(x)[t * C + cj] << 16);
    } else {
      a = reinterpret_cast<const float*>(x)[t * C + ci];
      c = reinterpret_cast<const float*>(x)[t * C + cj];
    }
    const double p = (double)a * (double)c;
    acc = acc + p;
  }
  out[gid] = acc;
}

// Local-Hessian block-scale search ("NVFP4 quantization" page, "Quantization
// method"): per 16-value block, among the E4M3 scale codes c0 - radius ..
// c0 + radius (c0 = round-to-nearest code, admissible codes 1..126) keep the
// one minimizing dw^T H_b dw, dw = w - q * s * S_g, evaluated in binary64 in a
// fixed order (t_i = sum_j H_ij dw_j, j ascending; e = sum_i dw_i t_i); ties go
// to the lower code.  The elements of a block quantize exactly as in the RTN
// encoder.  One thread per (block column b, row r); a wave shares b, so the
// 16 x 16 block of H is read once per wave.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_nvfp4_lh_encode(const void* __restrict__ w, int64_t R, int64_t C,
                                                               const double* __restrict__ hb,
                                                               const float* __restrict__ gs, int radius,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales) {
  const int64_t nb = C / 16;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= R * nb) return;
  const int64_t b = gid / R, r = gid % R;
  const int64_t f = r * nb + b;  // block index in the row-major block sequence
  float v[16];
  load16<BF16>(w, f, v);
  const float S = gs[0];
  const float d1 = 6.0f * S;
  float ab = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) ab = fmaxf(ab, fabsf(v[k]));
  const int c0 = (S != 0.0f) ? (int)e4m3_code_mag(ab / d1) : 0;
  int best = c0;
  if (c0 > 0) {
    const double* H = hb + b * 256;
    double best_e = __builtin_inf();
    for (int c = c0 - radius; c <= c0 + radius; ++c) {
      if (c < 1 || c > 126) continue;
      const float sv = e4m3_value_mag((uint32_t)c);
      const float d2 = sv * S;
      double dw[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint32_t mag = e2m1_code_mag(fabsf(v[k]) / d2);
        const double qm = (f2u(v[k]) >> 31) ? -(double)e2m1_value_mag(mag) : (double)e2m1_value_mag(mag);
        const double val = (qm * (double)sv) * (double)S;
        dw[k] = (double)v[k] - val;
      }
      double e = 0.0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        double t = 0.0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const double p = H[i * 16 + j] * dw[j];
          t = t + p;
        }
        const double p = dw[i] * t;
        e = e + p;
      }
      if (e < best_e) {
        best_e = e;
        best = c;
      }
    }
  }
  // encode with the chosen scale exactly as the RTN encoder does
  const float sv = e4m3_value_mag((uint32_t)best);
  const float d2 = sv * S;
  uint32_t q[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const uint32_t sgn = (f2u(v[k]) >> 31) << 3;
    const uint32_t mag = (sv == 0.0f) ? 0u : e2m1_code_mag(fabsf(v[k]) / d2);
    q[k] = sgn | mag;
  }
  uint2 packed;
  packed.x = q[0] | (q[1] << 4) | (q[2] << 8) | (q[3] << 12) | (q[4] << 16) | (q[5] << 20) | (q[6] << 24) |
             (q[7] << 28);
  packed.y = q[8] | (q[9] << 4) | (q[10] << 8) | (q[11] << 12) | (q[12] << 16) | (q[13] << 20) |
             (q[14] << 24) | (q[15] << 28);
  *reinterpret_cast<uint2*>(codes + f * 8) = packed;
  scales[f] = (uint8_t)best;
}

}  // namespace

int nvfp4_amax_parts(int64_t R, int64_t C) {
  const int64_t n_blk = R * C / 16;
  // one block per thread while that fits: small tensors (decode-sized x and h)
  // then cost one load latency instead of a serial chain of them
  int64_t p = (n_blk + kThreads - 1) / kThreads;
  if (p < 1) p = 1;
  if (p > kAmaxMaxParts) p = kAmaxMaxParts;
  return (int)p;
}

size_t nvfp4_quant_ws(int64_t B, int64_t, int64_t) { return align256((size_t)B * kAmaxMaxParts * sizeof(float)); }

static int encode_parts(int64_t n_blk, int64_t B) {
  int64_t p = (n_blk + kThreads - 1) / kThreads;
  if (p < 1) p = 1;
  const int64_t cap = B > 1 ? 256 : 4096;
  return (int)(p > cap ? cap : p);
}

hipError_t launch_nvfp4_quantize(const void* x, bool x_bf16, int64_t B, int64_t R, int64_t C, uint8_t* codes,
                                 uint8_t* scales, float* gs, bool dynamic, float* parts, hipStream_t st) {
  const int64_t n_blk = R * C / 16;
  if (n_blk == 0 || B == 0) return hipSuccess;
  const int np1 = nvfp4_amax_parts(R, C);
  if (dynamic) {
    dim3 g1(np1, (unsigned)B);
    if (x_bf16)
      k_amax_parts<true><<<g1, kThreads, 0, st>>>(x, n_blk, parts, np1);
    else
      k_amax_parts<false><<<g1, kThreads, 0, st>>>(x, n_blk, parts, np1);
  }
  const int np2 = encode_parts(n_blk, B);
  dim3 g2(np2, (unsigned)B);
  if (x_bf16)
    k_nvfp4_encode<true><<<g2, kThreads, 0, st>>>(x, n_blk, codes, scales, gs, parts, np1, nullptr, gs,
                                                   dynamic ? 0 : 1, np2, nullptr);
  else
    k_nvfp4_encode<false><<<g2, kThreads, 0, st>>>(x, n_blk, codes, scales, gs, parts, np1, nullptr, gs,
                                                    dynamic ? 0 : 1, np2, nullptr);
  return hipGetLastError();
}

hipError_t launch_nvfp4_quantize_from_amax(const void* x, bool x_bf16, int64_t B, int64_t R, int64_t C,
                                           uint8_t* codes, uint8_t* scales, float* gs, const uint32_t* amax_bits,
                                           const float* static_gs, hipStream_t st, _Float16* dec16) {
  const int64_t n_blk = R * C / 16;
  if (n_blk == 0 || B == 0) return hipSuccess;
  const int np2 = encode_parts(n_blk, B);
  dim3 g2(np2, (unsigned)B);
  if (x_bf16)
    k_nvfp4_encode<true><<<g2, kThreads, 0, st>>>(x, n_blk, codes, scales, gs, nullptr, 0, amax_bits, static_gs, 2,
                                                   np2, dec16);
  else
    k_nvfp4_encode<false><<<g2, kThreads, 0, st>>>(x, n_blk, codes, scales, gs, nullptr, 0, amax_bits, static_gs, 2,
                                                    np2, dec16);
  return hipGetLastError();
}

hipError_t launch_local_hessian(const void* x, bool x_bf16, int64_t N, int64_t C, double* out, hipStream_t st) {
  const int64_t n = (C / 16) * 256;
  if (n == 0) return hipSuccess;
  const unsigned g = (unsigned)((n + kThreads - 1) / kThreads);
  if (x_bf16)
    k_local_hessian<true><<<g, kThreads, 0, st>>>(x, N, C, out);
  else
    k_local_hessian<false><<<g, kThreads, 0, st>>>(x, N, C, out);
  return hipGetLastError();
}

hipError_t launch_nvfp4_quantize_lh(const void* w, bool w_bf16, int64_t R, int64_t C, const double* hb, int radius,
                                    uint8_t* codes, uint8_t* scales, float* gs, float* parts, hipStream_t st) {
  const int64_t nblk = R * (C / 16);
  if (nblk == 0) return hipSuccess;
  // round-to-nearest pass: the dynamic global scale (and a complete encoding the search then overwrites)
  hipError_t err = launch_nvfp4_quantize(w, w_bf16, 1, R, C, codes, scales, gs, true, parts, st);
  if (err != hipSuccess) return err;
  const unsigned g = (unsigned)((nblk + kThreads - 1) / kThreads);
  if (w_bf16)
    k_nvfp4_lh_encode<true><<<g, kThreads, 0, st>>>(w, R, C, hb, gs, radius, codes, scales);
  else
    k_nvfp4_lh_encode<false><<<g, kThreads, 0, st>>>(w, R, C, hb, gs, radius, codes, scales);
  return hipGetLastError();
}

hipError_t launch_nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* gs, int64_t B, int64_t R,
                                   int64_t C, bool bf16_out, void* out, hipStream_t st) {
  const int64_t n_blk = R * C / 16;
  if (n_blk == 0 || B == 0) return hipSuccess;
  int64_t p = (n_blk + kThreads * 4 - 1) / (kThreads * 4);
  if (p > 4096) p = 4096;
  dim3 g((unsigned)p, (unsigned)B);
  if (bf16_out)
    k_nvfp4_decode<true><<<g, kThreads, 0, st>>>(codes, scales, gs, n_blk, out);
  else
    k_nvfp4_decode<false><<<g, kThreads, 0, st>>>(codes, scales, gs, n_blk, out);
  return hipGetLastError();
}

hipError_t launch_fp8_quantize(const void* x, bool x_bf16, int64_t R, int64_t C, uint8_t* codes, float* scales,
                               hipStream_t st, _Float16* dec16) {
  if (R == 0) return hipSuccess;
  if (x_bf16)
    k_fp8_rows<true><<<(unsigned)R, kThreads, 0, st>>>(x, C, codes, scales, dec16);
  else
    k_fp8_rows<false><<<(unsigned)R, kThreads, 0, st>>>(x, C, codes, scales, dec16);
  return hipGetLastError();
}

}  // namespace bsm
