// bsm_moe.hip -- routed-expert MLP for gfx950: permutation, grouped gate/up
// GEMM with the SwiGLU product, re-quantization of h, grouped down GEMM and
// the weighted combine.
//
// Method: each expert is a SwiGLU MLP; expert outputs are combined with the
// normalized router weights and scaled by 2.5 ("Reflection releases Beam"
// news page, "Mixture-of-Experts details"); the SwiGLU product is computed in
// FP32 ("Residual stream and numerical decisions").  NVFP4 W4A4: both GEMM
// operands are E2M1 with E4M3 per-16 scales and a per-tensor global scale
// ("NVFP4 quantization" page, "Quantization scheme").  FP8_DYNAMIC W8A8:
// E4M3 operands, per-output-channel weight scales, per-token activation
// scales ("FP8 quantization" page, "Quantization scheme").
//
// Exactness of the NVFP4 operands on the matrix cores: a decoded element
// q * s_b has at most 6 significant bits (E2M1: 2, E4M3: 4) and lies in
// [2^-10, 2688], so it is exact in FP16.  The kernels decode codes and block
// scales to FP16 in registers and run v_mfma_f32_16x16x32_f16 with FP32
// accumulation; the two global scales multiply the FP32 accumulator in the
// epilogue.  The FP8 path feeds E4M3 codes straight to
// v_mfma_scale_f32_16x16x128_f8f6f4 (unit E8M0 scales) and applies the
// per-row x per-column scales as a rank-1 epilogue.
//
// Pipeline (all on the caller's stream, no host synchronization):
//   k_perm_masks   per 64-token chunk and expert: ballot mask of the tokens
//                  that selected the expert
//   k_perm_scan    per expert: prefix counts over chunks, counts, offsets,
//                  16-row tile work list; clears the h amax word
//   k_perm_rows    row of every (token, slot) pair: rows of an expert are in
//                  token order (stable)
//   k_gemm1_*      one wave = 16 rows x (16 gate + 16 up) columns over all of
//                  H; epilogue h = silu(g) * u, FP32 h to the workspace, wave
//                  max |h| into one atomicMax word (order independent)
//   h quantize     NVFP4 with one global scale over all rows / FP8 per row
//   k_gemm2_*      one wave = 16 rows x 32 output columns over all of I
//   k_combine      out[t] = scale * sum_j w[t,j] * y[row(t,j)] (binary64 sum)
//
// Rows of an expert are split into 16-row tiles; the grid is sized for the
// largest possible tile count (P/16 + E) and workgroups beyond the device-side
// tile count exit at once.

#include "bsm_internal.h"

namespace bsm {

namespace {

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef int i8v __attribute__((ext_vector_type(8)));

constexpr int kRowsPerTile = 16;
constexpr int kChunk = 64;  // tokens per permutation chunk

// FP16 high bytes of the E2M1 magnitudes {0, .5, 1, 1.5 | 2, 3, 4, 6}
constexpr uint32_t kLutLo = 0x3E3C3800u;
constexpr uint32_t kLutHi = 0x46444240u;

__device__ inline uint32_t pack_pair(uint32_t hbe, uint32_t hbo, uint32_t j) {
  // bytes [0, hbe_j, 0, hbo_j]: FP16 (even element) low half, (odd element) high half
  // selector bytes (LSB first): 0x0C -> 0x00, j -> byte j of hbe, 4+j -> byte j of hbo
  return __builtin_amdgcn_perm(hbo, hbe, 0x000C000Cu | (j << 8) | ((4u + j) << 24));
}

// 8 E2M1 codes (element i in nibble i of w) times the block scale, as FP16 (exact).
__device__ inline h8v decode8(uint32_t w, h2v s2) {
  const uint32_t ev = w & 0x0F0F0F0Fu;
  const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t hbe = __builtin_amdgcn_perm(kLutHi, kLutLo, ev & 0x07070707u) | ((ev & 0x08080808u) << 4);
  const uint32_t hbo = __builtin_amdgcn_perm(kLutHi, kLutLo, od & 0x07070707u) | ((od & 0x08080808u) << 4);
  h8v r;
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j) {
    const h2v p = __builtin_bit_cast(h2v, pack_pair(hbe, hbo, j)) * s2;
    r[2 * j] = p[0];
    r[2 * j + 1] = p[1];
  }
  return r;
}

__device__ inline h2v scale_pair(uint32_t code) {
  const _Float16 s = (_Float16)e4m3_value_mag(code);  // exact in FP16
  return h2v{s, s};
}

__device__ inline f4v mfma_f16(h8v a, h8v b, f4v c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

__device__ inline f4v mfma_fp8(i8v a, i8v b, f4v c) {
  // E4M3 x E4M3 (format 0 for both operands), unit E8M0 block scales (127)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ inline float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// 32 NVFP4 values (16 code bytes + 2 scale bytes) -> 4 FP16 octets, k order preserved
struct Nv32 {
  h8v q[4];
};
__device__ inline Nv32 load_nv32(const uint8_t* codes, const uint8_t* scales) {
  const uint4 c = *reinterpret_cast<const uint4*>(codes);
  const uint32_t s = *reinterpret_cast<const uint16_t*>(scales);
  const h2v s0 = scale_pair(s & 0xFFu), s1 = scale_pair(s >> 8);
  Nv32 r;
  r.q[0] = decode8(c.x, s0);
  r.q[1] = decode8(c.y, s0);
  r.q[2] = decode8(c.z, s1);
  r.q[3] = decode8(c.w, s1);
  return r;
}

__device__ inline i8v load_fp8_32(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
  return i8v{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

__device__ inline float silu_mul(float g, float u) { return (g / (1.0f + expf(-g))) * u; }

// ---------------------------------------------------------------------------
// permutation
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_perm_masks(const int32_t* __restrict__ ids, int64_t T, int topk, int64_t E,
                                                   int64_t nc, uint64_t* __restrict__ masks,
                                                   int* __restrict__ cnt) {
  const int64_t c = blockIdx.x;
  const int64_t t = c * kChunk + threadIdx.x;
  int my[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) my[j] = (t < T && j < topk) ? ids[t * topk + j] : -1;
  for (int64_t e = 0; e < E; ++e) {
    bool hit = false;
#pragma unroll
    for (int j = 0; j < 32; ++j) hit |= (my[j] == (int)e);
    const uint64_t m = __ballot(hit);
    if (threadIdx.x == (e & 63)) {
      masks[e * nc + c] = m;
      cnt[e * nc + c] = __popcll(m);
    }
  }
}

__global__ __launch_bounds__(1024) void k_perm_scan(const int* __restrict__ cnt, int64_t E, int64_t nc,
                                                    int* __restrict__ base, int* __restrict__ counts,
                                                    int* __restrict__ offsets, int4* __restrict__ tiles,
                                                    int* __restrict__ ntiles, uint32_t* __restrict__ h_amax) {
  __shared__ int s_cnt[1024];
  __shared__ int s_tl[1024];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
    for (int64_t c = 0; c < nc; ++c) {
      base[e * nc + c] = total;
      total += cnt[e * nc + c];
    }
    counts[e] = total;
  }
  s_cnt[e] = (e < E) ? total : 0;
  s_tl[e] = (e < E) ? (total + kRowsPerTile - 1) / kRowsPerTile : 0;
  __syncthreads();
  // inclusive scans (Hillis-Steele) over experts
  for (int o = 1; o < 1024; o <<= 1) {
    const int a = (e >= o) ? s_cnt[e - o] : 0;
    const int b = (e >= o) ? s_tl[e - o] : 0;
    __syncthreads();
    s_cnt[e] += a;
    s_tl[e] += b;
    __syncthreads();
  }
  if (e < E) {
    const int off = s_cnt[e] - total;
    const int nt = (total + kRowsPerTile - 1) / kRowsPerTile;
    const int toff = s_tl[e] - nt;
    offsets[e] = off;
    if (e == E - 1) {
      offsets[E] = s_cnt[e];
      *ntiles = s_tl[e];
    }
    for (int i = 0; i < nt; ++i) {
      const int r = total - i * kRowsPerTile;
      tiles[toff + i] = make_int4(e, off + i * kRowsPerTile, r < kRowsPerTile ? r : kRowsPerTile, 0);
    }
  }
  if (e == 0) *h_amax = 0u;
}

__global__ __launch_bounds__(256) void k_perm_rows(const int32_t* __restrict__ ids, int64_t P, int topk, int64_t nc,
                                                   const uint64_t* __restrict__ masks, const int* __restrict__ base,
                                                   const int* __restrict__ offsets, int* __restrict__ row_pair,
                                                   int* __restrict__ pair_row) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= P) return;
  const int64_t t = p / topk;
  const int e = ids[p];
  const int64_t c = t / kChunk;
  const uint32_t bit = (uint32_t)(t % kChunk);
  const uint64_t below = bit ? (masks[e * nc + c] & ((1ull << bit) - 1ull)) : 0ull;
  const int pos = offsets[e] + base[e * nc + c] + __popcll(below);
  row_pair[pos] = (int)p;
  pair_row[p] = pos;
}

// ---------------------------------------------------------------------------
// NVFP4 grouped GEMMs
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gemm1_nvfp4(const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                                     const float* __restrict__ xgs, const uint8_t* __restrict__ wc,
                                                     const uint8_t* __restrict__ wsc, const float* __restrict__ wgs,
                                                     const int4* __restrict__ tiles, const int* __restrict__ ntiles,
                                                     const int* __restrict__ row_pair, int topk, int64_t H,
                                                     int64_t I, float* __restrict__ h_out,
                                                     uint32_t* __restrict__ h_amax) {
  if ((int)blockIdx.y >= *ntiles) return;
  const int4 ti = tiles[blockIdx.y];
  const int e = ti.x, row0 = ti.y, nrows = ti.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n0 = ((int64_t)blockIdx.x * 4 + wave) * 16;
  const int m = lane & 15, g = lane >> 4;
  const int t = row_pair[row0 + (m < nrows ? m : 0)] / topk;
  const uint8_t* ac = xc + (int64_t)t * (H / 2) + 16 * g;
  const uint8_t* as = xs + (int64_t)t * (H / 16) + 2 * g;
  const int64_t rg = (int64_t)e * 2 * I + n0 + m, ru = rg + I;
  const uint8_t* gc = wc + rg * (H / 2) + 16 * g;
  const uint8_t* gs = wsc + rg * (H / 16) + 2 * g;
  const uint8_t* uc = wc + ru * (H / 2) + 16 * g;
  const uint8_t* us = wsc + ru * (H / 16) + 2 * g;
  f4v accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = 0; k0 < H; k0 += 128) {
    const int64_t cb = k0 / 2, sb = k0 / 16;
    const Nv32 a = load_nv32(ac + cb, as + sb);
    const Nv32 bg = load_nv32(gc + cb, gs + sb);
    const Nv32 bu = load_nv32(uc + cb, us + sb);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      accg = mfma_f16(a.q[s], bg.q[s], accg);
      accu = mfma_f16(a.q[s], bu.q[s], accu);
    }
  }
  const float sg = xgs[0] * wgs[2 * e], su = xgs[0] * wgs[2 * e + 1];
  float hmax = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ro = 4 * g + r;
    if (ro < nrows) {
      const float h = silu_mul(accg[r] * sg, accu[r] * su);
      h_out[(int64_t)(row0 + ro) * I + n0 + m] = h;
      hmax = fmaxf(hmax, fabsf(h));
    }
  }
  hmax = wave_max_f(hmax);
  if (lane == 0) atomicMax(h_amax, f2u(hmax));
}

__global__ __launch_bounds__(256) void k_gemm2_nvfp4(const uint8_t* __restrict__ hc, const uint8_t* __restrict__ hs,
                                                     const float* __restrict__ hgs, const uint8_t* __restrict__ wc,
                                                     const uint8_t* __restrict__ wsc, const float* __restrict__ wgs,
                                                     const int4* __restrict__ tiles, const int* __restrict__ ntiles,
                                                     int64_t H, int64_t I, float* __restrict__ y) {
  if ((int)blockIdx.y >= *ntiles) return;
  const int4 ti = tiles[blockIdx.y];
  const int e = ti.x, row0 = ti.y, nrows = ti.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n0 = ((int64_t)blockIdx.x * 4 + wave) * 32;
  const int m = lane & 15, g = lane >> 4;
  const int64_t ar = row0 + (m < nrows ? m : 0);
  const uint8_t* ac = hc + ar * (I / 2) + 16 * g;
  const uint8_t* as = hs + ar * (I / 16) + 2 * g;
  const int64_t r0 = (int64_t)e * H + n0 + m, r1 = r0 + 16;
  const uint8_t* b0c = wc + r0 * (I / 2) + 16 * g;
  const uint8_t* b0s = wsc + r0 * (I / 16) + 2 * g;
  const uint8_t* b1c = wc + r1 * (I / 2) + 16 * g;
  const uint8_t* b1s = wsc + r1 * (I / 16) + 2 * g;
  f4v acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = 0; k0 < I; k0 += 128) {
    const int64_t cb = k0 / 2, sb = k0 / 16;
    const Nv32 a = load_nv32(ac + cb, as + sb);
    const Nv32 b0 = load_nv32(b0c + cb, b0s + sb);
    const Nv32 b1 = load_nv32(b1c + cb, b1s + sb);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      acc0 = mfma_f16(a.q[s], b0.q[s], acc0);
      acc1 = mfma_f16(a.q[s], b1.q[s], acc1);
    }
  }
  const float sc = hgs[0] * wgs[e];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ro = 4 * g + r;
    if (ro < nrows) {
      float* yr = y + (int64_t)(row0 + ro) * H + n0 + m;
      yr[0] = acc0[r] * sc;
      yr[16] = acc1[r] * sc;
    }
  }
}

// ---------------------------------------------------------------------------
// FP8 grouped GEMMs
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gemm1_fp8(const uint8_t* __restrict__ xc, const float* __restrict__ xs,
                                                   const uint8_t* __restrict__ wc, const float* __restrict__ wsc,
                                                   const int4* __restrict__ tiles, const int* __restrict__ ntiles,
                                                   const int* __restrict__ row_pair, int topk, int64_t H, int64_t I,
                                                   float* __restrict__ h_out) {
  if ((int)blockIdx.y >= *ntiles) return;
  const int4 ti = tiles[blockIdx.y];
  const int e = ti.x, row0 = ti.y, nrows = ti.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n0 = ((int64_t)blockIdx.x * 4 + wave) * 16;
  const int m = lane & 15, g = lane >> 4;
  const int t = row_pair[row0 + (m < nrows ? m : 0)] / topk;
  const uint8_t* ap = xc + (int64_t)t * H + 32 * g;
  const int64_t rg = (int64_t)e * 2 * I + n0 + m, ru = rg + I;
  const uint8_t* gp = wc + rg * H + 32 * g;
  const uint8_t* up = wc + ru * H + 32 * g;
  f4v accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = 0; k0 < H; k0 += 128) {
    const i8v a = load_fp8_32(ap + k0);
    accg = mfma_fp8(a, load_fp8_32(gp + k0), accg);
    accu = mfma_fp8(a, load_fp8_32(up + k0), accu);
  }
  const float swg = wsc[rg], swu = wsc[ru];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ro = 4 * g + r;
    if (ro < nrows) {
      const float sx = xs[row_pair[row0 + ro] / topk];
      h_out[(int64_t)(row0 + ro) * I + n0 + m] = silu_mul(accg[r] * sx * swg, accu[r] * sx * swu);
    }
  }
}

__global__ __launch_bounds__(256) void k_gemm2_fp8(const uint8_t* __restrict__ hc, const float* __restrict__ hs,
                                                   const uint8_t* __restrict__ wc, const float* __restrict__ wsc,
                                                   const int4* __restrict__ tiles, const int* __restrict__ ntiles,
                                                   int64_t H, int64_t I, float* __restrict__ y) {
  if ((int)blockIdx.y >= *ntiles) return;
  const int4 ti = tiles[blockIdx.y];
  const int e = ti.x, row0 = ti.y, nrows = ti.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n0 = ((int64_t)blockIdx.x * 4 + wave) * 32;
  const int m = lane & 15, g = lane >> 4;
  const int64_t ar = row0 + (m < nrows ? m : 0);
  const uint8_t* ap = hc + ar * I + 32 * g;
  const int64_t r0 = (int64_t)e * H + n0 + m, r1 = r0 + 16;
  const uint8_t* b0 = wc + r0 * I + 32 * g;
  const uint8_t* b1 = wc + r1 * I + 32 * g;
  f4v acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = 0; k0 < I; k0 += 128) {
    const i8v a = load_fp8_32(ap + k0);
    acc0 = mfma_fp8(a, load_fp8_32(b0 + k0), acc0);
    acc1 = mfma_fp8(a, load_fp8_32(b1 + k0), acc1);
  }
  const float s0 = wsc[r0], s1 = wsc[r1];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ro = 4 * g + r;
    if (ro < nrows) {
      const float sa = hs[row0 + ro];
      float* yr = y + (int64_t)(row0 + ro) * H + n0 + m;
      yr[0] = acc0[r] * sa * s0;
      yr[16] = acc1[r] * sa * s1;
    }
  }
}

// ---------------------------------------------------------------------------
// combine
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y, const int* __restrict__ pair_row,
                                                 const float* __restrict__ wts, int topk, int64_t H, double scale,
                                                 float* __restrict__ out) {
  const int64_t t = blockIdx.y;
  const int64_t c4 = (int64_t)blockIdx.x * 256 + threadIdx.x;  // float4 column index
  if (c4 * 4 >= H) return;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int j = 0; j < topk; ++j) {
    const double w = (double)wts[t * topk + j];
    const float4 v = *reinterpret_cast<const float4*>(y + (int64_t)pair_row[t * topk + j] * H + c4 * 4);
    acc[0] += w * (double)v.x;
    acc[1] += w * (double)v.y;
    acc[2] += w * (double)v.z;
    acc[3] += w * (double)v.w;
  }
  *reinterpret_cast<float4*>(out + t * H + c4 * 4) =
      make_float4((float)(scale * acc[0]), (float)(scale * acc[1]), (float)(scale * acc[2]), (float)(scale * acc[3]));
}

__global__ void k_copy_f32(const float* src, float* dst) {
  if (threadIdx.x == 0) dst[0] = src[0];
}

}  // namespace

MoeLayout moe_layout(bool nvfp4, int64_t E, int64_t H, int64_t I, int64_t T, int topk) {
  MoeLayout L{};
  L.P = T * topk;
  L.n_chunks = (T + kChunk - 1) / kChunk;
  L.max_tiles = L.P / kRowsPerTile + E + 1;
  size_t o = 0;
  auto take = [&](size_t n) {
    const size_t r = o;
    o += align256(n);
    return r;
  };
  L.counts = take(sizeof(int) * E);
  L.offsets = take(sizeof(int) * (E + 1));
  L.row_pair = take(sizeof(int) * L.P);
  L.pair_row = take(sizeof(int) * L.P);
  L.tiles = take(sizeof(int4) * L.max_tiles);
  L.h_f32 = take(sizeof(float) * L.P * I);
  L.h_codes = take(nvfp4 ? (size_t)L.P * I / 2 : (size_t)L.P * I);
  L.h_scales = take(nvfp4 ? (size_t)L.P * I / 16 : sizeof(float) * L.P);
  L.h_gs = take(sizeof(float));
  L.y_f32 = take(sizeof(float) * L.P * H);
  L.scratch = o;
  L.sel_masks = take(sizeof(uint64_t) * E * L.n_chunks);
  L.chunk_cnt = take(sizeof(int) * E * L.n_chunks);
  L.chunk_base = take(sizeof(int) * E * L.n_chunks);
  L.ntiles = take(sizeof(int));
  L.h_amax = take(sizeof(uint32_t));
  L.total = o;
  return L;
}

hipError_t launch_moe(const MoeArgs& a, hipStream_t st) {
  const MoeLayout L = moe_layout(a.nvfp4, a.E, a.H, a.I, a.T, a.topk);
  if (a.T == 0) return hipSuccess;
  uint8_t* ws = a.ws;
  int* counts = reinterpret_cast<int*>(ws + L.counts);
  int* offsets = reinterpret_cast<int*>(ws + L.offsets);
  int* row_pair = reinterpret_cast<int*>(ws + L.row_pair);
  int* pair_row = reinterpret_cast<int*>(ws + L.pair_row);
  int4* tiles = reinterpret_cast<int4*>(ws + L.tiles);
  float* h_f32 = reinterpret_cast<float*>(ws + L.h_f32);
  uint8_t* h_codes = ws + L.h_codes;
  uint8_t* h_scales = ws + L.h_scales;
  float* h_gs = reinterpret_cast<float*>(ws + L.h_gs);
  float* y = reinterpret_cast<float*>(ws + L.y_f32);
  uint64_t* masks = reinterpret_cast<uint64_t*>(ws + L.sel_masks);
  int* ccnt = reinterpret_cast<int*>(ws + L.chunk_cnt);
  int* cbase = reinterpret_cast<int*>(ws + L.chunk_base);
  int* ntiles = reinterpret_cast<int*>(ws + L.ntiles);
  uint32_t* h_amax = reinterpret_cast<uint32_t*>(ws + L.h_amax);

  k_perm_masks<<<(unsigned)L.n_chunks, 64, 0, st>>>(a.ids, a.T, a.topk, a.E, L.n_chunks, masks, ccnt);
  k_perm_scan<<<1, 1024, 0, st>>>(ccnt, a.E, L.n_chunks, cbase, counts, offsets, tiles, ntiles, h_amax);
  k_perm_rows<<<(unsigned)((L.P + 255) / 256), 256, 0, st>>>(a.ids, L.P, a.topk, L.n_chunks, masks, cbase, offsets,
                                                              row_pair, pair_row);
  const dim3 g1((unsigned)(a.I / 64), (unsigned)L.max_tiles);
  const dim3 g2((unsigned)(a.H / 128), (unsigned)L.max_tiles);
  hipError_t err;
  if (a.nvfp4) {
    k_gemm1_nvfp4<<<g1, 256, 0, st>>>(a.x_codes, reinterpret_cast<const uint8_t*>(a.x_scales), a.x_gs, a.w13_codes,
                                       reinterpret_cast<const uint8_t*>(a.w13_scales), a.w13_gs, tiles, ntiles,
                                       row_pair, a.topk, a.H, a.I, h_f32, h_amax);
    err = launch_nvfp4_quantize_from_amax(h_f32, false, 1, L.P, a.I, h_codes, h_scales, h_gs, h_amax,
                                          a.h_static ? a.h_gs_user : nullptr, st);
    if (err != hipSuccess) return err;
    if (!a.h_static && a.h_gs_user) k_copy_f32<<<1, 64, 0, st>>>(h_gs, a.h_gs_user);
    k_gemm2_nvfp4<<<g2, 256, 0, st>>>(h_codes, h_scales, h_gs, a.w2_codes,
                                       reinterpret_cast<const uint8_t*>(a.w2_scales), a.w2_gs, tiles, ntiles, a.H,
                                       a.I, y);
  } else {
    k_gemm1_fp8<<<g1, 256, 0, st>>>(a.x_codes, reinterpret_cast<const float*>(a.x_scales), a.w13_codes,
                                     reinterpret_cast<const float*>(a.w13_scales), tiles, ntiles, row_pair, a.topk,
                                     a.H, a.I, h_f32);
    err = launch_fp8_quantize(h_f32, false, L.P, a.I, h_codes, reinterpret_cast<float*>(h_scales), st);
    if (err != hipSuccess) return err;
    k_gemm2_fp8<<<g2, 256, 0, st>>>(h_codes, reinterpret_cast<const float*>(h_scales), a.w2_codes,
                                     reinterpret_cast<const float*>(a.w2_scales), tiles, ntiles, a.H, a.I, y);
  }
  const dim3 gc((unsigned)((a.H / 4 + 255) / 256), (unsigned)a.T);
  k_combine<<<gc, 256, 0, st>>>(y, pair_row, a.wts, a.topk, a.H, (double)a.combine_scale, a.out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RMSNorm and residual
// ---------------------------------------------------------------------------
namespace {
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ x, int64_t H, float eps,
                                                 float* __restrict__ y) {
  __shared__ double part[4];
  const int64_t t = blockIdx.x;
  const float* xr = x + t * H;
  double ss = 0.0;
  for (int64_t k = threadIdx.x; k < H; k += 256) {
    const double v = (double)xr[k];
    ss += v * v;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const double tot = ((part[0] + part[1]) + part[2]) + part[3];
  const float ms = (float)(tot / (double)H);
  const float r = (float)(1.0 / sqrt((double)ms + (double)eps));
  for (int64_t k = threadIdx.x; k < H; k += 256) y[t * H + k] = xr[k] * r;
}

__global__ __launch_bounds__(256) void k_residual(float* __restrict__ x, const float* __restrict__ m, double a,
                                                  double b, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = (float)(a * (double)x[i] + b * (double)m[i]);
}
}  // namespace

hipError_t launch_rmsnorm(const float* x, int64_t T, int64_t H, float eps, float* y, hipStream_t st) {
  if (T == 0) return hipSuccess;
  k_rmsnorm<<<(unsigned)T, 256, 0, st>>>(x, H, eps, y);
  return hipGetLastError();
}

hipError_t launch_residual(float* x, const float* m, float a, float b, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  k_residual<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(x, m, (double)a, (double)b, n);
  return hipGetLastError();
}

}  // namespace bsm
