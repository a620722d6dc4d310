// bsm_moe.hip -- routed-expert MLP for gfx950: permutation, grouped gate/up
// GEMM with the SwiGLU product, re-quantization of h, grouped down GEMM and
// the weighted combine.
//
// Method: the experts are SwiGLU MLPs; the layer output adds up the chosen
// experts' outputs, each weighted by its router score over the sum of the
// chosen scores, and multiplies the total by 2.5 ("Reflection releases Beam"
// news page, "Mixture-of-Experts details"); the SwiGLU product is computed in
// FP32 ("Residual stream and numerical decisions").  NVFP4 W4A4: both GEMM
// operands are E2M1 with E4M3 per-16 scales and a per-tensor global scale
// ("NVFP4 quantization" page, "Quantization scheme").  FP8_DYNAMIC W8A8:
// E4M3 operands, per-output-channel weight scales, per-token activation
// scales ("FP8 quantization" page, "Quantization scheme").
//
// Exactness of the operands on the matrix cores: a decoded NVFP4 element
// q * s_b has at most 6 significant bits (E2M1: 2, E4M3: 4) and lies in
// [2^-10, 2688]; an E4M3 element has 4 significant bits and lies in
// [2^-9, 448].  Both are exact in FP16, so the GEMMs decode their operands to
// FP16 (weight-only W4A16: BF16) and run FP16 MFMA with FP32 accumulation
// (16x16x32 in the few-row kernels, 32x32x16 in the many-row one); the global
// scales (NVFP4) or the per-row x per-column scales (FP8) multiply the FP32
// accumulator in the epilogue.  gfx950's FP8/FP4 matrix cores are not used:
// their scaled MFMA adds each group of products with a fixed-point alignment
// to the largest one, which is not an FP32 accumulation.
//
// Pipeline (all on the caller's stream, no host synchronization):
//   k_perm_masks   per 64-token chunk: LDS bit mask of the chunk's tokens for
//                  every expert (atomicOr, order independent) and its popcount
//   k_perm_scan    per expert: prefix counts over chunks, counts, offsets, and
//                  two device-side tile lists: experts with <= 32 rows get
//                  16-row tiles (skinny kernels), larger ones 128-row tiles
//                  (many-row kernels); clears the h amax word
//   k_perm_rows    row of every (token, slot) pair; rows of an expert are in
//                  token order (stable)
//   k_perm_small   all three in one workgroup when the batch is one chunk
//                  (at most 64 tokens: every expert, up to 64 rows, in 16-row tiles)
//   k_decode_act   activation codes -> FP16 q * s_b (once per call), where a
//                  GEMM reads FP16 activations: NVFP4 gate/up with many-row
//                  experts, K not a multiple of the few-row super-step
//                  (k_skinny), the dense FP8 linear
//   k_skinny_rows<G1> (k_skinny<G1> when K is not a multiple of the super-step)
//                  gate/up for 16-row tiles: epilogue h = silu(g) * u (FP32)
//                  to the workspace, max |h| into one atomicMax word (order
//                  independent)
//   k_gemm_big<G1> the same for 128-row tiles (128 x 256 per workgroup,
//                  32x32x16 MFMA; k_gemm_wide is the 16x16x32 fallback)
//   k_dense_f8<G1> FP8 with one expert and at most 64 rows (dense layers)
//   h quantize     NVFP4 with one global scale over all rows / FP8 per row
//                  (plus an FP16 decoded copy only for k_skinny and k_gemm_wide,
//                  the fallbacks for I not a multiple of 512 or 256)
//   k_skinny_rows<!G1> / k_skinny<!G1>, k_gemm_big<!G1> (k_gemm_wide when
//                  I % 256 != 0): down projection -> y (FP32)
//   k_combine      out[t] = scale * sum_j w[t,j] * y[row(t,j)] (binary64 sum
//                  in slot order, rounded once)
//
// The grids are sized for the largest possible tile counts and workgroups
// beyond the device-side tile count exit at once.

#include <algorithm>

#include "bsm_internal.h"

namespace bsm {

namespace {

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kRowsPerTile = 16;
constexpr int kChunk = 64;  // tokens per permutation chunk
// Few-row (skinny) kernels: each wave owns kSkNT tiles of 16 weight rows; K is walked in super-steps of
// 4 x kNvKB (NVFP4) or 4 x kF8KB (FP8) values; FP8 keeps kSkDepthF8 super-steps of codes in flight per
// lane (NVFP4 one).  Measured at decode-64: NVFP4 gate/up 0.62 ms at depth 1 against 0.66 ms at depth 2
// (occupancy 3 -> 2 workgroups per CU); FP8 1.01 -> 0.995 ms with depth 2.
constexpr int kSkNT = 2;
constexpr int kNvKB = 128;
constexpr int kF8KB = 64;
constexpr int kSkDepthF8 = 2;

// FP16 high bytes of the E2M1 magnitudes {0, .5, 1, 1.5 | 2, 3, 4, 6}
__device__ inline h2v scale_pair(uint32_t code) {
  const _Float16 s = (_Float16)e4m3_value_mag(code);  // exact in FP16
  return h2v{s, s};
}

// (s, s) in FP16 for E4M3 scale byte K of w, through the hardware FP8 -> FP16
// converter (exact; unit scale): the byte is replicated into the low two bytes.
template <int K>
__device__ inline h2v scale_pair_hw(uint32_t w) {
  const uint32_t rep = __builtin_amdgcn_perm(w, w, (uint32_t)(K | (K << 8)));
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(rep, 1.0f, false);
}

__device__ inline f4v mfma_f16(h8v a, h8v b, f4v c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// Weight-only (W4A16) operands: BF16 bits carried in the same 8 x 16-bit containers.
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef float f2v __attribute__((ext_vector_type(2)));
template <bool A16>
__device__ inline f4v mfma_ab(h8v a, h8v b, f4v c) {
  if constexpr (A16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, a), __builtin_bit_cast(bf8v, b), c, 0, 0, 0);
  else
    return mfma_f16(a, b, c);
}

__device__ inline float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// SwiGLU product h = silu(g) * u = g * u / (1 + e^-g) in binary32: e^-g as 2^(-g log2 e) on the
// hardware exp2, and the hardware reciprocal (1 ulp each; the product is within a few ulp of the
// exactly rounded value).  Large negative g gives 2^x = inf, a reciprocal of 0 and h = +-0.
__device__ inline float silu_mul(float g, float u) {
  const float t = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return (g * u) * __builtin_amdgcn_rcpf(1.0f + t);
}

// max |h| of a 256-thread workgroup into the global amax word with one atomic (order independent).
// One atomic per wave had cost the decode gate/up GEMM about 16 us of contention on that word.
__device__ inline void wg_amax_atomic(float hmax, uint32_t* h_amax) {
  __shared__ float s_m[4];
  hmax = wave_max_f(hmax);
  if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = hmax;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(h_amax, f2u(fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]))));
}

// ---------------------------------------------------------------------------
// permutation
// ---------------------------------------------------------------------------
// One workgroup per 64-token chunk: every (token, slot) pair ORs its token bit
// into the chunk's LDS mask of its expert (order independent), then the masks
// ([expert][chunk]) and their popcounts ([chunk][expert], so that the scan's
// loads of one chunk are contiguous over the experts) are written out.
__global__ __launch_bounds__(256) void k_perm_masks(const int32_t* __restrict__ ids, int64_t T, int topk, int64_t E,
                                                    int64_t nc, uint64_t* __restrict__ masks,
                                                    int* __restrict__ cnt) {
  __shared__ unsigned long long lm[1024];
  const int64_t c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) lm[e] = 0ull;
  __syncthreads();
  const int64_t t0 = c * kChunk;
  const int64_t tn = (T - t0) < kChunk ? (T - t0) : kChunk;
  for (int64_t i = threadIdx.x; i < tn * topk; i += 256) {
    const int64_t t = t0 + i / topk;
    const int e = ids[t0 * topk + i];
    if ((uint32_t)e < (uint32_t)E) atomicOr(&lm[e], 1ull << (t - t0));  // ids outside [0, E) are dropped
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    const uint64_t m = lm[e];
    masks[e * nc + c] = m;
    cnt[c * E + e] = __popcll(m);
  }
}

// experts with more rows use the wide kernel; up to 4 row tiles of one expert
// run side by side on one XCD (consecutive grid rows), so their weight
// re-reads hit L2
constexpr int kSkinnyMaxRows = 64;
constexpr int kWideRows = 128;
// With several permutation chunks (the many-row kernel runs), experts of 33..64 rows go to it as well:
// two live 32-row sub-tiles of the many-row kernel measured faster than four 16-row few-row tiles
// (prefill-8192 NVFP4 5.59 -> 5.52 ms, FP8 6.28 -> 6.20 ms; a threshold of 16 gave the same).
constexpr int kFewRowsMulti = 32;

// Inclusive prefix sums of three per-thread counts over the 1024 threads of a workgroup (thread i's
// values are item i's): within each wave by shuffles, then each wave adds the totals of the waves before
// it from LDS.  One barrier instead of one pair per doubling step.
__device__ inline void block_scan3_1024(int& a, int& b, int& c, int (*wt)[3]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ya = __shfl_up(a, o, 64), yb = __shfl_up(b, o, 64), yc = __shfl_up(c, o, 64);
    if (lane >= o) {
      a += ya;
      b += yb;
      c += yc;
    }
  }
  if (lane == 63) {
    wt[wv][0] = a;
    wt[wv][1] = b;
    wt[wv][2] = c;
  }
  __syncthreads();
  for (int w = 0; w < wv; ++w) {
    a += wt[w][0];
    b += wt[w][1];
    c += wt[w][2];
  }
}

__global__ __launch_bounds__(1024) void k_perm_scan(const int* __restrict__ cnt, int64_t E, int64_t nc,
                                                    int* __restrict__ base, int* __restrict__ counts,
                                                    int* __restrict__ offsets, int4* __restrict__ tiles_s,
                                                    int* __restrict__ ntiles_s, int4* __restrict__ tiles_w,
                                                    int* __restrict__ ntiles_w, uint32_t* __restrict__ h_amax) {
  __shared__ int wtot[16][3];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
    // 32 chunk counts in flight per batch (independent loads, clamped in range), then their prefix
    // counts and bases are [chunk][expert]: each load and store of a wave covers 64 consecutive experts
    for (int64_t c0 = 0; c0 < nc; c0 += 32) {
      int v[32];
#pragma unroll
      for (int q = 0; q < 32; ++q) v[q] = cnt[(c0 + q < nc ? c0 + q : nc - 1) * E + e];
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        if (c0 + q < nc) {
          base[(c0 + q) * E + e] = total;
          total += v[q];
        }
      }
    }
    counts[e] = total;
  }
  const bool skinny = total <= kFewRowsMulti;
  const int nts = (e < E && skinny) ? (total + kRowsPerTile - 1) / kRowsPerTile : 0;
  const int ntw = (e < E && !skinny) ? (total + kWideRows - 1) / kWideRows : 0;
  int sc = (e < E) ? total : 0, st = nts, sw = ntw;
  block_scan3_1024(sc, st, sw, wtot);
  if (e < E) {
    const int off = sc - total;
    offsets[e] = off;
    if (e == E - 1) {
      offsets[E] = sc;
      *ntiles_s = st;
      *ntiles_w = sw;
    }
    const int ts0 = st - nts, tw0 = sw - ntw;
    for (int i = 0; i < nts; ++i) {
      const int r = total - i * kRowsPerTile;
      tiles_s[ts0 + i] = make_int4(e, off + i * kRowsPerTile, r < kRowsPerTile ? r : kRowsPerTile, 0);
    }
    for (int i = 0; i < ntw; ++i) {
      const int r = total - i * kWideRows;
      tiles_w[tw0 + i] = make_int4(e, off + i * kWideRows, r < kWideRows ? r : kWideRows, 0);
    }
  }
  if (e == 0) *h_amax = 0u;
}

__global__ __launch_bounds__(256) void k_perm_rows(const int32_t* __restrict__ ids, int64_t P, int topk, int64_t E, int64_t nc,
                                                   const uint64_t* __restrict__ masks, const int* __restrict__ base,
                                                   const int* __restrict__ offsets, int* __restrict__ row_pair,
                                                   int* __restrict__ pair_row) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= P) return;
  const int64_t t = p / topk;
  const int e = ids[p];
  if ((uint32_t)e >= (uint32_t)E) {  // a dropped pair: no row, nothing combined
    pair_row[p] = -1;
    return;
  }
  const int64_t c = t / kChunk;
  const uint32_t bit = (uint32_t)(t % kChunk);
  const uint64_t below = bit ? (masks[e * nc + c] & ((1ull << bit) - 1ull)) : 0ull;
  const int pos = offsets[e] + base[c * E + e] + __popcll(below);
  row_pair[pos] = (int)p;
  pair_row[p] = pos;
}

// ---------------------------------------------------------------------------
// Operand decoding to FP16 (exact)
// ---------------------------------------------------------------------------
// E2M1 x E4M3 block scale: the hardware FP4 -> FP16 converter (unit scale; it
// uses only the exponent of its scale operand) gives q exactly, one packed
// FP16 multiply by s_b gives q * s_b exactly (<= 6 significant bits, within
// [2^-10, 2688]).  E4M3 -> FP16 is exact with the FP8 converter.
__device__ inline h8v dec_fp4x8(uint32_t w, h2v s2) {
  h8v r;
  const h2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const h2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const h2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const h2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}
// E2M1 x E4M3 block scale -> BF16 (weight-only path): q exactly in FP32 from
// the hardware converter, times s_b in FP32 (exact, <= 6 significant bits),
// whose upper 16 bits are then the exact BF16 value.
__device__ inline h8v dec_fp4x8_bf16(uint32_t w, float s) {
  const f2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const f2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const f2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const f2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  return __builtin_bit_cast(h8v, make_uint4(__builtin_amdgcn_perm(f2u(p0[1] * s), f2u(p0[0] * s), 0x07060302u),
                                            __builtin_amdgcn_perm(f2u(p1[1] * s), f2u(p1[0] * s), 0x07060302u),
                                            __builtin_amdgcn_perm(f2u(p2[1] * s), f2u(p2[0] * s), 0x07060302u),
                                            __builtin_amdgcn_perm(f2u(p3[1] * s), f2u(p3[0] * s), 0x07060302u)));
}
__device__ inline h8v dec_fp8x8(uint32_t w0, uint32_t w1) {
  h8v r;
  const h2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const h2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const h2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const h2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Activations -> FP16 [T, H]: NVFP4 q * s_b (global scale applied later), FP8 q.
// 16 consecutive activation values as exact FP16: NVFP4 the q * s_b of 8 code bytes and the block's E4M3
// scale byte (the global scale stays in the epilogue), FP8 the E4M3 values of 16 code bytes.
template <bool NV>
__device__ inline void dec_act16(const uint8_t* __restrict__ c, const uint8_t* __restrict__ s, uint4& o0, uint4& o1) {
  if constexpr (NV) {
    const uint2 w = *reinterpret_cast<const uint2*>(c);
    const h2v s2 = scale_pair_hw<0>(*s);
    o0 = __builtin_bit_cast(uint4, dec_fp4x8(w.x, s2));
    o1 = __builtin_bit_cast(uint4, dec_fp4x8(w.y, s2));
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(c);
    o0 = __builtin_bit_cast(uint4, dec_fp8x8(w.x, w.y));
    o1 = __builtin_bit_cast(uint4, dec_fp8x8(w.z, w.w));
  }
}

template <bool NV>
__global__ __launch_bounds__(256) void k_decode_act(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                    int64_t n_blk, _Float16* __restrict__ out) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 16-value block
  if (f >= n_blk) return;
  uint4 o0, o1;
  dec_act16<NV>(codes + f * (NV ? 8 : 16), NV ? scales + f : nullptr, o0, o1);
  uint4* op = reinterpret_cast<uint4*>(out + f * 16);
  op[0] = o0;
  op[1] = o1;
}

// ---------------------------------------------------------------------------
// Grouped GEMM for few rows per expert ("skinny", decode-sized): one
// workgroup = 16 rows (one row tile of an expert) x 4 waves; each wave owns NT
// tiles of 16 weight rows (GEMM1: NT/2 gate + NT/2 up tiles of the same h
// columns) and streams them from HBM straight into registers, decoding every
// weight element once per row tile.  The 16 activation rows of a K step go
// through LDS once for all 4 waves.
//
// K is walked in super-steps of KS = 4*KB values; a row's codes of one
// super-step are one contiguous span, read by the row's 4 lanes (g = 0..3) as
// uint4 i = 0..KB/VPU-1 at byte i*64 + g*16, so every load instruction covers
// 64 contiguous bytes of each of its 16 rows.  Lane g thus holds values
// i*4*VPU + g*VPU .. +VPU-1 (VPU values per uint4); MFMA step J feeds 8 of
// them and reads the activations at the same k, so A and B agree on the k
// order.  NVFP4 block scales: lane g holds the whole scale span of its row for
// super-step 4q+g (the 4 lanes of a row together hold one cache line per 4
// super-steps); at super-step 4q+i every lane fetches its scale bytes from
// lane group i with ds_bpermute.  At super-step 4q+3, when all four spans are
// used, the four groups load the next line's spans together, so a row's
// line is requested once: loaded one span at a time, a line was evicted from
// L2 between the requests (each XCD streams about 3.4 MB of weights per
// super-step through its 4 MB L2) and fetched again, 8.5 % more HBM reads at
// decode.  The next super-step's codes are loaded while the
// current one is multiplied (two register sets).
// ---------------------------------------------------------------------------

template <bool NV>
struct SkGeom {
  static constexpr int VPU = NV ? 32 : 16;  // values per uint4 of codes
  static constexpr int SPU = VPU / 8;       // MFMA steps per uint4
};

template <bool NV, int KB>
struct BRegs {
  static constexpr int kVec = KB / SkGeom<NV>::VPU;  // uint4 of codes per lane and tile
  uint4 c[kVec];
};

template <bool NV, int KB>
__device__ inline void b_load(const uint8_t* codes, BRegs<NV, KB>& b) {
#pragma unroll
  for (int i = 0; i < BRegs<NV, KB>::kVec; ++i) b.c[i] = *reinterpret_cast<const uint4*>(codes + 64 * i);
}

// Whole-line weight loads (few-row kernel with chunk-staged rows).  A super-step span is 256 bytes per
// row; the 16 rows of a tile come in 4 load instructions of 8 rows x 128 bytes (8 lanes per row), each
// consuming whole cache lines, non-temporal since the weights are read once per call.  Measured on a
// streaming probe of this matrix shape: 7.0 TB/s, against 5.8 TB/s for 64 bytes of 16 rows per
// instruction (4.8 TB/s non-temporal: the second half of each line then misses).  Lines.v[2 rho + h]
// holds in lane l bytes h * 128 + (l % 8) * 16 of row 8 rho + l / 8.
typedef unsigned int u4v __attribute__((ext_vector_type(4)));
struct Lines {
  uint4 v[4];
};

__device__ inline uint4 nt_load16(const uint8_t* p) {
  const u4v z = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
  return make_uint4(z.x, z.y, z.z, z.w);
}

__device__ inline void b_load_lines(const uint8_t* span, int64_t cbytes, int lane, Lines& r) {
  const uint8_t* p = span + (int64_t)(lane >> 3) * cbytes + (lane & 7) * 16;
  r.v[0] = nt_load16(p);
  r.v[1] = nt_load16(p + 128);
  r.v[2] = nt_load16(p + 8 * cbytes);
  r.v[3] = nt_load16(p + 8 * cbytes + 128);
}

// Pair layout of the weight codes (bsm_codes_to_pairs): in every block of 16 rows, rows p and p + 8 (p < 8)
// form one double row of 2 * cbytes bytes whose 128-byte lines hold 64 bytes of row p, then the same 64
// bytes of row p + 8.  Lane (m, g) then loads its pieces of a super-step straight in the MFMA lane layout
// (piece i: bytes i * 64 + g * 16 of row m's span, at byte offset soff of the row), and each load
// instruction still covers 8 whole lines, one in each double row.  tile: the block's first byte.
__device__ inline void b_load_pairs(const uint8_t* tile, int64_t cbytes, int64_t soff, int lane, Lines& r) {
  const int m = lane & 15, g = lane >> 4;
  const uint8_t* p = tile + (int64_t)(m & 7) * 2 * cbytes + 2 * soff + (m >> 3) * 64 + g * 16;
  r.v[0] = nt_load16(p);
  r.v[1] = nt_load16(p + 128);
  r.v[2] = nt_load16(p + 256);
  r.v[3] = nt_load16(p + 384);
}

// Piece i (0..3) of the lane layout of b_load from whole-line loads: lane (m, g) takes bytes i * 64 + g * 16
// of row m, that is half i / 2, 16-byte piece (i % 2) * 4 + g of it, held by lane (m % 8) * 8 + (i % 2) * 4
// + g in Lines.v[2 (m / 8) + i / 2].  Every lane takes both candidates with ds_bpermute and keeps its own.
__device__ inline uint4 piece_from_lines(const Lines& r, int m, int g, int i) {
  const int addr = ((m & 7) * 8 + (i & 1) * 4 + g) * 4;
  const bool hi = m >= 8;
  const uint4 lo = r.v[i >> 1], up = r.v[2 + (i >> 1)];
  const uint32_t sl[4] = {lo.x, lo.y, lo.z, lo.w}, su[4] = {up.x, up.y, up.z, up.w};
  uint32_t o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t a = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)sl[d]);
    const uint32_t c = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)su[d]);
    o[d] = hi ? c : a;
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// scale span of one super-step (KB/4 bytes) held by a lane
template <int KB>
struct SRegs {
  static constexpr int kDw = KB / 16;
  uint32_t d[kDw];
};

template <int KB>
__device__ inline void s_load(const uint8_t* p, bool in, SRegs<KB>& s) {
  if constexpr (SRegs<KB>::kDw >= 4) {
#pragma unroll
    for (int q = 0; q < SRegs<KB>::kDw; q += 4) {
      const uint4 v = in ? *reinterpret_cast<const uint4*>(p + 4 * q) : make_uint4(0u, 0u, 0u, 0u);
      s.d[q] = v.x;
      s.d[q + 1] = v.y;
      s.d[q + 2] = v.z;
      s.d[q + 3] = v.w;
    }
  } else {
    const uint2 v = in ? *reinterpret_cast<const uint2*>(p) : make_uint2(0u, 0u);
    s.d[0] = v.x;
    s.d[1] = v.y;
  }
}

// This lane's scale dwords of the current super-step from lane group i:
// dword 2u + (g >> 1) of the span carries the lane's 2 bytes for uint4 u.
template <int KB>
__device__ inline void s_fetch(const SRegs<KB>& s, int src_addr, int ghi, uint32_t* out) {
  constexpr int kVec = KB / 32;
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src_addr, (int)s.d[2 * u]);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src_addr, (int)s.d[2 * u + 1]);
    out[u] = ghi ? hi : lo;
  }
}

__device__ inline h2v scale_pair_sel(uint32_t w, uint32_t sel) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__builtin_amdgcn_perm(w, w, sel), 1.0f, false);
}

// MFMA step J of a super-step from the lane's 16-byte piece c = J / SPU of its codes
template <bool NV, int KB, int J, bool A16>
__device__ inline h8v dec_piece(uint4 c, const uint32_t* sdw, uint32_t selA, uint32_t selB) {
  constexpr int SPU = SkGeom<NV>::SPU;
  if constexpr (NV) {
    const uint32_t w = (J & 3) == 0 ? c.x : (J & 3) == 1 ? c.y : (J & 3) == 2 ? c.z : c.w;
    const h2v s2 = scale_pair_sel(sdw[J / SPU], ((J & 3) >> 1) ? selB : selA);
    if constexpr (A16) return dec_fp4x8_bf16(w, (float)s2[0]);
    return dec_fp4x8(w, s2);
  } else {
    return (J & 1) ? dec_fp8x8(c.z, c.w) : dec_fp8x8(c.x, c.y);
  }
}

template <bool NV, int KB, int J, bool A16>
__device__ inline h8v b_dec(const BRegs<NV, KB>& b, const uint32_t* sdw, uint32_t selA, uint32_t selB) {
  return dec_piece<NV, KB, J, A16>(b.c[J / SkGeom<NV>::SPU], sdw, selA, selB);
}

template <bool NV, int KB, int NT, int J, bool A16>
__device__ inline void sk_mma_step(const _Float16* arow, const BRegs<NV, KB>* b, const uint32_t (*sdw)[KB / 32 > 0 ? KB / 32 : 1],
                                   uint32_t selA, uint32_t selB, f4v* acc) {
  constexpr int VPU = SkGeom<NV>::VPU, SPU = SkGeom<NV>::SPU;
  constexpr int col = (J / SPU) * 4 * VPU + (J % SPU) * 8;  // plus g * VPU, folded into arow
  const h8v a = *reinterpret_cast<const h8v*>(arow + col);
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = mfma_ab<A16>(a, b_dec<NV, KB, J, A16>(b[t], sdw[t], selA, selB), acc[t]);
  if constexpr (J + 1 < KB / 8) sk_mma_step<NV, KB, NT, J + 1, A16>(arow, b, sdw, selA, selB, acc);
}

// Piece J from the lane's scale pairs (sp[q]: the two FP16 block scales of scale dword q that this lane's
// group uses; the piece takes one of them, broadcast within the packed multiply).
template <bool NV, int KB, int J, bool A16>
__device__ inline h8v dec_piece_sp(uint4 c, const h2v* sp) {
  constexpr int SPU = SkGeom<NV>::SPU;
  if constexpr (NV) {
    const uint32_t w = (J & 3) == 0 ? c.x : (J & 3) == 1 ? c.y : (J & 3) == 2 ? c.z : c.w;
    const _Float16 sk = ((J & 3) >> 1) ? sp[J / SPU][1] : sp[J / SPU][0];
    if constexpr (A16) return dec_fp4x8_bf16(w, (float)sk);
    return dec_fp4x8(w, h2v{sk, sk});
  } else {
    return (J & 1) ? dec_fp8x8(c.z, c.w) : dec_fp8x8(c.x, c.y);
  }
}

// The same steps from whole-line loads: piece i of every tile is moved into the MFMA lane layout just
// before its first step (4 registers per tile live instead of the whole super-step).  PAIRS: the loads
// already hold piece i in register i (pair layout), nothing is moved.
template <bool NV, int KB, int NT, int J, bool A16, bool PAIRS>
__device__ inline void sk_mma_step_lines(const _Float16* arow, const Lines* r, int m, int g,
                                         const h2v (*sp)[KB / 32 > 0 ? KB / 32 : 1], f4v* acc, uint4* cur) {
  constexpr int VPU = SkGeom<NV>::VPU, SPU = SkGeom<NV>::SPU;
  constexpr int col = (J / SPU) * 4 * VPU + (J % SPU) * 8;  // plus g * VPU, folded into arow
  if constexpr (J % SPU == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) cur[t] = PAIRS ? r[t].v[J / SPU] : piece_from_lines(r[t], m, g, J / SPU);
  }
  const h8v a = *reinterpret_cast<const h8v*>(arow + col);
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = mfma_ab<A16>(a, dec_piece_sp<NV, KB, J, A16>(cur[t], sp[t]), acc[t]);
  if constexpr (J + 1 < KB / 8) sk_mma_step_lines<NV, KB, NT, J + 1, A16, PAIRS>(arow, r, m, g, sp, acc, cur);
}

template <bool NV, bool G1, int KB, int NT, bool A16 = false, int DEPTH = 1>
__global__ __launch_bounds__(256, DEPTH == 1 ? 3 : 2) void k_skinny(const _Float16* __restrict__ act, const int* __restrict__ row_pair,
                                                int topk, const float* __restrict__ a_gs,
                                                const float* __restrict__ a_rs, const uint8_t* __restrict__ wc,
                                                const uint8_t* __restrict__ wsc, const float* __restrict__ wgs,
                                                const int4* __restrict__ tiles, const int* __restrict__ ntiles,
                                                int64_t K, int64_t H, int64_t I, float* __restrict__ out,
                                                uint32_t* __restrict__ h_amax) {
  constexpr int KS = 4 * KB;         // k per super-step
  constexpr int kAs = KS + 8;        // LDS row stride (f16), +8 pad
  constexpr int kAv = KS / 16 / 8;   // uint4 of A staged per thread (16 threads per row)
  constexpr int VPU = SkGeom<NV>::VPU;
  constexpr int kSV = KB / 32 > 0 ? KB / 32 : 1;  // scale dwords per lane and tile per super-step
  __shared__ __attribute__((aligned(16))) _Float16 As[2][16][kAs];
  if ((int)blockIdx.y >= *ntiles) return;
  const int4 ti = tiles[blockIdx.y];
  const int e = ti.x, row0 = ti.y, nrows = ti.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  // activation staging: 16 threads per row.  Only the tile's nrows rows are staged: an MFMA output row
  // depends on its own A row only, and the rows past nrows are never stored, so their LDS rows may hold
  // anything (an expert at decode has about 2 of its 16 rows).
  const int sr = tid >> 4, sseg = tid & 15;
  const bool stage = sr < nrows;
  const int ar = stage ? sr : nrows - 1;
  const _Float16* asrc = (G1 ? act + (int64_t)(row_pair[row0 + ar] / topk) * K : act + (int64_t)(row0 + ar) * K) +
                         sseg * (KS / 16);
  // weight rows of this wave
  // GEMM1: NT/2 gate tiles + NT/2 up tiles -> 8*NT h columns per wave; GEMM2: 16*NT y columns
  const int64_t n0 = ((int64_t)blockIdx.x * 4 + wave) * (G1 ? 8 * NT : 16 * NT);
  const int64_t cbytes = NV ? K / 2 : K;
  constexpr int cstep = NV ? KS / 2 : KS;  // code bytes per row and super-step
  constexpr int sstep = KS / 16;           // NVFP4 scale bytes per row and super-step
  const int nsteps = (int)(K / KS);
  const uint8_t* crow[NT];
  const uint8_t* srow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int64_t r = G1 ? (int64_t)e * 2 * I + (j >= NT / 2 ? I : 0) + n0 + 16 * (j % (NT / 2)) + m
                         : (int64_t)e * H + n0 + 16 * j + m;
    crow[j] = wc + r * cbytes + 16 * g;
    srow[j] = NV ? wsc + r * (K / 16) + (int64_t)sstep * g : nullptr;  // lane g: super-step 4q + g
  }
  f4v acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f4v{0.f, 0.f, 0.f, 0.f};
  // scale byte selectors: lane g's two bytes sit in half (g & 1) of each fetched dword
  const uint32_t selA = (uint32_t)((g & 1) * 2) * 0x0101u, selB = selA + 0x0101u;
  const int ghi = g >> 1;

  static_assert(kAv == 1 || kAv == 2 || kAv == 4, "activation staging: 1, 2 or 4 uint4 per thread");
  // DEPTH + 1 register sets of codes: the codes of super-step s + DEPTH load while s is multiplied
  static_assert(DEPTH == 1 || DEPTH == 2, "weight prefetch depth 1 or 2 super-steps");
  BRegs<NV, KB> b0[NT], b1[NT], b2[DEPTH > 1 ? NT : 1];
  SRegs<KB> sc[NT];  // NVFP4 scale span of super-step 4q + g (this lane's share of the current group)
  uint32_t sdw[NT][kSV];
  uint4 ra0, ra1, ra2, ra3;
  // prologue: super-step 0 weights and scale group 0 first (their addresses depend only on the
  // tile descriptor), then the activations (GEMM1 gathers them through row_pair)
#pragma unroll
  for (int j = 0; j < NT; ++j) b_load<NV, KB>(crow[j], b0[j]);
  if constexpr (DEPTH > 1) {
    if (nsteps > 1) {
#pragma unroll
      for (int j = 0; j < NT; ++j) b_load<NV, KB>(crow[j] + cstep, b1[j]);
    }
  }
  if constexpr (NV) {
#pragma unroll
    for (int j = 0; j < NT; ++j) s_load<KB>(srow[j], g < nsteps, sc[j]);
  }
  if (stage) {
    ra0 = reinterpret_cast<const uint4*>(asrc)[0];
    if constexpr (kAv >= 2) ra1 = reinterpret_cast<const uint4*>(asrc)[1];
    if constexpr (kAv >= 4) {
      ra2 = reinterpret_cast<const uint4*>(asrc)[2];
      ra3 = reinterpret_cast<const uint4*>(asrc)[3];
    }
    reinterpret_cast<uint4*>(&As[0][sr][sseg * (KS / 16)])[0] = ra0;
    if constexpr (kAv >= 2) reinterpret_cast<uint4*>(&As[0][sr][sseg * (KS / 16)])[1] = ra1;
    if constexpr (kAv >= 4) {
      reinterpret_cast<uint4*>(&As[0][sr][sseg * (KS / 16)])[2] = ra2;
      reinterpret_cast<uint4*>(&As[0][sr][sseg * (KS / 16)])[3] = ra3;
    }
  }
  __syncthreads();
#define BSM_SK_STEP(ST, CUR, BC, BN)                                                                      \
  {                                                                                                       \
    const bool more = (ST) + 1 < nsteps;                                                                  \
    if constexpr (NV) {                                                                                   \
      /* every lane takes its scale bytes of this super-step from lane group gi; after the */            \
      /* fourth, the four groups load the next line of scale spans together */                           \
      const int gi = (ST) & 3;                                                                            \
      _Pragma("unroll") for (int j = 0; j < NT; ++j) s_fetch<KB>(sc[j], (m + 16 * gi) * 4, ghi, sdw[j]);  \
      if (gi == 3 && (ST) + 1 < nsteps) { /* the next line: span of super-step ST + 1 + g per group */    \
        _Pragma("unroll") for (int j = 0; j < NT; ++j)                                                   \
          s_load<KB>(srow[j] + (int64_t)((ST) + 1) * sstep, (ST) + 1 + g < nsteps, sc[j]);                \
      }                                                                                                   \
    }                                                                                                     \
    if (more) {                                                                                           \
      const int64_t ko = (int64_t)((ST) + 1) * KS;                                                        \
      if (stage) {                                                                                        \
        ra0 = reinterpret_cast<const uint4*>(asrc + ko)[0];                                               \
        if constexpr (kAv >= 2) ra1 = reinterpret_cast<const uint4*>(asrc + ko)[1];                       \
        if constexpr (kAv >= 4) {                                                                         \
          ra2 = reinterpret_cast<const uint4*>(asrc + ko)[2];                                             \
          ra3 = reinterpret_cast<const uint4*>(asrc + ko)[3];                                             \
        }                                                                                                 \
      }                                                                                                   \
    }                                                                                                     \
    if ((ST) + DEPTH < nsteps) {                                                                          \
      _Pragma("unroll") for (int j = 0; j < NT; ++j)                                                     \
        b_load<NV, KB>(crow[j] + ((ST) + DEPTH) * (int64_t)cstep, BN[j]);                                 \
    }                                                                                                     \
    sk_mma_step<NV, KB, NT, 0, A16>(&As[CUR][m][VPU * g], BC, sdw, selA, selB, acc);                      \
    if (more && stage) {                                                                                  \
      reinterpret_cast<uint4*>(&As[(CUR) ^ 1][sr][sseg * (KS / 16)])[0] = ra0;                            \
      if constexpr (kAv >= 2) reinterpret_cast<uint4*>(&As[(CUR) ^ 1][sr][sseg * (KS / 16)])[1] = ra1;    \
      if constexpr (kAv >= 4) {                                                                           \
        reinterpret_cast<uint4*>(&As[(CUR) ^ 1][sr][sseg * (KS / 16)])[2] = ra2;                          \
        reinterpret_cast<uint4*>(&As[(CUR) ^ 1][sr][sseg * (KS / 16)])[3] = ra3;                          \
      }                                                                                                   \
    }                                                                                                     \
    __syncthreads();                                                                                      \
  }
  if constexpr (DEPTH == 1) {
    // two super-steps per iteration so the code register set of each step is static
    for (int st = 0; st < nsteps; st += 2) {
      BSM_SK_STEP(st, 0, b0, b1)
      if (st + 1 < nsteps) BSM_SK_STEP(st + 1, 1, b1, b0)
    }
  } else {
    for (int st = 0; st < nsteps; st += 3) {
      BSM_SK_STEP(st, st & 1, b0, b2)
      if (st + 1 < nsteps) BSM_SK_STEP(st + 1, (st + 1) & 1, b1, b0)
      if (st + 2 < nsteps) BSM_SK_STEP(st + 2, st & 1, b2, b1)
    }
  }
#undef BSM_SK_STEP

  float hmax = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ro = 4 * g + r;
    if (ro >= nrows) continue;
    if (G1) {
#pragma unroll
      for (int q = 0; q < NT / 2; ++q) {
        const int64_t col = n0 + 16 * q + m;
        float sg, su;
        if (NV) {
          const float ag = A16 ? 1.0f : a_gs[0];  // weight-only: BF16 activations carry no scale
          sg = ag * wgs[2 * e];
          su = ag * wgs[2 * e + 1];
        } else {
          const float sx = a_rs[row_pair[row0 + ro] / topk];
          const float* ws = reinterpret_cast<const float*>(wsc) + (int64_t)e * 2 * I;
          sg = sx * ws[col];
          su = sx * ws[I + col];
        }
        const float h = silu_mul(acc[q][r] * sg, acc[NT / 2 + q][r] * su);
        out[(int64_t)(row0 + ro) * I + col] = h;
        hmax = fmaxf(hmax, fabsf(h));
      }
    } else {
      float* yr = out + (int64_t)(row0 + ro) * H + n0 + m;
      if (NV) {
        const float sc = (A16 ? 1.0f : a_gs[0]) * wgs[e];
#pragma unroll
        for (int j = 0; j < NT; ++j) yr[16 * j] = acc[j][r] * sc;
      } else {
        const float sa = a_rs[row0 + ro];
        const float* ws = reinterpret_cast<const float*>(wsc) + (int64_t)e * H + n0 + m;
#pragma unroll
        for (int j = 0; j < NT; ++j) yr[16 * j] = acc[j][r] * sa * ws[16 * j];
      }
    }
  }
  if constexpr (G1 && NV) wg_amax_atomic(hmax, h_amax);
}

// ---------------------------------------------------------------------------
// NVFP4 grouped GEMM for few rows per expert, activation rows staged in large
// chunks of K ("rows"): the lane mapping, weight streaming (two register sets
// of codes, one super-step ahead), scale handling and MFMA steps of k_skinny,
// but the tile's activation rows go to LDS for kc super-steps at a time
// (kc from the rows and kRowsLds bytes of LDS; the whole K when the tile has
// few rows, as at decode), so the waves run those super-steps without a
// barrier: a wave waiting for its weights does not hold the other three.
// QA: the rows are staged from their codes (acodes; NVFP4 with the block
// scales ascales) and decoded to FP16 on the way into LDS, instead of being
// read from an FP16 copy (act): each workgroup re-reads its rows, and the
// codes are 3.6 (NVFP4) or 2 (FP8) times fewer bytes.
// ---------------------------------------------------------------------------
constexpr int kRowsLds = 44 * 1024;  // LDS bytes for the staged rows (three workgroups per CU)

template <bool NV, bool G1, int NT, bool A16 = false, int DEPTH = 1, bool QA = false, bool PAIRS = false>
__global__ __launch_bounds__(256, DEPTH == 1 ? 3 : 2) void k_skinny_rows(
    const _Float16* __restrict__ act, const uint8_t* __restrict__ acodes, const uint8_t* __restrict__ ascales,
    const int* __restrict__ row_pair, int topk, const float* __restrict__ a_gs,
    const float* __restrict__ a_rs, const uint8_t* __restrict__ wc, const uint8_t* __restrict__ wsc,
    const float* __restrict__ wgs, const int4* __restrict__ tiles, const int* __restrict__ ntiles, int64_t K, int64_t H,
    int64_t I, float* __restrict__ out, uint32_t* __restrict__ h_amax) {
  constexpr int KB = NV ? kNvKB : kF8KB;
  constexpr int KS = 4 * KB;  // k per super-step
  constexpr int VPU = SkGeom<NV>::VPU;
  constexpr int kSV = KB / 32;
  constexpr int cstep = NV ? KS / 2 : KS, sstep = KS / 16;  // code (NVFP4: and scale) bytes per row and super-step
  constexpr int kU = DEPTH + 1;  // super-steps per unrolled iteration (one per register set)
  static_assert(!(NV && PAIRS) || DEPTH == 1, "lane-ordered NVFP4 scales: two register sets, depth 1");
  static_assert(!(NV && PAIRS) || KS == 512, "lane-ordered NVFP4 scales: 32 per row and super-step");
  __shared__ __attribute__((aligned(16))) _Float16 Ar[kRowsLds / 2];
  // Gate/up: workgroup i runs on XCD i % 8 (the dispatcher deals workgroups out round robin), so the live
  // workgroups are renumbered to give each XCD one contiguous run of (row tile, column block) items in
  // column order.  The column blocks of a row tile then run on one XCD at about the same time, and its
  // L2 fetches the tile's activation rows once instead of once per XCD and again after eviction.
  int bx = (int)blockIdx.x, by = (int)blockIdx.y;
  if constexpr (G1) {
    const int gx = (int)gridDim.x, live = *ntiles * gx, lin = by * gx + bx;
    if (lin >= live) return;
    int pre = 0;  // live workgroups on the XCDs before this one: those with index i (mod 8), i < lin % 8
    for (int i = 0; i < (lin & 7); ++i) pre += (live - i + 7) >> 3;
    const int q = pre + (lin >> 3);
    by = q / gx;
    bx = q - by * gx;
  } else {
    if (by >= *ntiles) return;
  }
  const int4 ti = tiles[by];
  const int e = ti.x, row0 = ti.y, nrows = ti.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int nsteps = (int)(K / KS);
  // super-steps per chunk (a multiple of kU): nrows rows of kc * KS values, +8 f16 per row so the
  // fragment reads of different rows start on different banks
  int kc = (int)((kRowsLds / nrows / 2 - 8) / KS) / kU * kU;
  kc = kc < kU ? kU : kc;
  const int rstride = kc * KS + 8;  // f16
  // this lane's A row (rows past nrows read the last real row: their outputs are never stored)
  const _Float16* arow = Ar + (m < nrows ? m : nrows - 1) * rstride + VPU * g;
  const int64_t n0 = ((int64_t)bx * 4 + wave) * (G1 ? 8 * NT : 16 * NT);
  const int64_t cbytes = NV ? K / 2 : K;
  const uint8_t* trow[NT];  // first weight row of each tile (its 16 rows are consecutive)
  const uint8_t* srow[NT];
  const uint8_t* stile[NT];
  // NVFP4 with the pair layout: the lane-ordered scales (bsm_scales_to_lanes) of a super-step are one 8-byte
  // load per lane and tile (the two blocks of each of its 4 pieces), two sets: super-step s + 1 loads while
  // s is multiplied
  uint2 q0[NT], q1[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int64_t r0 = G1 ? (int64_t)e * 2 * I + (j >= NT / 2 ? I : 0) + n0 + 16 * (j % (NT / 2))
                          : (int64_t)e * H + n0 + 16 * j;
    trow[j] = wc + r0 * cbytes;
    srow[j] = NV ? wsc + (r0 + m) * (K / 16) + (int64_t)sstep * g : nullptr;  // lane g: super-step 4q + g
    stile[j] = NV ? wsc + r0 * (K / 16) : nullptr;  // lane-ordered scales: the 16-row block's first byte
  }
  f4v acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f4v{0.f, 0.f, 0.f, 0.f};
  const uint32_t selA = (uint32_t)((g & 1) * 2) * 0x0101u, selB = selA + 0x0101u;
  const int ghi = g >> 1;
  Lines b0[NT], b1[NT], b2[DEPTH > 1 ? NT : 1];  // whole-line loads in flight (DEPTH + 1 sets)
  uint4 cur[NT];                                 // the current piece of every tile in the MFMA lane layout
  SRegs<KB> sc[NT];
  uint32_t sdw[NT][kSV > 0 ? kSV : 1];
  h2v sp[NT][kSV > 0 ? kSV : 1];  // NVFP4: this lane's two FP16 block scales of each scale dword
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if constexpr (PAIRS)
      b_load_pairs(trow[j], cbytes, 0, lane, b0[j]);
    else
      b_load_lines(trow[j], cbytes, lane, b0[j]);
  }
  if constexpr (DEPTH > 1) {
    if (nsteps > 1) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        if constexpr (PAIRS)
          b_load_pairs(trow[j], cbytes, cstep, lane, b1[j]);
        else
          b_load_lines(trow[j] + cstep, cbytes, lane, b1[j]);
      }
    }
  }
  if constexpr (NV) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if constexpr (PAIRS)
        q0[j] = *reinterpret_cast<const uint2*>(stile[j] + m * 32 + g * 8);
      else
        s_load<KB>(srow[j], g < nsteps, sc[j]);
    }
  }
  // one super-step: NVFP4 scale bytes (pair layout: the lane's own 8 bytes from SC; canonical: from lane
  // group (ST & 3), and after the fourth every group loads its span of the next line), the whole-line codes
  // (and lane-ordered scales into SN) of super-step ST + DEPTH into BN, the codes of ST from BC into the
  // MFMA lane layout, the multiplies from the staged rows
#define BSM_SKR_STEP(ST, BC, BN, SC, SN)                                                               \
  {                                                                                                    \
    if constexpr (NV && PAIRS) {                                                                       \
      _Pragma("unroll") for (int j = 0; j < NT; ++j) {                                                  \
        sp[j][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(SC[j].x, 1.0f, false);                      \
        sp[j][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(SC[j].x, 1.0f, true);                       \
        sp[j][2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(SC[j].y, 1.0f, false);                      \
        sp[j][3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(SC[j].y, 1.0f, true);                       \
      }                                                                                                \
    } else if constexpr (NV) {                                                                         \
      const int gi = (ST) & 3;                                                                         \
      _Pragma("unroll") for (int j = 0; j < NT; ++j) {                                                  \
        s_fetch<KB>(sc[j], (m + 16 * gi) * 4, ghi, sdw[j]);                                            \
        _Pragma("unroll") for (int q = 0; q < kSV; ++q) {                                              \
          const h2v p01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sdw[j][q], 1.0f, false);            \
          const h2v p23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sdw[j][q], 1.0f, true);             \
          sp[j][q] = (g & 1) ? p23 : p01;                                                              \
        }                                                                                              \
      }                                                                                                \
      if (gi == 3 && (ST) + 1 < nsteps) { /* the next line: span of super-step ST + 1 + g per group */ \
        _Pragma("unroll") for (int j = 0; j < NT; ++j)                                                \
          s_load<KB>(srow[j] + (int64_t)((ST) + 1) * sstep, (ST) + 1 + g < nsteps, sc[j]);             \
      }                                                                                                \
    }                                                                                                  \
    if ((ST) + DEPTH < nsteps) {                                                                       \
      if constexpr (NV && PAIRS) {                                                                     \
        _Pragma("unroll") for (int j = 0; j < NT; ++j)                                                \
          SN[j] = *reinterpret_cast<const uint2*>(stile[j] + ((ST) + DEPTH) * 512 + m * 32 + g * 8);   \
      }                                                                                                \
      _Pragma("unroll") for (int j = 0; j < NT; ++j) {                                                \
        if constexpr (PAIRS)                                                                           \
          b_load_pairs(trow[j], cbytes, ((ST) + DEPTH) * (int64_t)cstep, lane, BN[j]);                 \
        else                                                                                           \
          b_load_lines(trow[j] + ((ST) + DEPTH) * (int64_t)cstep, cbytes, lane, BN[j]);                \
      }                                                                                                \
    }                                                                                                  \
    sk_mma_step_lines<NV, KB, NT, 0, A16, PAIRS>(arow + ((ST) - c0) * KS, BC, m, g, sp, acc, cur);    \
  }
  for (int c0 = 0; c0 < nsteps; c0 += kc) {
    const int c1 = c0 + kc < nsteps ? c0 + kc : nsteps;
    // stage rows x [c0 KS, c1 KS): 16-byte pieces, consecutive threads along a row
    if (c0 > 0) __syncthreads();  // every wave is done with the previous chunk
    if constexpr (QA) {  // 16-value blocks, consecutive threads along a row
      const int pb = (c1 - c0) * KS / 16;  // blocks per row
      for (int q = tid; q < nrows * pb; q += 256) {
        const int r = q / pb, p = q - r * pb;
        const int64_t f = (G1 ? (int64_t)(row_pair[row0 + r] / topk) : (int64_t)(row0 + r)) * (K / 16) +
                          (int64_t)c0 * (KS / 16) + p;
        uint4 o0, o1;
        dec_act16<NV>(acodes + f * (NV ? 8 : 16), NV ? ascales + f : nullptr, o0, o1);
        uint4* d = reinterpret_cast<uint4*>(Ar + r * rstride + 16 * p);
        d[0] = o0;
        d[1] = o1;
      }
    } else {  // 16-byte pieces, consecutive threads along a row
      const int pr = (c1 - c0) * KS / 8;  // pieces per row
      for (int q = tid; q < nrows * pr; q += 256) {
        const int r = q / pr, p = q - r * pr;
        const _Float16* src = (G1 ? act + (int64_t)(row_pair[row0 + r] / topk) * K : act + (int64_t)(row0 + r) * K) +
                              (int64_t)c0 * KS + 8 * p;
        *reinterpret_cast<uint4*>(Ar + r * rstride + 8 * p) = *reinterpret_cast<const uint4*>(src);
      }
    }
    __syncthreads();
    if constexpr (DEPTH == 1) {
      for (int st = c0; st < c1; st += 2) {
        BSM_SKR_STEP(st, b0, b1, q0, q1)
        if (st + 1 < c1) BSM_SKR_STEP(st + 1, b1, b0, q1, q0)
      }
    } else {  // super-step st multiplies set st % 3 and loads st + 2 into set (st + 2) % 3
      for (int st = c0; st < c1; st += 3) {
        BSM_SKR_STEP(st, b0, b2, q0, q1)  /* NVFP4 runs depth 1: the scale sets are unused here */
        if (st + 1 < c1) BSM_SKR_STEP(st + 1, b1, b0, q0, q1)
        if (st + 2 < c1) BSM_SKR_STEP(st + 2, b2, b1, q0, q1)
      }
    }
  }
#undef BSM_SKR_STEP

  float hmax = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ro = 4 * g + r;
    if (ro >= nrows) continue;
    if (G1) {
#pragma unroll
      for (int q = 0; q < NT / 2; ++q) {
        const int64_t col = n0 + 16 * q + m;
        float sg, su;
        if (NV) {
          const float ag = A16 ? 1.0f : a_gs[0];  // weight-only: BF16 activations carry no scale
          sg = ag * wgs[2 * e];
          su = ag * wgs[2 * e + 1];
        } else {
          const float sx = a_rs[row_pair[row0 + ro] / topk];
          const float* ws = reinterpret_cast<const float*>(wsc) + (int64_t)e * 2 * I;
          sg = sx * ws[col];
          su = sx * ws[I + col];
        }
        const float h = silu_mul(acc[q][r] * sg, acc[NT / 2 + q][r] * su);
        out[(int64_t)(row0 + ro) * I + col] = h;
        hmax = fmaxf(hmax, fabsf(h));
      }
    } else {
      float* yr = out + (int64_t)(row0 + ro) * H + n0 + m;
      if (NV) {
        const float sc = (A16 ? 1.0f : a_gs[0]) * wgs[e];
#pragma unroll
        for (int j = 0; j < NT; ++j) yr[16 * j] = acc[j][r] * sc;
      } else {
        const float sa = a_rs[row0 + ro];
        const float* ws = reinterpret_cast<const float*>(wsc) + (int64_t)e * H + n0 + m;
#pragma unroll
        for (int j = 0; j < NT; ++j) yr[16 * j] = acc[j][r] * sa * ws[16 * j];
      }
    }
  }
  if constexpr (G1 && NV) wg_amax_atomic(hmax, h_amax);
}

// ---------------------------------------------------------------------------
// Dense FP8 GEMM for at most 64 rows (decode-sized dense projections and the
// dense SwiGLU MLP, one weight matrix): every workgroup covers all rows, so
// each weight byte is streamed from HBM once (the 16-row tiles of k_skinny
// would stream it once per tile).  The weights stream HBM -> registers as in
// k_skinny (lane g of a row holds the 16-byte pieces i*64 + g*16 of the
// row's super-step span), decoded once per workgroup and fed to up to 4
// row-tile MFMAs; the rows' E4M3 codes of a super-step are decoded to FP16
// once, into LDS.  Narrow outputs split K over gridDim.z (fixed ranges of
// super-steps); the partial sums go to a workspace and k_dense_reduce adds
// them in split order and applies the scales (and SwiGLU).
// ---------------------------------------------------------------------------
constexpr int kDenseRows = 64;

template <bool G1, int KB>
__global__ __launch_bounds__(256, 2) void k_dense_f8(const uint8_t* __restrict__ xc, const float* __restrict__ xs,
                                                     int64_t T, int64_t K, const uint8_t* __restrict__ wc,
                                                     const float* __restrict__ wsc, int64_t N, int64_t I,
                                                     float* __restrict__ out, float* __restrict__ part) {
  constexpr int NT = 2;              // 16-row weight tiles per wave (GEMM1: one gate, one up)
  constexpr int KS = 4 * KB;         // k per super-step
  constexpr int kAs = KS + 8;        // LDS row stride (f16), +8 pad
  constexpr int VPU = 16, SPU = 2;   // FP8 values per uint4 of codes; MFMA steps per uint4
  constexpr int kAq = KS / 4 / 16;   // uint4 of codes staged per thread (4 threads per row)
  __shared__ __attribute__((aligned(16))) _Float16 As[2][kDenseRows][kAs];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int nrt = (int)((T + 15) / 16);
  const int64_t n0 = ((int64_t)blockIdx.x * 4 + wave) * (G1 ? 8 * NT : 16 * NT);
  const uint8_t* crow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int64_t r = G1 ? (j == 1 ? I : 0) + n0 + m : n0 + 16 * j + m;
    crow[j] = wc + r * K + 16 * g;
  }
  const int nss = (int)(K / KS), nsplit = (int)gridDim.z, sp = (int)blockIdx.z;
  const int ss0 = (int)((int64_t)sp * nss / nsplit), ss1 = (int)((int64_t)(sp + 1) * nss / nsplit);
  // activation staging: row sr, quarter sq of the super-step (only the T real rows)
  const int sr = tid >> 2, sq = tid & 3;
  const bool stage = sr < T;
  const uint8_t* asrc = xc + (int64_t)(stage ? sr : 0) * K + sq * (KS / 4);
  uint4 ra[kAq];
  auto aload = [&](int ss) {
    if (stage) {
#pragma unroll
      for (int q = 0; q < kAq; ++q) ra[q] = reinterpret_cast<const uint4*>(asrc + (int64_t)ss * KS)[q];
    }
  };
  auto astore = [&](int buf) {
    if (stage) {
#pragma unroll
      for (int q = 0; q < kAq; ++q) {
        uint4* d = reinterpret_cast<uint4*>(&As[buf][sr][sq * (KS / 4) + 16 * q]);
        d[0] = __builtin_bit_cast(uint4, dec_fp8x8(ra[q].x, ra[q].y));
        d[1] = __builtin_bit_cast(uint4, dec_fp8x8(ra[q].z, ra[q].w));
      }
    }
  };
  BRegs<false, KB> b0[NT], b1[NT];
  f4v acc[4][NT];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[rt][j] = f4v{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](int buf, const BRegs<false, KB>* bc) {
#pragma unroll
    for (int J = 0; J < KB / 8; ++J) {
      const int col = (J / SPU) * 4 * VPU + (J % SPU) * 8 + g * VPU;
      h8v bd[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const uint4 c = bc[j].c[J / SPU];
        bd[j] = (J & 1) ? dec_fp8x8(c.z, c.w) : dec_fp8x8(c.x, c.y);
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if (rt < nrt) {
          const h8v a = *reinterpret_cast<const h8v*>(&As[buf][16 * rt + m][col]);
#pragma unroll
          for (int j = 0; j < NT; ++j) acc[rt][j] = mfma_ab<false>(a, bd[j], acc[rt][j]);
        }
      }
    }
  };
  if (ss0 < ss1) {
#pragma unroll
    for (int j = 0; j < NT; ++j) b_load<false, KB>(crow[j] + (int64_t)ss0 * KS, b0[j]);
    aload(ss0);
    astore(0);
    __syncthreads();
    for (int ss = ss0; ss < ss1; ss += 2) {
      // two super-steps per iteration so the code register set of each step is static
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int cur = ss + h;
        if (cur < ss1) {
          const bool more = cur + 1 < ss1;
          if (more) {
            aload(cur + 1);
#pragma unroll
            for (int j = 0; j < NT; ++j) b_load<false, KB>(crow[j] + (int64_t)(cur + 1) * KS, h ? b0[j] : b1[j]);
          }
          mma((cur - ss0) & 1, h ? b1 : b0);
          if (more) astore(((cur - ss0) & 1) ^ 1);
          __syncthreads();
        }
      }
    }
  }
  // epilogue: result register r of lane (m, g) is row 16 rt + 4 g + r, column m of the tile
  const int64_t ncols = G1 ? 2 * I : N;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = 16 * rt + 4 * g + r;
      if (t >= T) continue;
      if (nsplit > 1) {
        float* pr = part + ((int64_t)sp * T + t) * ncols;
        if (G1) {
          pr[n0 + m] = acc[rt][0][r];
          pr[I + n0 + m] = acc[rt][1][r];
        } else {
#pragma unroll
          for (int j = 0; j < NT; ++j) pr[n0 + 16 * j + m] = acc[rt][j][r];
        }
      } else if (G1) {
        const int64_t col = n0 + m;
        const float sx = xs[t];
        out[t * I + col] = silu_mul(acc[rt][0][r] * (sx * wsc[col]), acc[rt][1][r] * (sx * wsc[I + col]));
      } else {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int64_t col = n0 + 16 * j + m;
          out[t * N + col] = acc[rt][j][r] * xs[t] * wsc[col];
        }
      }
    }
  }
}

// Split-K partial sums of k_dense_f8, added in split order, then its epilogue.
template <bool G1>
__global__ __launch_bounds__(256) void k_dense_reduce(const float* __restrict__ part, int nsplit, int64_t T,
                                                      int64_t N, int64_t I, const float* __restrict__ xs,
                                                      const float* __restrict__ wsc, float* __restrict__ out) {
  const int64_t nout = G1 ? I : N, ncols = G1 ? 2 * I : N;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * nout) return;
  const int64_t t = i / nout, col = i % nout;
  float a = 0.0f, b = 0.0f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float* pr = part + ((int64_t)sp * T + t) * ncols;
    a += pr[col];
    if (G1) b += pr[I + col];
  }
  if (G1) {
    const float sx = xs[t];
    out[i] = silu_mul(a * (sx * wsc[col]), b * (sx * wsc[I + col]));
  } else {
    out[i] = a * xs[t] * wsc[col];
  }
}

// Split count of k_dense_f8 (at least one super-step per split, at most 16).  A workgroup streams its
// weights at a roughly fixed rate, so the time goes as (rounds of 512 resident workgroups: two per CU,
// the LDS tile takes 66 KB) / splits, and a partly filled last round costs a whole round.  Up to 256
// column blocks: as many splits as fill one round.  More (the dense MLP's gate/up, 320 blocks): the
// count with the fewest rounds per split, charging 1 % per split for the partial sums the reduction
// reads (320 blocks: 3 splits, 960 workgroups in two rounds).
inline int dense_splits(int64_t ncb, int64_t nss) {
  if (ncb <= 256) {
    int64_t sp = 512 / ncb;
    if (sp > 16) sp = 16;
    if (sp > nss) sp = nss;
    return (int)(sp < 1 ? 1 : sp);
  }
  int best = 1;
  double best_t = 1e30;
  for (int sp = 1; sp <= 16 && sp <= nss; ++sp) {
    const double t = (double)((ncb * sp + 511) / 512) / sp + 0.01 * sp;
    if (t < best_t - 1e-9) {
      best_t = t;
      best = sp;
    }
  }
  return best;
}
constexpr int kDenseMaxSplits = 16;

template <bool G1>
hipError_t launch_dense_f8(const uint8_t* xc, const float* xs, int64_t T, int64_t K, const uint8_t* wc,
                           const float* wsc, int64_t N, int64_t I, float* out, float* part, hipStream_t st) {
  const int64_t ncb = G1 ? I / 64 : N / 128;  // 4 waves x 16 h columns / 32 output columns
  const bool kb64 = K % 256 == 0;
  const int64_t nss = K / (kb64 ? 256 : 128);
  const int sp = dense_splits(ncb, nss);
  const dim3 grid((unsigned)ncb, 1, (unsigned)sp);
  if (kb64)
    k_dense_f8<G1, 64><<<grid, 256, 0, st>>>(xc, xs, T, K, wc, wsc, N, I, out, part);
  else
    k_dense_f8<G1, 32><<<grid, 256, 0, st>>>(xc, xs, T, K, wc, wsc, N, I, out, part);
  if (sp > 1) {
    const int64_t n = T * (G1 ? I : N);
    k_dense_reduce<G1><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(part, sp, T, N, I, xs, wsc, out);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped GEMM for many rows per expert ("wide"): 128 rows x 128 weight rows
// per workgroup, K in steps of 64 staged through LDS (double buffered).  The activation tile is staged as FP16; the weight
// tile is staged as its raw codes (and NVFP4 scale bytes), a quarter (half,
// FP8) of the FP16 bytes, and each wave decodes its B fragments after reading
// them, which keeps LDS traffic below the matrix cores' demand.  Each wave
// computes 64 rows x 64 weight rows with 16 MFMA 16x16x32 tiles.  GEMM1
// workgroup: weight rows = 64 gate rows c0.. and the 64 matching up rows, so
// each wave holds g and u of the same 32 h columns (SwiGLU fused).
// ---------------------------------------------------------------------------
constexpr int kWBM = 128, kWBN = 128, kWBK = 64, kLds = kWBK + 8;  // +8 f16 pad: conflict-free b128 reads
// raw weight rows in LDS: NVFP4 32 B of codes per row and K step (+4 pad), FP8 64 B (+8 pad)
template <bool NV>
struct WideB {
  static constexpr int kRow = NV ? 36 : 72;
};

template <bool NV, bool G1, bool A16 = false>
__global__ __launch_bounds__(256, 3) void k_gemm_wide(const _Float16* __restrict__ act, const int* __restrict__ row_pair,
                                                      int topk, const float* __restrict__ a_gs,
                                                      const float* __restrict__ a_rs, const uint8_t* __restrict__ wc,
                                                      const uint8_t* __restrict__ wsc, const float* __restrict__ wgs,
                                                      const int4* __restrict__ tiles, const int* __restrict__ ntiles,
                                                      int64_t K, int64_t H, int64_t I, float* __restrict__ out,
                                                      uint32_t* __restrict__ h_amax) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][kWBM][kLds];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][kWBN][WideB<NV>::kRow];
  __shared__ uint32_t Bsc[2][kWBN];  // NVFP4: the 4 scale bytes of a row and K step
  if ((int)blockIdx.y >= *ntiles) return;
  const int4 ti = tiles[blockIdx.y];
  const int e = ti.x, row0 = ti.y, nrows = ti.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  // output column base: GEMM1 -> h columns c0..c0+63, GEMM2 -> y columns c0..c0+127
  const int64_t c0 = (int64_t)blockIdx.x * (G1 ? 64 : 128);
  // staging roles: row r of the A and B tiles, k half kh (32 values)
  const int sr = tid >> 1, kh = tid & 1;
  const int ar = sr < nrows ? sr : nrows - 1;
  const _Float16* asrc = G1 ? act + (int64_t)(row_pair[row0 + ar] / topk) * K + 32 * kh
                            : act + (int64_t)(row0 + ar) * K + 32 * kh;
  int64_t wrow;
  if (G1) wrow = (int64_t)e * 2 * I + (sr < 64 ? c0 + sr : I + c0 + (sr - 64));
  else wrow = (int64_t)e * H + c0 + sr;
  const int64_t cbytes = NV ? K / 2 : K;
  const uint8_t* bsrc = wc + wrow * cbytes + (NV ? 16 : 32) * kh;
  const uint8_t* ssrc = NV ? wsc + wrow * (K / 16) + 2 * kh : nullptr;

  // one register set holds the global loads of the next K step
  uint4 raX0, raX1, raX2, raX3, rbX0, rbX1;
  uint32_t rsX = 0;
#define BSM_WIDE_GLOAD(k0, S)                                                       \
  {                                                                                 \
    const uint4* pa = reinterpret_cast<const uint4*>(asrc + (k0));                  \
    ra##S##0 = pa[0];                                                               \
    ra##S##1 = pa[1];                                                               \
    ra##S##2 = pa[2];                                                               \
    ra##S##3 = pa[3];                                                               \
    if (NV) {                                                                       \
      rb##S##0 = *reinterpret_cast<const uint4*>(bsrc + (k0) / 2);                  \
      rs##S = *reinterpret_cast<const uint16_t*>(ssrc + (k0) / 16);                 \
    } else {                                                                        \
      const uint4* pb = reinterpret_cast<const uint4*>(bsrc + (k0));                \
      rb##S##0 = pb[0];                                                             \
      rb##S##1 = pb[1];                                                             \
    }                                                                               \
  }
#define BSM_WIDE_LSTORE(buf, S)                                                     \
  {                                                                                 \
    uint4* da = reinterpret_cast<uint4*>(&As[buf][sr][32 * kh]);                    \
    da[0] = ra##S##0;                                                               \
    da[1] = ra##S##1;                                                               \
    da[2] = ra##S##2;                                                               \
    da[3] = ra##S##3;                                                               \
    uint32_t* db = reinterpret_cast<uint32_t*>(&Bs[buf][sr][0]);                    \
    if (NV) {                                                                       \
      db[4 * kh + 0] = (rb##S##0).x;                                                \
      db[4 * kh + 1] = (rb##S##0).y;                                                \
      db[4 * kh + 2] = (rb##S##0).z;                                                \
      db[4 * kh + 3] = (rb##S##0).w;                                                \
      reinterpret_cast<uint16_t*>(&Bsc[buf][sr])[kh] = (uint16_t)rs##S;             \
    } else {                                                                        \
      db[8 * kh + 0] = (rb##S##0).x;                                                \
      db[8 * kh + 1] = (rb##S##0).y;                                                \
      db[8 * kh + 2] = (rb##S##0).z;                                                \
      db[8 * kh + 3] = (rb##S##0).w;                                                \
      db[8 * kh + 4] = (rb##S##1).x;                                                \
      db[8 * kh + 5] = (rb##S##1).y;                                                \
      db[8 * kh + 6] = (rb##S##1).z;                                                \
      db[8 * kh + 7] = (rb##S##1).w;                                                \
    }                                                                               \
  }
  // B rows of this wave's 4 column tiles: GEMM1 gate 0,1 / up 2,3; GEMM2 4 consecutive
#define BSM_WIDE_BROW(j) (G1 ? (((j) < 2) ? wn * 32 + 16 * (j) : 64 + wn * 32 + 16 * ((j) - 2)) : wn * 64 + 16 * (j))

  f4v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f4v{0.f, 0.f, 0.f, 0.f};
  // NVFP4 block of this lane's 8 values in sub-step s: 2s + (g >> 1) of the row's 4 scale bytes
  const uint32_t selA = (uint32_t)(g >> 1) * 0x0101u, selB = selA + 0x0202u;

  const int nk = (int)(K / kWBK);
  BSM_WIDE_GLOAD(0, X)
  BSM_WIDE_LSTORE(0, X)
  __syncthreads();
  // step ks: load step ks + 1, multiply from LDS, store step ks + 1 into the other buffer
#define BSM_WIDE_STEP(ks)                                                           \
  {                                                                                 \
    const int buf = (ks) & 1;                                                       \
    if ((ks) + 1 < nk) BSM_WIDE_GLOAD((int64_t)((ks) + 1) * kWBK, X)               \
    _Pragma("unroll") for (int s = 0; s < 2; ++s) {                                 \
      h8v a[4], b[4];                                                               \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                                 \
        a[i] = *reinterpret_cast<const h8v*>(&As[buf][wm * 64 + 16 * i + m][32 * s + 8 * g]); \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) {                               \
        const uint8_t* brow = &Bs[buf][BSM_WIDE_BROW(j) + m][0];                    \
        if (NV) {                                                                   \
          const uint32_t w = *reinterpret_cast<const uint32_t*>(brow + 16 * s + 4 * g); \
          const h2v s2 = scale_pair_sel(Bsc[buf][BSM_WIDE_BROW(j) + m], s ? selB : selA); \
          b[j] = A16 ? dec_fp4x8_bf16(w, (float)s2[0]) : dec_fp4x8(w, s2);          \
        } else {                                                                    \
          const uint2 w = *reinterpret_cast<const uint2*>(brow + 32 * s + 8 * g);  \
          b[j] = dec_fp8x8(w.x, w.y);                                               \
        }                                                                           \
      }                                                                             \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                                 \
        _Pragma("unroll") for (int j = 0; j < 4; ++j) acc[i][j] = mfma_ab<A16>(a[i], b[j], acc[i][j]); \
    }                                                                               \
    if ((ks) + 1 < nk) BSM_WIDE_LSTORE(buf ^ 1, X)                                  \
    __syncthreads();                                                                \
  }
  for (int ks = 0; ks < nk; ++ks) BSM_WIDE_STEP(ks)
#undef BSM_WIDE_STEP
#undef BSM_WIDE_GLOAD
#undef BSM_WIDE_LSTORE
#undef BSM_WIDE_BROW

  float hmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ro = wm * 64 + 16 * i + 4 * g + r;
      if (ro >= nrows) continue;
      if (G1) {
        float sg0, su0, sg1, su1;
        const int64_t col0 = c0 + wn * 32 + m, col1 = col0 + 16;
        if (NV) {
          const float ag = A16 ? 1.0f : a_gs[0];
          sg0 = sg1 = ag * wgs[2 * e];
          su0 = su1 = ag * wgs[2 * e + 1];
        } else {
          const float sx = a_rs[row_pair[row0 + ro] / topk];
          const float* ws = reinterpret_cast<const float*>(wsc) + (int64_t)e * 2 * I;
          sg0 = sx * ws[col0];
          sg1 = sx * ws[col1];
          su0 = sx * ws[I + col0];
          su1 = sx * ws[I + col1];
        }
        const float h0 = silu_mul(acc[i][0][r] * sg0, acc[i][2][r] * su0);
        const float h1 = silu_mul(acc[i][1][r] * sg1, acc[i][3][r] * su1);
        float* hr = out + (int64_t)(row0 + ro) * I;
        hr[col0] = h0;
        hr[col1] = h1;
        hmax = fmaxf(hmax, fmaxf(fabsf(h0), fabsf(h1)));
      } else {
        float* yr = out + (int64_t)(row0 + ro) * H + c0 + wn * 64 + m;
        if (NV) {
          const float sc = (A16 ? 1.0f : a_gs[0]) * wgs[e];
#pragma unroll
          for (int j = 0; j < 4; ++j) yr[16 * j] = acc[i][j][r] * sc;
        } else {
          const float sa = a_rs[row0 + ro];
          const float* ws = reinterpret_cast<const float*>(wsc) + (int64_t)e * H + c0 + wn * 64 + m;
#pragma unroll
          for (int j = 0; j < 4; ++j) yr[16 * j] = acc[i][j][r] * sa * ws[16 * j];
        }
      }
    }
  }
  if constexpr (G1 && NV) wg_amax_atomic(hmax, h_amax);
}

// ---------------------------------------------------------------------------
// Grouped GEMM for many rows per expert on the 32x32x16 matrix cores ("big"):
// 128 rows x 256 weight rows per workgroup, 4 waves of 128 rows x 64 weight
// rows (4 x 2 MFMA tiles of 32 x 32, 128 accumulators per lane), K in steps
// of 64 staged through LDS (double buffered; the next step's global loads go
// to registers during the current step).  The activation tile is staged as
// FP16 (W4A16: BF16); the weight tile as raw codes and scale bytes.  Each
// weight fragment is used by exactly one wave, which decodes it once for all
// 128 rows.  GEMM1 workgroup: weight rows = 128 gate rows c0.. and the 128
// matching up rows; each wave holds g and u of the same 32 h columns, so
// SwiGLU fuses into the epilogue.
// MFMA 32x32x16 operands: lane l carries row / column l % 32 and k values
// 8 (l / 32) .. +7 of the 16; result register 4q + j of lane l is row
// 8q + 4 (l / 32) + j, column l % 32.
// ---------------------------------------------------------------------------
constexpr int kGBM = 128, kGBN = 256, kGBK = 64;
// Fourth word of a raw buffer descriptor (stride 0, byte offsets): 32-bit data format, as the buffer
// instructions of gfx9-family GPUs expect; records up to 2^31 bytes from the base, far beyond one expert.
constexpr int kBufDword3 = 0x00020000;
template <int N>
struct IntC {
  static constexpr int value = N;
};
template <bool NV>
struct BigB {
  static constexpr int kRow = NV ? 36 : 72;  // LDS bytes per weight row and K step (+4 / +8 pad)
};
typedef float f16v __attribute__((ext_vector_type(16)));
template <bool A16>
__device__ inline f16v mfma32(h8v a, h8v b, f16v c) {
  if constexpr (A16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8v, a), __builtin_bit_cast(bf8v, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <bool NV, bool G1, bool A16 = false, bool QA = false>
__global__ __launch_bounds__(256, 2) void k_gemm_big(const _Float16* __restrict__ act, const int* __restrict__ row_pair,
                                                     int topk, const float* __restrict__ a_gs,
                                                     const float* __restrict__ a_rs, const uint8_t* __restrict__ wc,
                                                     const uint8_t* __restrict__ wsc, const float* __restrict__ wgs,
                                                     const int4* __restrict__ tiles, const int* __restrict__ ntiles,
                                                     int64_t K, int64_t H, int64_t I, float* __restrict__ out,
                                                     uint32_t* __restrict__ h_amax, const uint8_t* __restrict__ acodes,
                                                     const uint8_t* __restrict__ ascales, int pairs) {
  constexpr int kBRow = BigB<NV>::kRow;
  // Weights come in groups of GS K steps, 128 code bytes per row (one cache line, loaded by 8 lanes;
  // NVFP4 4 steps with K % 256 == 0, FP8 2 steps with K % 128 == 0), into one LDS buffer that the
  // group's steps read.  Per-step pieces of 32 or 64 bytes left the lines to be evicted between steps.
  constexpr int GS = NV ? 4 : 2;               // K steps per weight group
  constexpr int kSB = NV ? kGBK / 2 : kGBK;    // code bytes per row and K step
  constexpr int kGP = NV ? 132 : 136;          // LDS bytes per weight row of a group (+pad: conflict-free reads)
  (void)kBRow;
  // NVFP4 (and W4A16): the activation tile is written by direct-to-LDS loads (lane l of a load -> 16
  // bytes at base + 16 l, so a load fills 8 whole 128-byte rows): unpadded rows, 16-byte chunk c of
  // row r stored at chunk c ^ ((r >> 1) & 7), which keeps the fragment reads of 16 consecutive rows
  // on distinct banks.  FP8 (measured slower that way) stages it through registers into padded rows.
  // QA: the tile is staged from the activation codes (NVFP4 codes and block scales, FP8 codes; acodes,
  // ascales) and decoded to FP16 on the way into LDS, through registers: thread t takes 32 values of row
  // t / 2, so no FP16 copy of the activations is read (or written before).
  // Two separate arrays, so the compiler sees that loads into one do not alias reads of the other.
  constexpr bool kAdma = NV && !QA;
  constexpr int kAS = kAdma ? kGBK : kGBK + 8;  // LDS row stride (f16)
  __shared__ __attribute__((aligned(16))) _Float16 As0[kGBM][kAS];
  __shared__ __attribute__((aligned(16))) _Float16 As1[kGBM][kAS];
  _Float16* const Ab[2] = {&As0[0][0], &As1[0][0]};
  __shared__ __attribute__((aligned(16))) uint8_t Bg[kGBN][kGP];
  __shared__ uint32_t Bsc[GS][kGBN];  // NVFP4: scale dwords of the group's weight rows, by K step
  if ((int)blockIdx.y >= *ntiles) return;
  const int4 ti = tiles[blockIdx.y];
  const int e = ti.x, row0 = ti.y, nrows = ti.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, lh = lane >> 5;
  const int64_t c0 = (int64_t)blockIdx.x * (G1 ? kGBN / 2 : kGBN);
  // Staging: each load instruction covers whole row segments with consecutive
  // lanes (8 lanes per 128-byte activation row segment, 2 (FP8: 4) lanes per
  // weight row segment), so one instruction touches few cache lines.
  // Activation rows ar(i) = 32 i + tid / 8, 16-byte part tid % 8.
  constexpr int kBI = 8;  // weight rows per thread and group: kGBN / (256 / kBP)
  constexpr int kBP = 8;  // 16-byte parts per weight row and group
  const int apart = tid & 7, bpart = tid & (kBP - 1);
  // direct-to-LDS: load i of wave w fills rows 32 w + 8 i .. + 7; lane l writes chunk l % 8 of row
  // 32 w + 8 i + l / 8, which holds the row's logical chunk (l % 8) ^ ((row >> 1) & 7).
  // Through registers: rows 32 i + tid / 8, 16-byte part tid % 8.
  auto arow = [&](int i) -> const _Float16* {
    const int r = kAdma ? 32 * wave + 8 * i + (lane >> 3) : 32 * i + (tid >> 3);
    const int ar = r < nrows ? r : nrows - 1;
    const int c = kAdma ? (lane & 7) ^ ((r >> 1) & 7) : apart;
    return (G1 ? act + (int64_t)(row_pair[row0 + ar] / topk) * K : act + (int64_t)(row0 + ar) * K) + 8 * c;
  };
  const _Float16 *as0 = QA ? nullptr : arow(0), *as1 = QA ? nullptr : arow(1), *as2 = QA ? nullptr : arow(2),
                 *as3 = QA ? nullptr : arow(3);
  // QA: row qr = tid / 2, values 32 qh .. +31 of each K step (qh = tid % 2)
  const int qr = tid >> 1, qh = tid & 1;
  const uint8_t *qc = nullptr, *qs = nullptr;
  if constexpr (QA) {
    const int ar = qr < nrows ? qr : nrows - 1;
    const int64_t ri = G1 ? (int64_t)(row_pair[row0 + ar] / topk) : (int64_t)(row0 + ar);
    qc = acodes + ri * (NV ? K / 2 : K) + (NV ? 16 : 32) * qh;
    qs = NV ? ascales + ri * (K / 16) : nullptr;
  }
  uint4 qa0 = make_uint4(0, 0, 0, 0), qa1 = make_uint4(0, 0, 0, 0);
  uint32_t qsw = 0;
  // weight row r of the tile: GEMM1 gate rows c0.. then the matching up rows
  auto wrow_of = [&](int r) -> int64_t {
    if (G1) return (int64_t)e * 2 * I + (r < kGBN / 2 ? c0 + r : I + c0 + (r - kGBN / 2));
    return (int64_t)e * H + c0 + r;
  };
  const int64_t cbytes = NV ? K / 2 : K;
  // Weight (and scale) loads are buffer loads: a descriptor of the tile's first weight row (uniform), a
  // 32-bit per-lane byte offset (within one expert) and the K step's offset in a scalar register, so no
  // vector instruction computes an address inside the K loop.
  const uint8_t* bbase = wc + wrow_of(0) * cbytes;
  const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(bbase), (short)0,
                                                                       0x7FFFFFFF, kBufDword3);
  // Pair layout (pairs != 0; 16-row blocks of double rows, see b_load_pairs): load i of lane tid takes the
  // 16-byte part tid % 8 of line (256 i + tid) / 8 of the group, which holds 64 bytes of row p and then of
  // row p + 8 of a 16-row block.  Its row in the tile is 32 i + brow0 and its bytes in the row's group
  // bcol .. +15 (canonical rows: row 32 i + tid / 8, part tid % 8); the group of K step s starts at byte
  // s * kSB of a row, at 2 s * kSB of a double row.
  const int brow0 = pairs ? 16 * (tid >> 7) + ((tid >> 4) & 7) + (((tid & 7) >> 2) << 3) : tid / kBP;
  // Weight row r of the tile sits in group-buffer row r ^ (bit 3 of r moved to bit 1): rows are 33 dwords
  // apart, so a pair-layout store's rows p and p + 8 (same bytes of both) would share banks; permuted they
  // fall on four different banks mod 4, and the fragment reads of 32 consecutive rows stay on 32 banks.
  auto bg_row = [](int r) { return r ^ (((r >> 3) & 1) << 1); };
  const int bcol = pairs ? ((tid >> 3) & 1) * 64 + (tid & 3) * 16 : 16 * bpart;
  const int smul = pairs ? 2 : 1;
  auto boff_of = [&](int i) -> uint32_t {
    if (pairs)
      return (uint32_t)((wrow_of(32 * i + 16 * (tid >> 7)) - wrow_of(0)) * cbytes + ((tid >> 4) & 7) * 2 * cbytes +
                        ((tid >> 3) & 1) * 128 + ((tid & 7) >> 2) * 64 + (tid & 3) * 16);
    return (uint32_t)((wrow_of((256 / kBP) * i + tid / kBP) - wrow_of(0)) * cbytes + 16 * bpart);
  };
  uint32_t bo[kBI];
#pragma unroll
  for (int i = 0; i < kBI; ++i) bo[i] = boff_of(i);
  // scale bytes: thread tid holds weight row tid; 16 bytes (the 4 K steps of a group) per load
  const uint8_t* sbase = NV ? wsc + wrow_of(0) * (K / 16) : wc;
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sbase), (short)0,
                                                                       0x7FFFFFFF, kBufDword3);
  // (the block scales are row-major in both code layouts: the lane-ordered copy is the few-row GEMM's)
  const uint32_t soff = NV ? (uint32_t)((wrow_of(tid) - wrow_of(0)) * (K / 16)) : 0u;

  uint4 ra0, ra1, ra2, ra3, rb[kBI], sc4 = make_uint4(0, 0, 0, 0);
  auto aload = [&](int s, _Float16* __restrict__ wr) {  // activations of K step s (into LDS tile wr)
    if constexpr (QA) {
      (void)wr;
      if constexpr (NV) {
        qa0 = *reinterpret_cast<const uint4*>(qc + (int64_t)s * (kGBK / 2));
        qsw = *reinterpret_cast<const uint32_t*>(qs + (int64_t)s * (kGBK / 16));
      } else {
        qa0 = *reinterpret_cast<const uint4*>(qc + (int64_t)s * kGBK);
        qa1 = *reinterpret_cast<const uint4*>(qc + (int64_t)s * kGBK + 16);
      }
    } else if constexpr (kAdma) {
      __builtin_amdgcn_global_load_lds(as0 + s * kGBK, wr + (32 * wave) * kGBK, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(as1 + s * kGBK, wr + (32 * wave + 8) * kGBK, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(as2 + s * kGBK, wr + (32 * wave + 16) * kGBK, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(as3 + s * kGBK, wr + (32 * wave + 24) * kGBK, 16, 0, 0);
    } else {
      ra0 = *reinterpret_cast<const uint4*>(as0 + s * kGBK);
      ra1 = *reinterpret_cast<const uint4*>(as1 + s * kGBK);
      ra2 = *reinterpret_cast<const uint4*>(as2 + s * kGBK);
      ra3 = *reinterpret_cast<const uint4*>(as3 + s * kGBK);
    }
  };
  auto bload = [&](int s) {  // weight codes (and NVFP4 scale bytes) of the group that starts at K step s
#pragma unroll
    for (int i = 0; i < kBI; ++i)
      rb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(brs, bo[i], s * kSB * smul, 0));
    if constexpr (NV) sc4 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(srs, soff, 4 * s, 0));
  };
  auto bstore = [&]() {  // weight registers of a group into the group buffer, scale dwords by K step
#pragma unroll
    for (int i = 0; i < kBI; ++i) {
      uint32_t* d = reinterpret_cast<uint32_t*>(&Bg[bg_row(32 * i + brow0)][bcol]);
      d[0] = rb[i].x;
      d[1] = rb[i].y;
      d[2] = rb[i].z;
      d[3] = rb[i].w;
    }
    if constexpr (NV) {
      Bsc[0][tid] = sc4.x;
      Bsc[1][tid] = sc4.y;
      Bsc[2][tid] = sc4.z;
      Bsc[3][tid] = sc4.w;
    }
  };
  // Direct-to-LDS: this wave's loads are complete once at most n later loads are in flight (loads
  // complete in issue order); the barrier after it publishes every wave's rows.  Through
  // registers: the activation registers into LDS tile buf.
  auto lstore = [&](int buf, int n) {
    if constexpr (QA) {  // decode the row's 32 values: NVFP4 two blocks (scale bytes 2 qh, 2 qh + 1)
      (void)n;
      uint4 o[4];
      if constexpr (NV) {
        const uint32_t sa = (uint32_t)(2 * qh) * 0x0101u, sb = sa + 0x0101u;
        const h2v s2a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__builtin_amdgcn_perm(qsw, qsw, sa), 1.0f, false);
        const h2v s2b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__builtin_amdgcn_perm(qsw, qsw, sb), 1.0f, false);
        o[0] = __builtin_bit_cast(uint4, dec_fp4x8(qa0.x, s2a));
        o[1] = __builtin_bit_cast(uint4, dec_fp4x8(qa0.y, s2a));
        o[2] = __builtin_bit_cast(uint4, dec_fp4x8(qa0.z, s2b));
        o[3] = __builtin_bit_cast(uint4, dec_fp4x8(qa0.w, s2b));
      } else {
        o[0] = __builtin_bit_cast(uint4, dec_fp8x8(qa0.x, qa0.y));
        o[1] = __builtin_bit_cast(uint4, dec_fp8x8(qa0.z, qa0.w));
        o[2] = __builtin_bit_cast(uint4, dec_fp8x8(qa1.x, qa1.y));
        o[3] = __builtin_bit_cast(uint4, dec_fp8x8(qa1.z, qa1.w));
      }
      uint4* d = reinterpret_cast<uint4*>(Ab[buf] + qr * kAS + 32 * qh);
      d[0] = o[0];
      d[1] = o[1];
      d[2] = o[2];
      d[3] = o[3];
    } else if constexpr (kAdma) {
      if (n == 0)
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt not waited for
      else
        __builtin_amdgcn_s_waitcnt(0x0F70 | (kBI + 1));  // vmcnt(the group's weight and scale loads)
    } else {
      _Float16* d = Ab[buf] + (tid >> 3) * kAS + 8 * apart;
      *reinterpret_cast<uint4*>(d) = ra0;
      *reinterpret_cast<uint4*>(d + 32 * kAS) = ra1;
      *reinterpret_cast<uint4*>(d + 64 * kAS) = ra2;
      *reinterpret_cast<uint4*>(d + 96 * kAS) = ra3;
    }
  };
  // Workgroup barrier.  With direct-to-LDS loads, __syncthreads() (also a workgroup release fence)
  // would make the compiler wait for every load in flight, the next weight group's included, since
  // such a load writes LDS.  There: this wave's LDS accesses complete (lgkmcnt(0)), the barrier, and
  // compiler-only fences that keep memory accesses on their side of it; the direct-to-LDS loads are
  // waited for explicitly in lstore.
  auto lds_barrier = []() {
    if constexpr (kAdma) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt(63), expcnt(7): not waited for
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    } else {
      __syncthreads();
    }
  };
  // LDS weight row of this wave's N tile t: GEMM1 gate tile 0 / up tile 1; GEMM2 2 consecutive
#define BSM_BIG_BROW(t) (G1 ? ((t) == 0 ? 32 * wave : kGBN / 2 + 32 * wave) : 64 * wave + 32 * (t))

  f16v acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mt][t][q] = 0.0f;

  // The K loop is compiled for MT = 1..4 live 32-row sub-tiles (MT = ceil(nrows / 32), uniform per
  // workgroup): the last, ragged row tile of an expert skips the multiplies and fragment reads of its
  // empty sub-tiles.
  auto kloop = [&](auto mtc) {
    constexpr int MT = decltype(mtc)::value;
    // K step j of the current group from LDS buffer buf
    // rd: the activation tile of this K step (rows of kAS; swizzled chunks with direct-to-LDS staging)
    auto mma_step = [&](int j, const _Float16* __restrict__ rd) {
      // NVFP4: the step's four block scales of each weight row as FP16, two converts per row and step
      h2v s01[2], s23[2];
      if constexpr (NV) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t sw = Bsc[j][BSM_BIG_BROW(t) + l32];
          s01[t] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
          s23[t] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true);
        }
      }
#pragma unroll
      for (int k16 = 0; k16 < kGBK / 16; ++k16) {
        h8v a[4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          a[mt] = *reinterpret_cast<const h8v*>(
              rd + (mt * 32 + l32) * kAS + (kAdma ? 8 * ((2 * k16 + lh) ^ ((l32 >> 1) & 7)) : k16 * 16 + lh * 8));
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int brow = bg_row(BSM_BIG_BROW(t) + l32);
          h8v b;
          if constexpr (NV) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(&Bg[brow][j * 32 + k16 * 8 + lh * 4]);
            const _Float16 sk = k16 == 0 ? s01[t][0] : k16 == 1 ? s01[t][1] : k16 == 2 ? s23[t][0] : s23[t][1];
            const h2v s2 = {sk, sk};
            if constexpr (A16)
              b = dec_fp4x8_bf16(w, (float)sk);
            else
              b = dec_fp4x8(w, s2);
          } else {
            const uint2 w = *reinterpret_cast<const uint2*>(&Bg[brow][j * 64 + k16 * 16 + lh * 8]);
            b = dec_fp8x8(w.x, w.y);
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][t] = mfma32<A16>(a[mt], b, acc[mt][t]);
        }
      }
    };

    // The K loop runs over weight groups with the group's steps unrolled, so no load sits under a
    // branch (indices past the end are clamped to the last step or group and their data is never
    // read) and the wait counts stay exact.  A step's activations load one step ahead; a group's
    // weights load two steps ahead, after the activations of that step, so that the activation
    // store of the step before the group boundary does not wait for them.
    const int nk = (int)(K / kGBK), ng = nk / GS;
    // The step's loads and multiplies in one function whose two tile pointers are restrict-qualified:
    // the compiler then knows the direct-to-LDS writes into one buffer do not alias the reads of the
    // other, and does not make the reads wait for the writes.
    auto issue_and_multiply = [&](int j, int snext, int gnext, _Float16* __restrict__ wr,
                                  const _Float16* __restrict__ rd) {
      aload(snext, wr);
      if (j == GS - 2) bload(gnext);
      __builtin_amdgcn_sched_barrier(0);  // the scheduler would otherwise sink the loads to their stores
      mma_step(j, rd);
    };
    aload(0, Ab[0]);
    bload(0);
    bstore();
    lstore(0, 0);
    __syncthreads();
    for (int gi = 0; gi < ng; ++gi) {
#pragma unroll
      for (int j = 0; j < GS; ++j) {
        const int ks = gi * GS + j;  // GS is even, so ks & 1 == j & 1
        issue_and_multiply(j, ks + 1 < nk ? ks + 1 : ks, gi + 1 < ng ? (gi + 1) * GS : gi * GS,
                           Ab[(j & 1) ^ 1], Ab[j & 1]);
        if (j == GS - 1) {  // next group: every wave has finished reading the current one
          lds_barrier();
          bstore();
        }
        lstore((j & 1) ^ 1, j == GS - 2);
        lds_barrier();
      }
    }
  };
  const int live = (nrows + 31) / 32;
  if (live >= 4)
    kloop(IntC<4>{});
  else if (live == 3)
    kloop(IntC<3>{});
  else if (live == 2)
    kloop(IntC<2>{});
  else
    kloop(IntC<1>{});
#undef BSM_BIG_BROW

  // Epilogue.  Accumulator register 4q + j of m tile mt is row mt * 32 + 8q + 4 (lane / 32) + j and
  // column lane % 32 of the wave's 32-column tile: one base address per lane, and every other element
  // sits a wave-uniform number of rows further.  Full tiles skip the row checks.
  float hmax = 0.0f;
  const int64_t ld = G1 ? I : H;
  float* const obase = out + (int64_t)(row0 + 4 * lh) * ld + (G1 ? c0 + 32 * wave + l32 : c0 + 64 * wave + l32);
  const bool full = nrows == kGBM;
  float sg = 0.0f, su = 0.0f, sy = 0.0f;  // NVFP4: the product of the global scales
  if constexpr (NV) {
    const float ag = A16 ? 1.0f : a_gs[0];  // weight-only: BF16 activations carry no scale
    if (G1) {
      sg = ag * wgs[2 * e];
      su = ag * wgs[2 * e + 1];
    } else {
      sy = ag * wgs[e];
    }
  }
  const float* wsf = reinterpret_cast<const float*>(wsc);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = mt * 32 + 8 * q + j;  // row offset from this lane's base row
        if (!full && rr + 4 * lh >= nrows) continue;
        const int r = 4 * q + j;
        float* const p = obase + (int64_t)rr * ld;
        if (G1) {
          float g = acc[mt][0][r], u = acc[mt][1][r];
          if (NV) {
            g *= sg;
            u *= su;
          } else {
            const int64_t col = c0 + 32 * wave + l32;
            const float sx = a_rs[row_pair[row0 + rr + 4 * lh] / topk];
            g *= sx * wsf[(int64_t)e * 2 * I + col];
            u *= sx * wsf[(int64_t)e * 2 * I + I + col];
          }
          const float h = silu_mul(g, u);
          p[0] = h;
          hmax = fmaxf(hmax, fabsf(h));
        } else {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if (NV) {
              p[32 * t] = acc[mt][t][r] * sy;
            } else {
              const int64_t col = c0 + 64 * wave + 32 * t + l32;
              p[32 * t] = acc[mt][t][r] * a_rs[row0 + rr + 4 * lh] * wsf[(int64_t)e * H + col];
            }
          }
        }
      }
    }
  }
  if constexpr (G1 && NV) wg_amax_atomic(hmax, h_amax);
}

// ---------------------------------------------------------------------------
// combine
// ---------------------------------------------------------------------------
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y, const int* __restrict__ pair_row,
                                                 const float* __restrict__ wts, int topk, int64_t H, double scale,
                                                 float* __restrict__ out) {
  const int64_t t = blockIdx.y;
  const int64_t c4 = (int64_t)blockIdx.x * 256 + threadIdx.x;  // float4 column index
  if (c4 * 4 >= H) return;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int j0 = 0; j0 < topk; j0 += 8) {
    // all row indices, then all y loads of up to 8 slots in flight; the sum stays in slot order
    int row[8];
    double w[8];
    bool in[8];  // slot present and its pair not dropped (expert id outside [0, E))
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool slot = j0 + q < topk;
      row[q] = slot ? pair_row[t * topk + j0 + q] : -1;
      in[q] = row[q] >= 0;
      w[q] = in[q] ? (double)wts[t * topk + j0 + q] : 0.0;
    }
    // y is read once: non-temporal loads keep it from displacing cached data (0.30 -> 0.25 ms at 8192 tokens)
    float4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const f32x4_t z = in[q]
                            ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(y + (int64_t)row[q] * H + c4 * 4))
                            : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      v[q] = make_float4(z.x, z.y, z.z, z.w);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (in[q]) {
        acc[0] += w[q] * (double)v[q].x;
        acc[1] += w[q] * (double)v[q].y;
        acc[2] += w[q] * (double)v[q].z;
        acc[3] += w[q] * (double)v[q].w;
      }
    }
  }
  *reinterpret_cast<float4*>(out + t * H + c4 * 4) =
      make_float4((float)(scale * acc[0]), (float)(scale * acc[1]), (float)(scale * acc[2]), (float)(scale * acc[3]));
}

__global__ void k_copy_f32(const float* src, float* dst) {
  if (threadIdx.x == 0) dst[0] = src[0];
}

// Batches of at most one 64-token chunk (decode): masks, counts, offsets,
// tile lists and rows in one workgroup.  Same results as the three kernels
// above with a single chunk.
__global__ __launch_bounds__(1024) void k_perm_small(const int32_t* __restrict__ ids, int64_t T, int topk, int64_t E,
                                                     int* __restrict__ counts, int* __restrict__ offsets,
                                                     int4* __restrict__ tiles_s, int* __restrict__ ntiles_s,
                                                     int4* __restrict__ tiles_w, int* __restrict__ ntiles_w,
                                                     int* __restrict__ row_pair, int* __restrict__ pair_row,
                                                     uint32_t* __restrict__ h_amax) {
  __shared__ unsigned long long lm[1024];
  __shared__ int s_cnt[1024];
  __shared__ int wtot[16][3];
  const int e = threadIdx.x;
  lm[e] = 0ull;
  __syncthreads();
  const int64_t P = T * topk;
  for (int64_t p = threadIdx.x; p < P; p += 1024) {
    const int ex = ids[p];
    if ((uint32_t)ex < (uint32_t)E) atomicOr(&lm[ex], 1ull << (p / topk));  // ids outside [0, E) are dropped
  }
  __syncthreads();
  const int total = (e < E) ? __popcll(lm[e]) : 0;
  if (e < E) counts[e] = total;
  const bool skinny = total <= kSkinnyMaxRows;
  const int nts = (e < E && skinny) ? (total + kRowsPerTile - 1) / kRowsPerTile : 0;
  const int ntw = (e < E && !skinny) ? (total + kWideRows - 1) / kWideRows : 0;
  int sc = total, st = nts, sw = ntw;
  block_scan3_1024(sc, st, sw, wtot);
  s_cnt[e] = sc;  // inclusive prefix counts, read by every thread below
  if (e < E) {
    const int off = sc - total;
    offsets[e] = off;
    if (e == E - 1) {
      offsets[E] = sc;
      *ntiles_s = st;
      *ntiles_w = sw;
    }
    const int ts0 = st - nts, tw0 = sw - ntw;
    for (int i = 0; i < nts; ++i) {
      const int r = total - i * kRowsPerTile;
      tiles_s[ts0 + i] = make_int4(e, off + i * kRowsPerTile, r < kRowsPerTile ? r : kRowsPerTile, 0);
    }
    for (int i = 0; i < ntw; ++i) {
      const int r = total - i * kWideRows;
      tiles_w[tw0 + i] = make_int4(e, off + i * kWideRows, r < kWideRows ? r : kWideRows, 0);
    }
  }
  if (e == 0) *h_amax = 0u;
  __syncthreads();  // s_cnt holds inclusive prefix counts
  for (int64_t p = threadIdx.x; p < P; p += 1024) {
    const int ex = ids[p];
    if ((uint32_t)ex >= (uint32_t)E) {
      pair_row[p] = -1;
      continue;
    }
    const uint32_t bit = (uint32_t)(p / topk);
    const uint64_t below = bit ? (lm[ex] & ((1ull << bit) - 1ull)) : 0ull;
    const int pos = s_cnt[ex] - __popcll(lm[ex]) + __popcll(below);
    row_pair[pos] = (int)p;
    pair_row[p] = pos;
  }
}

// h (FP32) -> BF16, round to nearest even (weight-only path's 16-bit activations); finite inputs
__global__ __launch_bounds__(256) void k_h_to_bf16(const float* __restrict__ h, int64_t n4, uint16_t* __restrict__ o) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4 v = reinterpret_cast<const float4*>(h)[i];
  const float f[4] = {v.x, v.y, v.z, v.w};
  uint32_t r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t b = f2u(f[q]);
    r[q] = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
  }
  reinterpret_cast<uint2*>(o)[i] = make_uint2(r[0] | (r[1] << 16), r[2] | (r[3] << 16));
}

// Dense linear: all T rows belong to one weight matrix ("expert" 0).  At most
// kSkinnyMaxRows rows use 16-row tiles of the register-streaming kernel, more
// use 128-row tiles of the LDS-tiled kernel (weights read once per 128 rows).
__global__ void k_dense_tiles(int64_t T, int4* __restrict__ tiles_s, int* __restrict__ ntiles_s,
                              int4* __restrict__ tiles_w, int* __restrict__ ntiles_w, uint32_t* __restrict__ amax) {
  const bool skinny = T <= kSkinnyMaxRows;
  const int nts = skinny ? (int)((T + kRowsPerTile - 1) / kRowsPerTile) : 0;
  const int ntw = skinny ? 0 : (int)((T + kWideRows - 1) / kWideRows);
  for (int i = threadIdx.x; i < nts; i += blockDim.x) {
    const int64_t r = T - (int64_t)i * kRowsPerTile;
    tiles_s[i] = make_int4(0, i * kRowsPerTile, r < kRowsPerTile ? (int)r : kRowsPerTile, 0);
  }
  for (int i = threadIdx.x; i < ntw; i += blockDim.x) {
    const int64_t r = T - (int64_t)i * kWideRows;
    tiles_w[i] = make_int4(0, i * kWideRows, r < kWideRows ? (int)r : kWideRows, 0);
  }
  if (threadIdx.x == 0) {
    *ntiles_s = nts;
    *ntiles_w = ntw;
    *amax = 0u;
  }
}

struct LinLayout {
  size_t act, tiles_s, ntiles_s, tiles_w, ntiles_w, amax, part, total;
  int64_t max_s, max_w;
};

LinLayout lin_layout(int64_t T, int64_t K, int64_t N) {
  LinLayout L{};
  L.max_s = (kSkinnyMaxRows + kRowsPerTile - 1) / kRowsPerTile;
  L.max_w = (T + kWideRows - 1) / kWideRows;
  size_t o = 0;
  auto take = [&](size_t n) {
    const size_t r = o;
    o += align256(n);
    return r;
  };
  L.act = take(2 * (size_t)T * (size_t)K);
  L.tiles_s = take(sizeof(int4) * L.max_s);
  L.ntiles_s = take(sizeof(int));
  L.tiles_w = take(sizeof(int4) * (L.max_w > 0 ? L.max_w : 1));
  L.ntiles_w = take(sizeof(int));
  L.amax = take(sizeof(uint32_t));
  // split-K partial sums of the dense kernel (T <= kDenseRows)
  L.part = take(T <= kDenseRows ? sizeof(float) * kDenseMaxSplits * (size_t)T * (size_t)N : 16);
  L.total = o;
  return L;
}

}  // namespace

size_t fp8_linear_ws(int64_t T, int64_t K, int64_t N) { return lin_layout(T, K, N).total; }

hipError_t launch_fp8_linear(const uint8_t* xc, const float* xs, const uint8_t* wc, const float* wsc, int64_t T,
                             int64_t K, int64_t N, float* out, uint8_t* ws, hipStream_t st) {
  const LinLayout L = lin_layout(T, K, N);
  if (T == 0) return hipSuccess;
  if (T <= kDenseRows)  // every workgroup covers all rows; weights streamed once
    return launch_dense_f8<false>(xc, xs, T, K, wc, wsc, N, 0, out, reinterpret_cast<float*>(ws + L.part), st);
  _Float16* act = reinterpret_cast<_Float16*>(ws + L.act);
  int4* tiles_s = reinterpret_cast<int4*>(ws + L.tiles_s);
  int* ntiles_s = reinterpret_cast<int*>(ws + L.ntiles_s);
  int4* tiles_w = reinterpret_cast<int4*>(ws + L.tiles_w);
  int* ntiles_w = reinterpret_cast<int*>(ws + L.ntiles_w);
  uint32_t* amax = reinterpret_cast<uint32_t*>(ws + L.amax);
  k_dense_tiles<<<1, 64, 0, st>>>(T, tiles_s, ntiles_s, tiles_w, ntiles_w, amax);
  const int64_t xblk = T * K / 16;
  k_decode_act<false><<<(unsigned)((xblk + 255) / 256), 256, 0, st>>>(xc, nullptr, xblk, act);
  const dim3 gs((unsigned)(N / (64 * kSkNT)), (unsigned)L.max_s);
  const dim3 gw((unsigned)(N / 128), (unsigned)(L.max_w > 0 ? L.max_w : 1));
  if (T <= kSkinnyMaxRows) {
    if (K % (4 * kF8KB) == 0)
      k_skinny<false, false, kF8KB, kSkNT><<<gs, 256, 0, st>>>(
          act, nullptr, 1, nullptr, xs, wc, reinterpret_cast<const uint8_t*>(wsc), nullptr, tiles_s, ntiles_s, K, N, 0,
          out, amax);
    else
      k_skinny<false, false, 32, kSkNT><<<gs, 256, 0, st>>>(
          act, nullptr, 1, nullptr, xs, wc, reinterpret_cast<const uint8_t*>(wsc), nullptr, tiles_s, ntiles_s, K, N, 0,
          out, amax);
  } else {
    k_gemm_wide<false, false><<<gw, 256, 0, st>>>(act, nullptr, 1, nullptr, xs, wc,
                                                  reinterpret_cast<const uint8_t*>(wsc), nullptr, tiles_w, ntiles_w, K,
                                                  N, 0, out, amax);
  }
  return hipGetLastError();
}

MoeLayout moe_layout(bool nvfp4, int64_t E, int64_t H, int64_t I, int64_t T, int topk) {
  MoeLayout L{};
  L.P = T * topk;
  L.n_chunks = (T + kChunk - 1) / kChunk;
  constexpr int64_t kMaxSkinnyTiles = (kSkinnyMaxRows + kRowsPerTile - 1) / kRowsPerTile;
  L.max_tiles = std::min<int64_t>(kMaxSkinnyTiles * E, L.P / kRowsPerTile + E) + 1;  // skinny tiles
  // many-row tiles: sum over experts above kFewRowsMulti rows of ceil(rows / kWideRows), at most
  // P / kWideRows plus one partial tile per such expert
  L.max_tiles_w = L.P / kWideRows + std::min<int64_t>(E, L.P / (kFewRowsMulti + 1)) + 1;
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
  L.act_f16 = take(2 * (size_t)T * H);
  L.h_f16 = take(2 * (size_t)L.P * I);
  L.scratch = o;
  L.sel_masks = take(sizeof(uint64_t) * E * L.n_chunks);
  L.chunk_cnt = take(sizeof(int) * E * L.n_chunks);
  L.chunk_base = take(sizeof(int) * E * L.n_chunks);
  L.ntiles = take(sizeof(int));
  L.tiles_w = take(sizeof(int4) * L.max_tiles_w);
  L.ntiles_w = take(sizeof(int));
  L.h_amax = take(sizeof(uint32_t));
  // split-K partial sums of the dense FP8 kernel (one expert, top-1, at most kDenseRows tokens)
  const bool dense = !nvfp4 && E == 1 && topk == 1 && T <= kDenseRows;
  L.part = take(dense ? sizeof(float) * kDenseMaxSplits * (size_t)T * (size_t)std::max<int64_t>(2 * I, H) : 16);
  L.total = o;
  return L;
}

namespace {

// Pair layout of weight codes, out of place: 16-byte unit u of row r goes to block r / 16, double row
// (r % 16) % 8, 128-byte line u / 4 of it, half (r % 16) / 8, unit u % 4 (see b_load_pairs).
__global__ __launch_bounds__(256) void k_codes_to_pairs(const uint4* __restrict__ in, uint4* __restrict__ out,
                                                        int64_t n, int64_t ru) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 16-byte unit of the input
  if (i >= n) return;
  const int64_t r = i / ru, u = i - r * ru;
  const int64_t m = r & 15;
  out[(r - m) * ru + (m & 7) * 2 * ru + (u >> 2) * 8 + (m >> 3) * 4 + (u & 3)] = in[i];
}

// Lane order of NVFP4 block scales, out of place: row r's 32 scale bytes of super-step st (512 values) go to
// 16-row block r / 16, super-step st, row r % 16, block b to byte ((b >> 1) & 3) * 8 + (b >> 3) * 2 + (b & 1):
// lane group g of the few-row GEMM finds the two blocks of each of its four pieces as 8 consecutive bytes
// (one load; two dword loads per lane measured slower, decode-64 0.865 -> 0.90 ms).  The many-row GEMM keeps
// the row-major scales: its weight groups take 16 blocks of a row at a time (prefill-8192 gate/up 3.03 ->
// 3.16 ms reading this order).
__global__ __launch_bounds__(256) void k_scales_to_lanes(const uint8_t* __restrict__ in, uint8_t* __restrict__ out,
                                                         int64_t n, int64_t nst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (row, super-step) span of 32 bytes
  if (i >= n) return;
  const int64_t r = i / nst, st = i - r * nst;
  const uint4* src = reinterpret_cast<const uint4*>(in + (r * nst + st) * 32);
  const uint4 a = src[0], c = src[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
  uint32_t o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int b = 0; b < 32; ++b) {
    const uint32_t v = (w[b >> 2] >> (8 * (b & 3))) & 0xFFu;
    const int q = ((b >> 1) & 3) * 8 + (b >> 3) * 2 + (b & 1);
    o[q >> 2] |= v << (8 * (q & 3));
  }
  uint4* dst = reinterpret_cast<uint4*>(out + (((r >> 4) * nst + st) * 16 + (r & 15)) * 32);
  dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
  dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// k_skinny_rows for the canonical or the pair layout of the weight codes
template <bool NV, bool G1, bool A16, int DEPTH, bool QA, typename... Args>
void launch_skr(bool pairs, dim3 grid, hipStream_t st, Args... args) {
  if (pairs)
    k_skinny_rows<NV, G1, kSkNT, A16, DEPTH, QA, true><<<grid, 256, 0, st>>>(args...);
  else
    k_skinny_rows<NV, G1, kSkNT, A16, DEPTH, QA, false><<<grid, 256, 0, st>>>(args...);
}

}  // namespace

hipError_t launch_scales_to_lanes(const uint8_t* in, uint8_t* out, int64_t rows, int64_t row_bytes, hipStream_t st) {
  const int64_t nst = row_bytes / 32, n = rows * nst;
  if (n == 0) return hipSuccess;
  k_scales_to_lanes<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(in, out, n, nst);
  return hipGetLastError();
}

hipError_t launch_codes_to_pairs(const uint8_t* in, uint8_t* out, int64_t rows, int64_t row_bytes, hipStream_t st) {
  const int64_t ru = row_bytes / 16, n = rows * ru;
  if (n == 0) return hipSuccess;
  k_codes_to_pairs<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(reinterpret_cast<const uint4*>(in),
                                                                 reinterpret_cast<uint4*>(out), n, ru);
  return hipGetLastError();
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
  int4* tiles_w = reinterpret_cast<int4*>(ws + L.tiles_w);
  int* ntiles_w = reinterpret_cast<int*>(ws + L.ntiles_w);
  uint32_t* h_amax = reinterpret_cast<uint32_t*>(ws + L.h_amax);

  stage_mark(0, 0, st);
  if (L.n_chunks == 1) {
    k_perm_small<<<1, 1024, 0, st>>>(a.ids, a.T, a.topk, a.E, counts, offsets, tiles, ntiles, tiles_w, ntiles_w,
                                     row_pair, pair_row, h_amax);
  } else {
    k_perm_masks<<<(unsigned)L.n_chunks, 256, 0, st>>>(a.ids, a.T, a.topk, a.E, L.n_chunks, masks, ccnt);
    k_perm_scan<<<1, 1024, 0, st>>>(ccnt, a.E, L.n_chunks, cbase, counts, offsets, tiles, ntiles, tiles_w, ntiles_w,
                                     h_amax);
    k_perm_rows<<<(unsigned)((L.P + 255) / 256), 256, 0, st>>>(a.ids, L.P, a.topk, a.E, L.n_chunks, masks, cbase,
                                                                offsets, row_pair, pair_row);
  }
  const dim3 g1((unsigned)(a.I / (32 * kSkNT)), (unsigned)L.max_tiles);  // 4 waves x 8*NT h columns
  const dim3 g2((unsigned)(a.H / (64 * kSkNT)), (unsigned)L.max_tiles);  // 4 waves x 16*NT y columns
  // One permutation chunk (T <= kChunk) counts an expert's rows over a kChunk-bit token mask, so no
  // expert exceeds kSkinnyMaxRows rows and the many-row kernels have no tiles: they are not launched.
  static_assert(kChunk <= kSkinnyMaxRows, "a single chunk never yields a many-row expert");
  const bool many = L.n_chunks > 1;
  // dense FP8 MLP (one expert, top-1, at most kDenseRows tokens): every workgroup covers all rows
  const bool dense = !a.nvfp4 && !a.a16 && a.E == 1 && a.topk == 1 && a.T <= kDenseRows;
  float* part = reinterpret_cast<float*>(ws + L.part);
  // the many-row kernel reads weights in groups of 4 K steps (K % 256 == 0): always for the gate/up
  // projection (H % 256 == 0), for the down projection when I % 256 == 0 (else the 16x16x32 kernel)
  const bool big_dn = a.I % 256 == 0;
  const dim3 w1((unsigned)(a.I / (kGBN / 2)), (unsigned)L.max_tiles_w);
  const dim3 w2((unsigned)(a.H / (big_dn ? kGBN : 128)), (unsigned)L.max_tiles_w);
  _Float16* act = reinterpret_cast<_Float16*>(ws + L.act_f16);
  _Float16* hdec = reinterpret_cast<_Float16*>(ws + L.h_f16);
  const int64_t xblk = a.T * a.H / 16;
  const unsigned gx = (unsigned)((xblk + 255) / 256);
  // The GEMMs stage their activation rows from the codes (the few-row kernels when K is a multiple of their
  // super-step; k_gemm_big): x is not decoded to FP16 first (qa1), and the h quantization writes no FP16
  // copy of h (qa2; not when the down projection of many-row experts falls back to k_gemm_wide).  NVFP4
  // gate/up with many-row experts keeps the FP16 copy of x, which k_gemm_big stages with direct-to-LDS
  // loads: staging x from its codes measured slower there (prefill-8192 gate/up 2.99 -> 3.11 ms, against
  // 0.02 ms saved by not decoding x).  The NVFP4 down projection went 1.59-1.62 -> 1.60-1.67 ms and the h
  // quantization 0.19-0.21 -> 0.15 ms without the FP16 copy (layer unchanged within the spread of runs);
  // FP8: gate/up 3.55 -> 3.43 ms, down 1.85 -> 1.75 ms, layer 6.30 -> 6.01 ms.
  const int64_t ks_vals = 4 * (a.nvfp4 ? kNvKB : kF8KB);  // k_skinny_rows super-step
  const bool qa1 = a.H % ks_vals == 0 && (!many || !a.nvfp4), qa2 = a.I % ks_vals == 0 && (!many || big_dn);
  if (a.a16)
    act = reinterpret_cast<_Float16*>(const_cast<uint8_t*>(a.x_codes));  // BF16 x, read as 16-bit containers
  else if (a.nvfp4 && !qa1)
    k_decode_act<true><<<gx, 256, 0, st>>>(a.x_codes, reinterpret_cast<const uint8_t*>(a.x_scales), xblk, act);
  else if (!a.nvfp4 && !dense && !qa1)
    k_decode_act<false><<<gx, 256, 0, st>>>(a.x_codes, nullptr, xblk, act);
  stage_mark(0, 1, st);
  const uint8_t* w13s = reinterpret_cast<const uint8_t*>(a.w13_scales);
  const uint8_t* w2s = reinterpret_cast<const uint8_t*>(a.w2_scales);
  // the few-row GEMMs' NVFP4 block scales: lane-ordered with the pair layout, else row-major
  const uint8_t* w13sk = a.pairs && a.nvfp4 ? reinterpret_cast<const uint8_t*>(a.w13_scales_lanes) : w13s;
  const uint8_t* w2sk = a.pairs && a.nvfp4 ? reinterpret_cast<const uint8_t*>(a.w2_scales_lanes) : w2s;
  const float* xrs = reinterpret_cast<const float*>(a.x_scales);
  const uint8_t* xsb = reinterpret_cast<const uint8_t*>(a.x_scales);  // NVFP4: E4M3 block scales
  const float* hsc = reinterpret_cast<const float*>(h_scales);        // FP8: per-row h scales
  // Few-row experts: k_skinny_rows when K is a multiple of its super-step (NVFP4 512, FP8 256 values),
  // else k_skinny with 32-value quarters; many-row experts: k_gemm_big (k_gemm_wide for the down
  // projection when I % 256 != 0).
#define BSM_G1(NV)                                                                                             \
  if (qa1)                                                                                                     \
    launch_skr<NV, true, false, NV ? 1 : kSkDepthF8, true>(a.pairs, g1, st,                                    \
        nullptr, a.x_codes, NV ? xsb : nullptr, row_pair, a.topk, a.x_gs, xrs, a.w13_codes, w13sk, a.w13_gs,   \
        tiles, ntiles, a.H, a.H, a.I, h_f32, h_amax);                                                          \
  else if (a.H % (4 * (NV ? kNvKB : kF8KB)) == 0)                                                              \
    launch_skr<NV, true, false, NV ? 1 : kSkDepthF8, false>(a.pairs, g1, st,                                   \
        act, nullptr, nullptr, row_pair, a.topk, a.x_gs, xrs, a.w13_codes, w13sk, a.w13_gs, tiles, ntiles,    \
        a.H, a.H, a.I, h_f32, h_amax);                                                                              \
  else                                                                                                         \
    k_skinny<NV, true, 32, kSkNT, false, NV ? 1 : kSkDepthF8><<<g1, 256, 0, st>>>(                             \
        act, row_pair, a.topk, a.x_gs, xrs, a.w13_codes, w13s, a.w13_gs, tiles, ntiles, a.H, a.H, a.I, h_f32,  \
        h_amax);                                                                                               \
  if (many && qa1)                                                                                             \
    k_gemm_big<NV, true, false, true><<<w1, 256, 0, st>>>(nullptr, row_pair, a.topk, a.x_gs, xrs, a.w13_codes, \
                                                          w13s, a.w13_gs, tiles_w, ntiles_w, a.H, a.H, a.I,    \
                                                          h_f32, h_amax, a.x_codes, NV ? xsb : nullptr,        \
                                                          a.pairs ? 1 : 0);                                    \
  else if (many)                                                                                               \
    k_gemm_big<NV, true><<<w1, 256, 0, st>>>(act, row_pair, a.topk, a.x_gs, xrs, a.w13_codes, w13s, a.w13_gs, \
                                             tiles_w, ntiles_w, a.H, a.H, a.I, h_f32, h_amax, nullptr, nullptr,  \
                                             a.pairs ? 1 : 0)
#define BSM_G2(NV, HSC)                                                                                        \
  if (qa2)                                                                                                     \
    launch_skr<NV, false, false, NV ? 1 : kSkDepthF8, true>(a.pairs, g2, st,                                   \
        nullptr, h_codes, NV ? h_scales : nullptr, row_pair, a.topk, h_gs, HSC, a.w2_codes, w2sk, a.w2_gs,     \
        tiles, ntiles, a.I, a.H, a.I, y, h_amax);                                                              \
  else if (a.I % (4 * (NV ? kNvKB : kF8KB)) == 0)                                                              \
    launch_skr<NV, false, false, NV ? 1 : kSkDepthF8, false>(a.pairs, g2, st,                                  \
        hdec, nullptr, nullptr, row_pair, a.topk, h_gs, HSC, a.w2_codes, w2sk, a.w2_gs, tiles, ntiles, a.I,    \
        a.H, a.I, y, h_amax);                                                                                  \
  else                                                                                                         \
    k_skinny<NV, false, 32, kSkNT, false, NV ? 1 : kSkDepthF8><<<g2, 256, 0, st>>>(                            \
        hdec, row_pair, a.topk, h_gs, HSC, a.w2_codes, w2s, a.w2_gs, tiles, ntiles, a.I, a.H, a.I, y, h_amax); \
  if (many && qa2)                                                                                             \
    k_gemm_big<NV, false, false, true><<<w2, 256, 0, st>>>(nullptr, row_pair, a.topk, h_gs, HSC, a.w2_codes,  \
                                                           w2s, a.w2_gs, tiles_w, ntiles_w, a.I, a.H, a.I, y,  \
                                                           h_amax, h_codes, NV ? h_scales : nullptr,           \
                                                           a.pairs ? 1 : 0);                                   \
  else if (many && big_dn)                                                                                     \
    k_gemm_big<NV, false><<<w2, 256, 0, st>>>(hdec, row_pair, a.topk, h_gs, HSC, a.w2_codes, w2s, a.w2_gs,     \
                                              tiles_w, ntiles_w, a.I, a.H, a.I, y, h_amax, nullptr, nullptr,   \
                                              a.pairs ? 1 : 0);                                                \
  else if (many)                                                                                               \
    k_gemm_wide<NV, false><<<w2, 256, 0, st>>>(hdec, row_pair, a.topk, h_gs, HSC, a.w2_codes, w2s, a.w2_gs,    \
                                               tiles_w, ntiles_w, a.I, a.H, a.I, y, h_amax)
  hipError_t err;
  if (a.a16) {
    // weight-only W4A16: BF16 activations, NVFP4 weights decoded to BF16, h rounded to BF16
#define BSM_A16_G(G, A, SC, W, WS, WSK, WGS, OUT, GRID, WGRID, K)                                                 \
  if (K % (4 * kNvKB) == 0)                                                                                    \
    launch_skr<true, G, true, 1, false>(a.pairs, GRID, st, A, nullptr, nullptr, row_pair, a.topk, nullptr, SC,  \
                                        W, WSK, WGS, tiles, ntiles, K, a.H, a.I, OUT, h_amax);                 \
  else                                                                                                         \
    k_skinny<true, G, 32, kSkNT, true><<<GRID, 256, 0, st>>>(A, row_pair, a.topk, nullptr, SC, W, WS, WGS,     \
                                                             tiles, ntiles, K, a.H, a.I, OUT, h_amax);         \
  if (many && (G || big_dn))                                                                                   \
    k_gemm_big<true, G, true><<<WGRID, 256, 0, st>>>(A, row_pair, a.topk, nullptr, SC, W, WS, WGS, tiles_w,    \
                                                     ntiles_w, K, a.H, a.I, OUT, h_amax, nullptr, nullptr,     \
                                                     a.pairs ? 1 : 0);                                         \
  else if (many)                                                                                               \
    k_gemm_wide<true, G, true><<<WGRID, 256, 0, st>>>(A, row_pair, a.topk, nullptr, SC, W, WS, WGS, tiles_w,   \
                                                      ntiles_w, K, a.H, a.I, OUT, h_amax)
    BSM_A16_G(true, act, xrs, a.w13_codes, w13s, w13sk, a.w13_gs, h_f32, g1, w1, a.H);
    stage_mark(0, 2, st);
    const int64_t n4 = L.P * a.I / 4;
    k_h_to_bf16<<<(unsigned)((n4 + 255) / 256), 256, 0, st>>>(h_f32, n4, reinterpret_cast<uint16_t*>(hdec));
    stage_mark(0, 3, st);
    BSM_A16_G(false, hdec, nullptr, a.w2_codes, w2s, w2sk, a.w2_gs, y, g2, w2, a.I);
#undef BSM_A16_G
  } else if (a.nvfp4) {
    BSM_G1(true);
    stage_mark(0, 2, st);
    err = launch_nvfp4_quantize_from_amax(h_f32, false, 1, L.P, a.I, h_codes, h_scales, h_gs, h_amax,
                                          a.h_static ? a.h_gs_user : nullptr, st, qa2 ? nullptr : hdec);
    if (err != hipSuccess) return err;
    if (!a.h_static && a.h_gs_user) k_copy_f32<<<1, 64, 0, st>>>(h_gs, a.h_gs_user);
    stage_mark(0, 3, st);
    BSM_G2(true, hsc);
  } else {
    // FP8: E4M3 operands decoded exactly to FP16 in both projections (FP32 accumulation)
    const float* w13f = reinterpret_cast<const float*>(a.w13_scales);
    const float* w2f = reinterpret_cast<const float*>(a.w2_scales);
    if (dense) {
      err = launch_dense_f8<true>(a.x_codes, xrs, a.T, a.H, a.w13_codes, w13f, 0, a.I, h_f32, part, st);
      if (err != hipSuccess) return err;
    } else {
      BSM_G1(false);
    }
    stage_mark(0, 2, st);
    err = launch_fp8_quantize(h_f32, false, L.P, a.I, h_codes, reinterpret_cast<float*>(h_scales), st,
                              qa2 || dense ? nullptr : hdec);
    if (err != hipSuccess) return err;
    stage_mark(0, 3, st);
    if (dense) {
      err = launch_dense_f8<false>(h_codes, hsc, L.P, a.I, a.w2_codes, w2f, a.H, 0, y, part, st);
      if (err != hipSuccess) return err;
    } else {
      BSM_G2(false, hsc);
    }
  }
#undef BSM_G1
#undef BSM_G2
  stage_mark(0, 4, st);
  const dim3 gc((unsigned)((a.H / 4 + 255) / 256), (unsigned)a.T);
  k_combine<<<gc, 256, 0, st>>>(y, pair_row, a.wts, a.topk, a.H, (double)a.combine_scale, a.out);
  stage_mark(0, 5, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RMSNorm and residual
// ---------------------------------------------------------------------------
namespace {
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ x, int64_t H, float eps,
                                                 const float* __restrict__ gamma, float* __restrict__ y) {
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
  if (gamma)
    for (int64_t k = threadIdx.x; k < H; k += 256) y[t * H + k] = (xr[k] * r) * gamma[k];
  else
    for (int64_t k = threadIdx.x; k < H; k += 256) y[t * H + k] = xr[k] * r;
}

__global__ __launch_bounds__(256) void k_residual(float* __restrict__ x, const float* __restrict__ m, double a,
                                                  double b, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = (float)(a * (double)x[i] + b * (double)m[i]);
}
}  // namespace

hipError_t launch_rmsnorm(const float* x, int64_t T, int64_t H, float eps, const float* gamma, float* y,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  k_rmsnorm<<<(unsigned)T, 256, 0, st>>>(x, H, eps, gamma, y);
  return hipGetLastError();
}

hipError_t launch_residual(float* x, const float* m, float a, float b, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  k_residual<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(x, m, (double)a, (double)b, n);
  return hipGetLastError();
}

}  // namespace bsm
