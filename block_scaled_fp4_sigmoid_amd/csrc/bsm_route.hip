// bsm_route.hip -- group-limited sigmoid router for gfx950.
//
// Method ("Reflection releases Beam" news page, "Mixture-of-Experts
// details"): sigmoid score per expert, experts split into n_group groups,
// keep the topk_group groups with the largest sum of their two best scores,
// select the topk best experts inside them, weights normalized by the sum of
// the selected scores.  The router runs in FP32 ("Residual stream and
// numerical decisions") on unquantized inputs ("NVFP4 quantization" page,
// "Quantization scheme").
//
// To make the FP32 result independent of summation order, a logit is the
// exactly rounded binary32 value of the exact dot product, and a score the
// exactly rounded binary32 value of 1/(1+exp(-l)):
//
//   k_logits_rb   small batches, fp32 x or w: 4 tokens x 8 experts per workgroup over the
//                 whole row (lanes own K slices); binary64 FMA accumulation of
//                 products that are exact in binary64, and binary64 sums of
//                 squares of the workgroup's rows (an upper bound of each
//                 2-norm).  The epilogue proves the binary32 rounding of each
//                 logit by an error bound away from every rounding boundary;
//                 for the rest, by exactness (lowest set bits of its two
//                 rows); failing both, the workgroup recomputes it
//                 exactly (fixed-point window / superaccumulator, rounded once)
//   k_rowstats    large batches, fp32 x or w: per row of x and w, an upper bound of the
//                 2-norm and the lowest set-bit exponent of its nonzero entries
//   k_logits      large batches: 64x64 double-buffered LDS tiles, 8x4 logits
//                 per thread, K cut into slices (binary64 partial sums)
//   k_logits_fin  large batches: adds the slices in order, tries exactness
//                 first, then the error bound, and lists the rest
//   k_exact_list  the listed logits (tiled binary64 and int8 paths) recomputed exactly, one
//                 workgroup per logit
//   k_select      one workgroup per token: certified binary64 sigmoid
//                 (double-double fallback), group top-2 sums, group
//                 selection, iterative 64-bit (score, index) argmax,
//                 normalization.
//   k_slice8      bf16 x and w: per row an exponent bound, a truncation
//                 residual, a norm bound, and four int8 digits of every value
//   k_logits_i8   bf16 x and w: the dot products as exact int32 digit sums on
//                 the int8 matrix cores, rounded once; rows with a residual
//                 prove the rounding by a bound or list the logit for
//                 k_exact_list.  Small batches cut K into splits and store
//                 exact partials, which k_fin_i8 adds and rounds
//   k_select256   256 experts: the same selection, one wave per token with
//                 four experts per lane and shuffles in place of LDS.
//   k_select256_fin  256 experts, bf16 x and w at small batches: k_fin_i8's
//                 rounding, the exact recomputation of what it leaves
//                 unproven, and k_select256's selection in one kernel

#include "bsm_internal.h"

namespace bsm {

namespace {

constexpr int kTile = 64;  // tokens x experts per workgroup of the tiled logits kernel
constexpr int kBK = 16;    // K step of the tiled logits kernel staged in LDS (32 KB double-buffered)
constexpr int kRbT = 4;    // tokens per workgroup of the small-batch logits kernel
constexpr int kRbE = 8;    // experts per workgroup of the small-batch logits kernel
constexpr int kRbK = 2048; // K covered by one pass of a small-batch workgroup (256 lanes x 8)
constexpr int kExactWgs = 1024;  // workgroups sharing the list of logits recomputed exactly

// bf16 x bf16 tiled path on the int8 matrix cores (see k_slice8 below)
constexpr int kI8Rows = 64;       // tokens and experts per workgroup
constexpr int kI8ChunkB = 128;    // digit bytes per row and chunk of 32 k (4 digits x 32 values)
constexpr int kI8Stage = 2;       // chunks per LDS stage
constexpr int kI8Ld = kI8Stage * kI8ChunkB + 16;  // LDS bytes per row and stage (16-byte pad)
constexpr int kI8MaxH = 16384;    // keeps every int32 diagonal sum below 2^31
constexpr int kI8ZeroRow = -4096; // exponent bound recorded for a row without finite nonzero values

struct RouteWs {
  size_t norm, lsb, part, ulist, logits, blk, diag, total;  // norm, lsb, part, ulist: tiled path only
  size_t rexp, rres;  // int8 path: per-row exponent bound and truncation residual (dig shares part's space)
  size_t dig, spart;  // int8 path: digits; small batches: per K split and logit an exact (hi, lo) partial
  bool i8ok;          // the int8 path fits this shape (the launch also needs bf16 x and w)
  int64_t ncp;        // int8 path: chunks of 32 k per row, rounded up to an even number of stages
  int64_t s8, sps8;   // int8 path: K splits (1 at large batches) and stages per split (even)
  int64_t nblk8;      // int8 path: workgroups that count list entries (the finalize kernel's at small batches)
  bool rb;    // small-batch kernel (full K per workgroup, lanes own K slices)
  int nadd;   // roundings along the longest summation path of one logit
  int64_t nblk;  // logits workgroups (one exact-recomputation count each)
  int ks;        // tiled path: K slices (one binary64 partial sum per logit each)
  int64_t kslice;  // tiled path: K per slice (a multiple of kBK)
};

RouteWs route_layout(int64_t T, int64_t H, int64_t E) {
  RouteWs L;
  const int64_t tiles = ((T + kTile - 1) / kTile) * ((E + kTile - 1) / kTile);
  L.rb = (H % 8 == 0) && tiles < 128;
  // Tiled path: K is cut into slices so that the grid holds about 16 waves per CU (a 64 x 64 tile
  // is two waves, 32 KB of LDS); every slice holds at least one LDS step.
  const int64_t nst = (H + kBK - 1) / kBK;
  int64_t ks = (2048 + tiles - 1) / (tiles > 0 ? tiles : 1);
  ks = ks < 1 ? 1 : ks > 8 ? 8 : ks;
  ks = ks > nst ? (nst > 0 ? nst : 1) : ks;
  const int64_t sps = (nst + ks - 1) / ks;  // LDS steps per slice
  L.ks = (int)(sps > 0 ? (nst + sps - 1) / sps : 1);
  L.kslice = sps * kBK;
  // small batch: one FMA chain of 8 per pass, 6 shuffle levels, 3 cross-wave adds;
  // tiled: an FMA chain of kBK per LDS step, added to the slice's running sum, then the slices
  // added in order
  L.nadd = L.rb ? (int)(((H + kRbK - 1) / kRbK) * 8 + 9) : (int)(kBK + sps + L.ks + 1);
  // int8 path: small batches cut K into splits (an even number of stages each) so that the grid holds
  // about 256 workgroups of at least 4 stages; their exact partials are added by k_fin_i8
  L.i8ok = H % 16 == 0 && H <= kI8MaxH;
  L.ncp = (((H + 31) / 32 + 2 * kI8Stage - 1) / (2 * kI8Stage)) * (2 * kI8Stage);  // an even number of stages
  {
    const int64_t nst8 = L.ncp / kI8Stage, nwg8 = ((T + kI8Rows - 1) / kI8Rows) * ((E + kI8Rows - 1) / kI8Rows);
    int64_t s8 = L.rb ? (256 + nwg8 - 1) / (nwg8 > 0 ? nwg8 : 1) : 1;
    const int64_t smax = nst8 / 4 > 1 ? nst8 / 4 : 1;
    s8 = s8 < 1 ? 1 : s8 > smax ? smax : s8;
    const int64_t pairs = nst8 / 2, ppers = (pairs + s8 - 1) / s8;
    L.sps8 = 2 * ppers;
    L.s8 = (nst8 + L.sps8 - 1) / L.sps8;
    L.nblk8 = L.rb ? (T * E + 255) / 256 : nwg8;
  }
  const bool big = !L.rb, i8s = L.rb && L.i8ok;  // i8s: the small-batch int8 path may run
  L.nblk = L.rb ? ((T + kRbT - 1) / kRbT) * ((E + kRbE - 1) / kRbE) : tiles;
  if (L.i8ok && L.nblk8 > L.nblk) L.nblk = L.nblk8;
  size_t o = 0;
  L.norm = o;
  if (big || i8s) o += align256(sizeof(double) * (size_t)(T + E));
  L.lsb = o;
  if (big) o += align256(sizeof(int) * (size_t)(T + E));
  L.part = o;  // binary64 partial sums, or the int8 path's digits of every row of x and w
  const size_t db = L.i8ok ? (size_t)(T + E) * (size_t)L.ncp * kI8ChunkB : 0;
  if (big) {
    const size_t pb = sizeof(double) * (size_t)L.ks * (size_t)T * (size_t)E;
    o += align256(pb > db ? pb : db);
  } else if (i8s) {
    o += align256(db);
  }
  L.dig = L.part;
  L.spart = o;
  if (i8s) o += align256(2 * sizeof(int64_t) * (size_t)L.s8 * (size_t)T * (size_t)E);
  L.rexp = o;
  if (L.i8ok) o += align256(sizeof(int) * (size_t)(T + E));
  L.rres = o;
  if (L.i8ok) o += align256(sizeof(double) * (size_t)(T + E));
  L.ulist = o;  // count, then the flat indices of the logits left for exact recomputation
  if (big || i8s) o += align256(sizeof(int) * (size_t)(T * E + 1));
  L.logits = o;
  o += align256(sizeof(float) * (size_t)T * (size_t)E);
  L.blk = o;
  o += align256(sizeof(int) * (size_t)(L.nblk > 0 ? L.nblk : 1));
  L.diag = o;
  o += align256(sizeof(int) * 4);
  L.total = o;
  return L;
}

template <bool BF16>
__device__ inline float ld1(const void* p, int64_t i) {
  if (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  return reinterpret_cast<const float*>(p)[i];
}

// 8 consecutive values (16-byte aligned start) as binary32
template <bool BF16>
__device__ inline void ld8(const void* p, int64_t i, float* v) {
  if (BF16) {
    const uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p) + i);
    const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = u2f(d[j] << 16);
      v[2 * j + 1] = u2f(d[j] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Exact binary32 logit of one (token, expert) pair, computed by the whole
// workgroup (every thread calls it; the result is valid in thread 0).  Every
// product is exact in binary64.  Fast path: the fixed-point window of
// bsm_numerics.h anchored one binade above A = |x|_2 |w|_2, which bounds every
// product; a product more than 120 bits below it switches the workgroup to the
// 22-digit superaccumulator.
struct ExactLds {
  long long d[4][WIN_DIGITS];
  long long sa[SA_NDIG];
  int bad;
};

template <bool XB, bool WB, int NT>
__device__ float exact_logit_wg(const void* __restrict__ x, const void* __restrict__ w, int64_t t, int64_t e,
                                int64_t H, double A, ExactLds* L) {
  static_assert(NT % 64 == 0 && NT <= 256, "one to four waves");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int base = win_base((int)((d2u(A) >> 52) & 0x7FF) + 1);
  if (tid == 0) L->bad = 0;
  __syncthreads();
  int64_t dig[WIN_DIGITS] = {0, 0, 0, 0, 0};
  bool bad = false;
  // 8 consecutive k per thread and pass: the 16 loads of a pass are independent (the digit sums are exact,
  // so the order of the additions does not matter); a product past H is zero, which adds nothing
  constexpr int U = 8;
  for (int64_t k0 = (int64_t)tid * U; k0 < H; k0 += (int64_t)NT * U) {
    float xv[U], wv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = k0 + u < H;
      xv[u] = in ? ld1<XB>(x, t * H + k0 + u) : 0.0f;
      wv[u] = in ? ld1<WB>(w, e * H + k0 + u) : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) bad |= !win_add(dig, (double)xv[u] * (double)wv[u], base);
  }
  if (bad) atomicOr(&L->bad, 1);
#pragma unroll
  for (int q = 0; q < WIN_DIGITS; ++q) {
    long long v = dig[q];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) L->d[wv][q] = v;
  }
  __syncthreads();
  float r = 0.0f;
  if (!L->bad) {
    if (tid == 0) {
      int64_t D[WIN_DIGITS];
      for (int q = 0; q < WIN_DIGITS; ++q) {
        long long acc = 0;
        for (int ww = 0; ww < NW; ++ww) acc += L->d[ww][q];
        D[q] = acc;
      }
      r = win_round_f32(D, base);
    }
  } else {
    if (tid < SA_NDIG) L->sa[tid] = 0;
    __syncthreads();
    int64_t loc[SA_NDIG];
    for (int q = 0; q < SA_NDIG; ++q) loc[q] = 0;
    for (int64_t k0 = (int64_t)tid * U; k0 < H; k0 += (int64_t)NT * U) {
      float xv[U], wv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool in = k0 + u < H;
        xv[u] = in ? ld1<XB>(x, t * H + k0 + u) : 0.0f;
        wv[u] = in ? ld1<WB>(w, e * H + k0 + u) : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) sa_add(loc, (double)xv[u] * (double)wv[u]);
    }
    for (int q = 0; q < SA_NDIG; ++q)
      if (loc[q]) atomicAdd(reinterpret_cast<unsigned long long*>(&L->sa[q]), (unsigned long long)loc[q]);
    __syncthreads();
    if (tid == 0) {
      int64_t dg[SA_NDIG];
      for (int q = 0; q < SA_NDIG; ++q) dg[q] = L->sa[q];
      r = sa_round_f32(dg);
    }
  }
  __syncthreads();
  return r;
}

// Upper bound of a row's 2-norm from its binary64 sum of squares: along any
// summation chain of n <= 2^22 terms the relative error of the sum is below
// (n + 8) * 2^-53; the inflation is generous.
__device__ inline double norm_bound(double ss) { return sqrt(ss * (1.0 + 0x1p-30)) * (1.0 + 0x1p-40); }

// A >= sum_k |x_k w_k| from the two rows' norm bounds.
__device__ inline double abs_bound(double nx, double nw) { return nx * nw * (1.0 + 0x1p-40); }

// Binary32 rounding of a binary64 dot-product estimate S.  (b) certified: the
// error bound (nadd + 4) * 2^-53 * A keeps S away from every binary32 rounding
// boundary; NaN when it does not.  A zero bound means every product is zero.
__device__ inline float certify_bound(double S, double A, int nadd) {
  if (A == 0.0) return 0.0f;
  float r;
  if (f32_certified(S, (double)(nadd + 4) * 0x1p-53 * A * 1.0001, &r)) return r;
  return __builtin_nanf("");
}

// (a) exact: every product is a multiple of 2^L (L = lsb(x) + lsb(w)) and
// every partial sum lies below A < 2^(L+53) in magnitude, so no addition
// rounded and S is the exact sum.
__device__ inline bool certify_exact(double S, double A, int lx, int lw, float* r) {
  if (lx == 0x7FFFFFFF || lw == 0x7FFFFFFF) return false;
  const int L = lx + lw;
  if (L + 53 > -1000 && A < ldexp(1.0, L + 53)) {
    *r = (float)S;
    return true;
  }
  return false;
}

// Large batches: per row of x (rows 0..T-1) and of w (rows T..T+E-1), one
// wave per row: an upper bound of the 2-norm and the lowest set-bit exponent
// of the row's nonzero entries, read by the tiled logits kernel.
template <bool XB, bool WB, bool VEC>
__global__ __launch_bounds__(256) void k_rowstats(const void* __restrict__ x, const void* __restrict__ w, int64_t T,
                                                  int64_t E, int64_t H, double* __restrict__ norm,
                                                  int* __restrict__ lsb) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= T + E) return;
  const bool isx = r < T;
  const void* p = isx ? x : w;
  const int64_t row = isx ? r : r - T;
  double ss = 0.0;
  int lmin = 0x7FFFFFFF;
  if (VEC) {
    for (int64_t k = (int64_t)lane * 8; k < H; k += 512) {
      float v[8];
      if (isx) ld8<XB>(p, row * H + k, v);
      else ld8<WB>(p, row * H + k, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const double d = (double)v[q];
        ss = fma(d, d, ss);
        if (v[q] != 0.0f) {
          const int l = f32_lsb_exp(v[q]);
          lmin = l < lmin ? l : lmin;
        }
      }
    }
  } else {
    for (int64_t k = lane; k < H; k += 64) {
      const float v = isx ? ld1<XB>(p, row * H + k) : ld1<WB>(p, row * H + k);
      const double d = (double)v;
      ss = fma(d, d, ss);
      if (v != 0.0f) {
        const int l = f32_lsb_exp(v);
        lmin = l < lmin ? l : lmin;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ss += __shfl_xor(ss, o, 64);
    const int ol = __shfl_xor(lmin, o, 64);
    lmin = ol < lmin ? ol : lmin;
  }
  if (lane == 0) {
    // relative error of the sum of squares is below (H + 8) * 2^-53; inflate generously
    norm[r] = norm_bound(ss);
    lsb[r] = lmin;
  }
}

// Both tests with precomputed row statistics (norm bounds and lowest set bits):
// exactness first, then the error bound; NaN when neither proves the rounding.
__device__ inline float certify_logit(double S, double nx, double nw, int lx, int lw, int nadd) {
  const double A = abs_bound(nx, nw);
  if (A == 0.0) return 0.0f;
  float r;
  if (certify_exact(S, A, lx, lw, &r)) return r;
  return certify_bound(S, A, nadd);
}

// Small batches: a workgroup owns kRbT tokens x kRbE experts over the whole
// row; each lane accumulates 8-wide K slices of all kRbT x kRbE products in
// binary64 registers, then a fixed-order reduce-scatter across the wave and a
// fixed-order sum of the four waves.  Consecutive workgroups land on
// different XCDs; each XCD gets a contiguous range of expert tiles so its L2
// holds all of x and one eighth of w.
template <bool XB, bool WB>
__global__ __launch_bounds__(256) void k_logits_rb(const void* __restrict__ x, const void* __restrict__ w, int64_t T,
                                                   int64_t E, int64_t H, int nadd, float* __restrict__ logits,
                                                   int* __restrict__ blk, int* __restrict__ diag) {
  constexpr int TT = kRbT, TE = kRbE, NV = TT * TE;
  static_assert(NV == 32, "reduce-scatter below assumes 32 outputs per workgroup");
  __shared__ double s_red[4][NV];
  __shared__ double s_ss[4][TT + TE];  // per wave: sums of squares of the TT x rows and TE w rows
  __shared__ double s_n[TT + TE];      // norm bounds of those rows
  __shared__ int unc[NV];
  __shared__ double uS[NV];
  __shared__ int s_lo[4][2];  // per wave: lowest set-bit exponents of one x row and one w row
  __shared__ int n_unc;
  __shared__ ExactLds xl;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (blockIdx.x == 0 && tid >= 1 && tid < 4) diag[tid] = 0;  // counters of the selection kernel that follows
  const int64_t nte = (E + TE - 1) / TE;
  const int64_t b = blockIdx.x;
  int64_t te, tt;
  if (nte % 8 == 0) {
    const int64_t per = nte / 8, loc = b >> 3;
    te = (b & 7) * per + loc % per;
    tt = loc / per;
  } else {
    te = b % nte;
    tt = b / nte;
  }
  const int64_t t0 = tt * TT, e0 = te * TE;
  double acc[TT][TE], ssx[TT], ssw[TE];
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    ssx[i] = 0.0;
#pragma unroll
    for (int j = 0; j < TE; ++j) acc[i][j] = 0.0;
  }
#pragma unroll
  for (int j = 0; j < TE; ++j) ssw[j] = 0.0;
  // raw 8-value slices of the TT x rows and TE w rows; the next pass's slices
  // are loaded before the current pass is multiplied
  constexpr int XW = XB ? 4 : 8, WW = WB ? 4 : 8;  // dwords per 8-value slice
  uint32_t xr[TT][XW], wr[TE][WW], xn[TT][XW], wn[TE][WW];
  auto load_pass = [&](int64_t k, uint32_t (*xo)[XW], uint32_t (*wo)[WW]) {
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      const bool in = (t0 + i < T) && (k < H);
      const uint32_t* p = reinterpret_cast<const uint32_t*>(x) + ((t0 + i) * H + k) / (XB ? 2 : 1);
#pragma unroll
      for (int q = 0; q < XW; q += 4) {
        const uint4 v = in ? *reinterpret_cast<const uint4*>(p + q) : make_uint4(0u, 0u, 0u, 0u);
        xo[i][q] = v.x; xo[i][q + 1] = v.y; xo[i][q + 2] = v.z; xo[i][q + 3] = v.w;
      }
    }
#pragma unroll
    for (int j = 0; j < TE; ++j) {
      const bool in = (e0 + j < E) && (k < H);
      const uint32_t* p = reinterpret_cast<const uint32_t*>(w) + ((e0 + j) * H + k) / (WB ? 2 : 1);
#pragma unroll
      for (int q = 0; q < WW; q += 4) {
        const uint4 v = in ? *reinterpret_cast<const uint4*>(p + q) : make_uint4(0u, 0u, 0u, 0u);
        wo[j][q] = v.x; wo[j][q + 1] = v.y; wo[j][q + 2] = v.z; wo[j][q + 3] = v.w;
      }
    }
  };
  auto val = [](const uint32_t* r, int q, bool bf) -> double {
    if (bf) return (double)u2f((q & 1) ? (r[q >> 1] & 0xFFFF0000u) : (r[q >> 1] << 16));
    return (double)u2f(r[q]);
  };
  int64_t k = (int64_t)tid * 8;
  load_pass(k, xr, wr);
  for (; k < H; k += kRbK) {
    load_pass(k + kRbK, xn, wn);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      double wd[TE];
#pragma unroll
      for (int j = 0; j < TE; ++j) {
        wd[j] = val(wr[j], q, WB);
        ssw[j] = fma(wd[j], wd[j], ssw[j]);
      }
#pragma unroll
      for (int i = 0; i < TT; ++i) {
        const double xd = val(xr[i], q, XB);
        ssx[i] = fma(xd, xd, ssx[i]);
#pragma unroll
        for (int j = 0; j < TE; ++j) acc[i][j] = fma(xd, wd[j], acc[i][j]);
      }
    }
#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
      for (int q = 0; q < XW; ++q) xr[i][q] = xn[i][q];
#pragma unroll
    for (int j = 0; j < TE; ++j)
#pragma unroll
      for (int q = 0; q < WW; ++q) wr[j][q] = wn[j][q];
  }
  double v[NV];
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < TE; ++j) v[i * TE + j] = acc[i][j];
  // reduce-scatter: after the offset-32..2 steps lane l holds output l >> 1
  // summed over the 32 lanes that share bit 0; the offset-1 step completes it
#pragma unroll
  for (int s = 0; s < 5; ++s) {
    const int off = 32 >> s, h = NV >> (s + 1);
    const bool up = (lane & off) != 0;
#pragma unroll
    for (int q = 0; q < NV / 2; ++q) {
      if (q < h) {
        const double send = up ? v[q] : v[q + h];
        const double keep = up ? v[q + h] : v[q];
        v[q] = keep + __shfl_xor(send, off, 64);
      }
    }
  }
  v[0] += __shfl_xor(v[0], 1, 64);
  if ((lane & 1) == 0) s_red[wv][lane >> 1] = v[0];
  // sums of squares: butterfly over the wave, then the four waves in a fixed order
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
#pragma unroll
    for (int i = 0; i < TT; ++i) ssx[i] += __shfl_xor(ssx[i], o, 64);
#pragma unroll
    for (int j = 0; j < TE; ++j) ssw[j] += __shfl_xor(ssw[j], o, 64);
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < TT; ++i) s_ss[wv][i] = ssx[i];
#pragma unroll
    for (int j = 0; j < TE; ++j) s_ss[wv][TT + j] = ssw[j];
  }
  if (tid == 0) n_unc = 0;
  __syncthreads();
  if (tid < TT + TE) s_n[tid] = norm_bound(((s_ss[0][tid] + s_ss[1][tid]) + s_ss[2][tid]) + s_ss[3][tid]);
  __syncthreads();
  if (tid < NV) {
    const double S = ((s_red[0][tid] + s_red[1][tid]) + s_red[2][tid]) + s_red[3][tid];
    const int64_t t = t0 + tid / TE, e = e0 + tid % TE;
    if (t < T && e < E) {
      const float r = certify_bound(S, abs_bound(s_n[tid / TE], s_n[TT + tid % TE]), nadd);
      logits[t * E + e] = r;
      if (r != r) {
        const int u = atomicAdd(&n_unc, 1);
        unc[u] = tid;
        uS[u] = S;
      }
    }
  }
  __syncthreads();
  const int nu = n_unc;
  int nexact = 0;
  for (int u = 0; u < nu; ++u) {
    // exactness test: lowest set-bit exponents of the two rows (8-value loads; H % 8 == 0 on this path)
    const int i = unc[u] / TE, j = unc[u] % TE;
    const int64_t t = t0 + i, e = e0 + j;
    int a = 0x7FFFFFFF, c = 0x7FFFFFFF;
    for (int64_t k = (int64_t)tid * 8; k < H; k += 256 * 8) {
      float xv[8], wv[8];
      ld8<XB>(x, t * H + k, xv);
      ld8<WB>(w, e * H + k, wv);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (xv[q] != 0.0f) a = min(a, f32_lsb_exp(xv[q]));
        if (wv[q] != 0.0f) c = min(c, f32_lsb_exp(wv[q]));
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      a = min(a, __shfl_xor(a, o, 64));
      c = min(c, __shfl_xor(c, o, 64));
    }
    if (lane == 0) {
      s_lo[wv][0] = a;
      s_lo[wv][1] = c;
    }
    __syncthreads();
    const int lx = min(min(s_lo[0][0], s_lo[1][0]), min(s_lo[2][0], s_lo[3][0]));
    const int lw = min(min(s_lo[0][1], s_lo[1][1]), min(s_lo[2][1], s_lo[3][1]));
    __syncthreads();
    const double A = abs_bound(s_n[i], s_n[TT + j]);
    float r;
    if (!certify_exact(uS[u], A, lx, lw, &r)) {  // uniform across the workgroup
      r = exact_logit_wg<XB, WB, 256>(x, w, t, e, H, A, &xl);
      ++nexact;
    }
    if (tid == 0) logits[t * E + e] = r;
  }
  if (tid == 0) blk[blockIdx.x] = nexact;
}

// Large batches: 64x64 token x expert tiles staged through LDS, 4x4 outputs
// per thread; binary64 FMA chains of kBK products added to running sums.
// Large batches: a workgroup of 128 threads owns 64 tokens x 64 experts and
// one K slice (blockIdx.z); each thread accumulates 8 tokens x 4 experts.  K
// steps of kBK are staged through double-buffered LDS as binary64 (converted
// once per element), laid out [k][row] so a wave's staging stores and its
// expert reads are contiguous and its token reads are broadcasts.  Per logit
// and slice: an FMA chain over the kBK products of a step (k ascending),
// added to the slice's running sum (steps ascending), stored as a binary64
// partial sum.
template <bool XB, bool WB, bool VEC>
__global__ __launch_bounds__(128) void k_logits(const void* __restrict__ x, const void* __restrict__ w, int64_t T,
                                                int64_t E, int64_t H, int64_t kslice, double* __restrict__ part,
                                                int* __restrict__ ulist) {
  __shared__ __attribute__((aligned(16))) double tl[2][2][kBK][kTile];  // [buffer][x, w][k][row]
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && tid == 0) *ulist = 0;  // read by the finalize kernel
  const int tx = tid & 15, ty = tid >> 4;  // experts {2tx, 2tx+1, 32+2tx, 33+2tx}; tokens {4ty+i, 32+4ty+i}
  const int64_t t0 = (int64_t)blockIdx.x * kTile, e0 = (int64_t)blockIdx.y * kTile;
  const int64_t k0 = (int64_t)blockIdx.z * kslice;
  const int64_t k1 = k0 + kslice < H ? k0 + kslice : H;  // k0 < H: every slice holds at least one step
  // staging: row sr of the x and w tiles, k values kPer sh .. + kPer - 1 of the step.  Rows past
  // T or E repeat the last row: their logits are never stored, and no other logit reads them.
  constexpr int kPer = kBK / 2;  // values of each operand per thread and step
  static_assert(kPer % 8 == 0, "staging in 8-value loads");
  const int sr = tid & 63, sh = tid >> 6;
  const int64_t xr = t0 + sr < T ? t0 + sr : T - 1, wr = e0 + sr < E ? e0 + sr : E - 1;
  const int64_t xo = xr * H + kPer * sh, wo = wr * H + kPer * sh;
  float xv[kPer], wv[kPer];
  auto gload = [&](int64_t kb) {
    if constexpr (VEC) {  // H % kBK == 0: every k of the step is in range
#pragma unroll
      for (int q = 0; q < kPer; q += 8) {
        ld8<XB>(x, xo + kb + q, xv + q);
        ld8<WB>(w, wo + kb + q, wv + q);
      }
    } else {
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const bool kin = kb + kPer * sh + q < H;
        xv[q] = kin ? ld1<XB>(x, xo + kb + q) : 0.0f;
        wv[q] = kin ? ld1<WB>(w, wo + kb + q) : 0.0f;
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      tl[buf][0][kPer * sh + q][sr] = (double)xv[q];
      tl[buf][1][kPer * sh + q][sr] = (double)wv[q];
    }
  };
  double acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  const int nst = (int)((k1 - k0 + kBK - 1) / kBK);
  gload(k0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int buf = s & 1;
    if (s + 1 < nst) gload(k0 + (int64_t)(s + 1) * kBK);
    double blk[8][4];  // chain of kBK products per step, then one add
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) blk[i][j] = 0.0;
#pragma unroll 2
    for (int kk = 0; kk < kBK; ++kk) {
      const double2 a0 = *reinterpret_cast<const double2*>(&tl[buf][0][kk][4 * ty]);
      const double2 a1 = *reinterpret_cast<const double2*>(&tl[buf][0][kk][4 * ty + 2]);
      const double2 a2 = *reinterpret_cast<const double2*>(&tl[buf][0][kk][32 + 4 * ty]);
      const double2 a3 = *reinterpret_cast<const double2*>(&tl[buf][0][kk][32 + 4 * ty + 2]);
      const double2 b0 = *reinterpret_cast<const double2*>(&tl[buf][1][kk][2 * tx]);
      const double2 b1 = *reinterpret_cast<const double2*>(&tl[buf][1][kk][32 + 2 * tx]);
      const double av[8] = {a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
      const double bv[4] = {b0.x, b0.y, b1.x, b1.y};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) blk[i][j] = fma(av[i], bv[j], blk[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += blk[i][j];
    if (s + 1 < nst) lstore(buf ^ 1);
    __syncthreads();
  }
  double* pz = part + (int64_t)blockIdx.z * T * E;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t t = t0 + (i < 4 ? 0 : 32) + 4 * ty + (i & 3);
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t e = e0 + (j < 2 ? 0 : 32) + 2 * tx + (j & 1);
      if (e < E) pz[t * E + e] = acc[i][j];
    }
  }
}

// Large batches, per 64 x 64 tile: the K slices' partial sums added in slice
// order, then exactness first and the error bound second.  The logits neither
// proves go to a list (ulist[0] counts them) for k_exact_list.
__global__ __launch_bounds__(256) void k_logits_fin(int64_t T, int64_t E, int ks, const double* __restrict__ part,
                                                    const double* __restrict__ norm, const int* __restrict__ lsb,
                                                    int nadd, float* __restrict__ logits, int* __restrict__ ulist,
                                                    int* __restrict__ blk, int* __restrict__ diag) {
  __shared__ int n_unc;
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid >= 1 && tid < 4) diag[tid] = 0;  // selection-kernel counters
  const int64_t t0 = (int64_t)blockIdx.x * kTile, e0 = (int64_t)blockIdx.y * kTile;
  if (tid == 0) n_unc = 0;
  __syncthreads();
  for (int q = tid; q < kTile * kTile; q += 256) {
    const int tr = q / kTile, ec = q % kTile;
    const int64_t t = t0 + tr, e = e0 + ec;
    if (t >= T || e >= E) continue;
    double S = part[t * E + e];
    for (int z = 1; z < ks; ++z) S += part[(int64_t)z * T * E + t * E + e];
    const float r = certify_logit(S, norm[t], norm[T + e], lsb[t], lsb[T + e], nadd);
    logits[t * E + e] = r;
    if (r != r) {
      atomicAdd(&n_unc, 1);
      ulist[1 + atomicAdd(ulist, 1)] = (int)(t * E + e);
    }
  }
  __syncthreads();
  if (tid == 0) blk[blockIdx.y * gridDim.x + blockIdx.x] = n_unc;
}

// ---------------------------------------------------------------------------
// bf16 x and w: the dot products in exact integer arithmetic on the int8
// matrix cores (fp32 inputs take the binary64 kernels above).
//
// Every bf16 value is m * 2^l with an integer m < 2^8.  For a row (of x or of
// w) with every |v_k| < 2^X, N_k = trunc(v_k * 2^(30 - X)) is an integer with
// |N_k| < 2^30, equal to v_k * 2^(30 - X) unless v_k has bits below 2^(X - 30)
// (then |v_k - N_k 2^(X - 30)| is recorded in the row's residual).  N_k is
// written as four balanced base-256 digits, N = d0 2^24 + d1 2^16 + d2 2^8 + d3
// with d1..d3 in [-128, 127] and d0 in [-64, 64], each one int8.  For a token
// row x and an expert row w,
//   sum_k N_k M_k = sum_{j=0..6} D_j 2^(8 (6 - j)),   D_j = sum_k sum_{a+b=j} d_a[k] e_b[k],
// and every D_j is an exact int32 sum (|D_j| <= 4 H 2^14 < 2^31 for H <= 16384),
// whatever order the matrix cores add in.  The logit is then rounded once from
// the exact integer.  When a row has a residual, the truncated sum is off by at
// most rx 2^Xw + 2^Xx rw; the binary32 rounding is taken only when that bound
// keeps the value away from every rounding boundary, else the logit goes to the
// exact-recomputation list like the binary64 path's.
// ---------------------------------------------------------------------------

// One wave per row (four when rows are few; x rows 0..T-1, then w rows): the row's exponent bound X
// (from the largest magnitude's bits: bf16 magnitudes order like their bit
// patterns), its residual, a norm bound sqrt(H) max|v| (for the exact
// recomputation), and its digits: a row is ncp / 2 stage blocks of 64 k, each
// [digit][4 half chunks of 16 k][16 values] (zero past H).  A stage block is
// what the logits kernel loads as one contiguous 256 bytes, and each store
// instruction of a wave here writes runs of 64 bytes.
// N = trunc(v 2^(30 - X)) comes from a binary32 scaling (exact: the result is
// below 2^30) and a truncating conversion; v - N 2^(X - 30) is exact in
// binary32 (the low bits of v's 8-bit significand), so a nonzero difference
// flags a truncated value.  For rows with X < -100 that difference could fall
// below the binary32 range, and the digits come from the integer fields.
// Balanced digits: with M = N + 0x808080, the low three bytes of M xor 0x80
// are d3, d2, d1 and the top byte is d0 = M >> 24.
__device__ inline uint32_t slice_n(uint32_t b, int ex, bool flt, double& res) {
  if (flt) {
    const float f = u2f(b << 16);
    const int n = (int)ldexpf(f, 30 - ex);
    const float back = ldexpf((float)n, ex - 30);
    const float r = f - back;
    if (r != 0.0f) res += fabs((double)r);
    return (uint32_t)n;
  }
  const int eb = (int)((b >> 7) & 0xFFu);
  if (!(b & 0x7FFFu)) return 0u;
  const int el = eb ? eb - 134 : -133;  // value = mi 2^el
  const uint32_t mi = eb ? ((b & 0x7Fu) | 0x80u) : (b & 0x7Fu);
  const int sh = el - (ex - 30);
  uint32_t a;
  if (sh >= 0) {
    a = mi << sh;  // < 2^30
  } else if (sh > -32) {
    a = mi >> -sh;
    const uint32_t lo = mi & ((1u << -sh) - 1u);
    if (lo) res += ldexp((double)lo, el);
  } else {
    a = 0u;
    res += ldexp((double)mi, el);
  }
  return (b & 0x8000u) ? (uint32_t)(-(int)a) : a;
}

// Digits of 16 values (a half chunk) for digit-major storage.
__device__ inline void slice16(const uint32_t* u, int ex, bool flt, double& res, uint32_t (*o4)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {  // values 4c .. 4c+3
    uint32_t P[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t word = u[(4 * c + i) >> 1];
      const uint32_t b = (i & 1) ? (word >> 16) : (word & 0xFFFFu);
      P[i] = slice_n(b, ex, flt, res) + 0x808080u;
    }
    // byte transpose: row k holds byte k of P[0..3]
    const uint32_t A = __builtin_amdgcn_perm(P[1], P[0], 0x05010400u);  // P0b0 P1b0 P0b1 P1b1
    const uint32_t B = __builtin_amdgcn_perm(P[1], P[0], 0x07030602u);  // P0b2 P1b2 P0b3 P1b3
    const uint32_t C = __builtin_amdgcn_perm(P[3], P[2], 0x05010400u);
    const uint32_t D = __builtin_amdgcn_perm(P[3], P[2], 0x07030602u);
    o4[3][c] = __builtin_amdgcn_perm(C, A, 0x05040100u) ^ 0x80808080u;  // byte 0: d3
    o4[2][c] = __builtin_amdgcn_perm(C, A, 0x07060302u) ^ 0x80808080u;  // byte 1: d2
    o4[1][c] = __builtin_amdgcn_perm(D, B, 0x05040100u) ^ 0x80808080u;  // byte 2: d1
    o4[0][c] = __builtin_amdgcn_perm(D, B, 0x07060302u);                 // byte 3: d0
  }
}

__device__ inline uint32_t max_mag16(const uint32_t* u) {
  uint32_t mx = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t m = u[i] & 0x7FFF7FFFu;
    mx = max(mx, max(m & 0xFFFFu, m >> 16));
  }
  return mx;
}

// The same over the values that are not NaN (patterns above 0x7F80): max|x| as the NVFP4 global scale takes it.
__device__ inline uint32_t max_fin16(const uint32_t* u) {
  uint32_t mx = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t lo = u[i] & 0x7FFFu, hi = (u[i] >> 16) & 0x7FFFu;
    mx = max(mx, max(lo > 0x7F80u ? 0u : lo, hi > 0x7F80u ? 0u : hi));
  }
  return mx;
}

// WPR waves share a row (1, or 4 when there are few rows); NC > 0: the row
// (at most 64 WPR NC half chunks) stays in registers between the exponent pass
// and the digit pass; NC == 0: the digit pass reads it again.  rowam (optional,
// WPR > 1 only): for each row of x, the bit pattern of its largest magnitude that
// is not NaN, as a binary32 (max|x| for the NVFP4 quantization of x).
template <int NC, int WPR>
__global__ __launch_bounds__(256) void k_slice8(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                int64_t T, int64_t E, int64_t H, int64_t ncp,
                                                int8_t* __restrict__ dig, int* __restrict__ rexp,
                                                double* __restrict__ rres, double* __restrict__ norm,
                                                int* __restrict__ ulist, int* __restrict__ diag,
                                                uint32_t* __restrict__ rowam) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (blockIdx.x == 0 && tid < 4) {  // the list filled by k_logits_i8; the selection kernel's counters
    if (tid == 0) *ulist = 0;
    diag[tid] = 0;
  }
  __shared__ uint32_t s_mx[4], s_fm[4];
  __shared__ double s_res[4];
  const int sub = (tid >> 6) % WPR;  // this wave's share of the row
  const int64_t r = (int64_t)blockIdx.x * (4 / WPR) + (tid >> 6) / WPR;
  if (WPR == 1 && r >= T + E) return;  // WPR > 1: one row per workgroup, the grid holds exactly T + E
  const uint16_t* p = r < T ? x + r * H : w + (r - T) * H;
  const int nh = (int)(H / 16), nhp = (int)(ncp * 2);
  const int lj = sub * 64 + lane;  // first half chunk of this lane; then every 64 WPR
  constexpr int JS = 64 * WPR;
  auto load16 = [&](int j, uint32_t* u) {
    const uint4 q0 = *reinterpret_cast<const uint4*>(p + 16 * (int64_t)j);
    const uint4 q1 = *reinterpret_cast<const uint4*>(p + 16 * (int64_t)j + 8);
    u[0] = q0.x; u[1] = q0.y; u[2] = q0.z; u[3] = q0.w;
    u[4] = q1.x; u[5] = q1.y; u[6] = q1.z; u[7] = q1.w;
  };
  constexpr int NCC = NC > 0 ? NC : 1;
  uint32_t cu[NCC][8];
  uint32_t mx = 0u;  // largest magnitude bit pattern
  uint32_t fm = 0u;  // the same without NaN (x rows, when rowam is given)
  const bool want_fm = WPR > 1 && rowam && r < T;  // the same in the workgroup
  if constexpr (NC > 0) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {  // clamped loads: no load under a branch
      const int j = lj + JS * c;
      load16(j < nh ? j : nh - 1, cu[c]);
      if (j >= nh)
#pragma unroll
        for (int i = 0; i < 8; ++i) cu[c][i] = 0u;
      mx = max(mx, max_mag16(cu[c]));
      if constexpr (WPR > 1)
        if (want_fm) fm = max(fm, max_fin16(cu[c]));
    }
  } else {
    for (int j = lj; j < nh; j += JS) {
      load16(j, cu[0]);
      mx = max(mx, max_mag16(cu[0]));
      if constexpr (WPR > 1)
        if (want_fm) fm = max(fm, max_fin16(cu[0]));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  if constexpr (WPR > 1) {
    if (want_fm)
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) fm = max(fm, (uint32_t)__shfl_xor((int)fm, o, 64));
    if (lane == 0) {
      s_mx[tid >> 6] = mx;
      s_fm[tid >> 6] = fm;
    }
    __syncthreads();
    mx = max(max(s_mx[0], s_mx[1]), max(s_mx[2], s_mx[3]));
    fm = max(max(s_fm[0], s_fm[1]), max(s_fm[2], s_fm[3]));
    if (want_fm && lane == 0 && sub == 0) rowam[r] = fm << 16;
  }
  const bool bad = mx >= 0x7F80u;  // Inf or NaN in the row
  const int meb = (int)(mx >> 7);
  const int ex = mx == 0u ? kI8ZeroRow : meb ? meb - 126 : -133 + (32 - __builtin_clz(mx));
  const bool flt = ex >= -100, live = !bad && mx != 0u;
  double res = 0.0;
  int8_t* drow = dig + r * ncp * kI8ChunkB;
  auto emit = [&](int j, const uint32_t* u, bool data) {
    uint32_t o4[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) o4[a][c] = 0u;
    if (data && live) slice16(u, ex, flt, res, o4);
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<uint4*>(drow + 256 * (int64_t)(j >> 2) + 64 * a + 16 * (j & 3)) =
          make_uint4(o4[a][0], o4[a][1], o4[a][2], o4[a][3]);
  };
  int j0 = lj;
  if constexpr (NC > 0) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int j = lj + JS * c;
      if (j < nhp) emit(j, cu[c], j < nh);
    }
    j0 = lj + JS * NC;
  }
  for (int j = j0; j < nhp; j += JS) {  // NC == 0: every half chunk; NC > 0: the zero padding past them
    const bool data = j < nh;
    if (data) load16(j, cu[0]);
    emit(j, cu[0], data);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) res += __shfl_xor(res, o, 64);
  if constexpr (WPR > 1) {
    if (lane == 0) s_res[tid >> 6] = res;
    __syncthreads();
    res = ((s_res[0] + s_res[1]) + s_res[2]) + s_res[3];
  }
  if (lane == 0 && sub == 0) {
    rexp[r] = ex;
    // fewer than 2^15 nonnegative terms: the binary64 sum is within a factor 1 + 2^-30 of the exact one
    rres[r] = bad ? (double)INFINITY : res * (1.0 + 0x1p-30);
    // sqrt(H) max|v| >= the 2-norm; max|v| < 2^X
    norm[r] = mx == 0u ? 0.0 : sqrt((double)H) * ldexp(1.0, ex) * (1.0 + 0x1p-40);
  }
}

// Round hi 2^(base + 48) + lo 2^base (exact integers) once to binary32.
__device__ inline float round_i128_f32(int64_t hi, int64_t lo, int base) {
  const __int128 v = ((__int128)hi << 48) + (__int128)lo;
  if (v == 0) return 0.0f;
  const bool neg = v < 0;
  const unsigned __int128 m = neg ? (unsigned __int128)(-v) : (unsigned __int128)v;
  const uint64_t mh = (uint64_t)(m >> 64), ml = (uint64_t)m;
  if (mh == 0) return round_u64_to_f32(ml, false, base, neg);
  const int lz = __builtin_clzll(mh);
  const uint64_t W = lz ? ((mh << lz) | (ml >> (64 - lz))) : mh;
  return round_u64_to_f32(W, (ml << lz) != 0ull, base + 64 - lz, neg);
}

// The logit from its exact digit sum hi 2^48 + lo (in units of 2^(Xx - 30) 2^(Xw - 30)) and the two rows'
// exponent bounds and residuals; NaN when a residual leaves the binary32 rounding unproven.
__device__ inline float i8_round(int64_t hi, int64_t lo, int xe, int we, double rx, double rw) {
  const int base = (xe - 30) + (we - 30);
  if (rx == 0.0 && rw == 0.0) return round_i128_f32(hi, lo, base);
  const int64_t c = lo >> 48;  // hi 2^48 + lo = (hi + c) 2^48 + (lo - c 2^48), the second part in [0, 2^48)
  const double S = ldexp((double)(hi + c), base + 48) + ldexp((double)(lo - c * (1ll << 48)), base);  // one rounding
  const double err = rx * ldexp(1.0, we) + ldexp(1.0, xe) * rw + fabs(S) * 0x1p-52;
  float r;
  if (!f32_certified(S, err, &r)) r = __builtin_nanf("");
  return r;
}

typedef int i8x16_t __attribute__((ext_vector_type(4)));   // 16 int8 digits
typedef int i32x16_t __attribute__((ext_vector_type(16)));

// A workgroup owns 64 tokens x 64 experts, each of its 4 waves 32 x 32 on
// v_mfma_i32_32x32x32_i8 with seven accumulators (one per digit diagonal j).
// K goes in stages of two chunks through double-buffered LDS (rows padded by
// 16 bytes; a stage block's [digit][half chunk] pieces stored as [half chunk][digit]).  Lane l of an operand carries row l % 32 and half l / 32 of a
// chunk (the same k for both operands, which is all the sum needs); result
// register 4q + i of lane l is token row 8q + 4 (l / 32) + i, expert l % 32.
// With a multiple of 8 workgroups, the expert tiles of one token tile run on
// one XCD, so the token digits are read from HBM once.  SPLIT (small
// batches): blockIdx.y takes sps stages of K and the workgroup stores its
// exact partial (hi, lo) of every logit for k_fin_i8.
template <bool SPLIT>
__global__ __launch_bounds__(256, 2) void k_logits_i8(const int8_t* __restrict__ dig, int64_t T, int64_t E,
                                                      int64_t ncp, int64_t sps, const int* __restrict__ rexp,
                                                      const double* __restrict__ rres, float* __restrict__ logits,
                                                      int* __restrict__ ulist, int* __restrict__ blk,
                                                      int64_t* __restrict__ spart) {
  __shared__ __attribute__((aligned(16))) int8_t tl[2][2][kI8Rows * kI8Ld];  // [buffer][x, w]
  __shared__ int n_unc;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t ne = (E + kI8Rows - 1) / kI8Rows, nwg = ((T + kI8Rows - 1) / kI8Rows) * ne;
  const int64_t b = blockIdx.x;
  const int64_t lt = (nwg % 8 == 0) ? (b % 8) * (nwg / 8) + b / 8 : b;
  const int64_t t0 = (lt / ne) * kI8Rows, e0 = (lt % ne) * kI8Rows;
  if (tid == 0) n_unc = 0;
  // staging: 8 loads of 16 bytes per thread and stage (piece seg of the stage block: digit seg / 4, half
  // chunk seg % 4); rows past T or E repeat the last row
  const int64_t rowb = ncp * kI8ChunkB;
  const int8_t* src[8];
  int dst[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int idx = q * 256 + tid, op = idx >> 10, rr = (idx >> 4) & 63, seg = idx & 15;
    const int d = seg >> 2, hj = seg & 3;
    const int64_t row = op == 0 ? (t0 + rr < T ? t0 + rr : T - 1) : T + (e0 + rr < E ? e0 + rr : E - 1);
    src[q] = dig + row * rowb + seg * 16;
    dst[q] = op * (kI8Rows * kI8Ld) + rr * kI8Ld + (hj >> 1) * kI8ChunkB + (hj & 1) * 64 + d * 16;
  }
  // two register sets: a stage's digits are loaded two stages before they are multiplied; indices past
  // the last stage are clamped (those loads are never stored), so no load sits under a branch
  i8x16_t ga[8], gb[8];
  const int64_t nst = ncp / kI8Stage;  // even
  const int64_t sb = SPLIT ? (int64_t)blockIdx.y * sps : 0;
  const int64_t se = SPLIT ? (sb + sps < nst ? sb + sps : nst) : nst;  // stages [sb, se), an even count
  auto gload = [&](i8x16_t* g, int64_t s) {
    const int64_t sc = s < se ? s : se - 1;
#pragma unroll
    for (int q = 0; q < 8; ++q) g[q] = *reinterpret_cast<const i8x16_t*>(src[q] + sc * (kI8Stage * kI8ChunkB));
  };
  auto lstore = [&](const i8x16_t* g, int buf) {
#pragma unroll
    for (int q = 0; q < 8; ++q) *reinterpret_cast<i8x16_t*>(&tl[buf][0][0] + dst[q]) = g[q];
  };
  i32x16_t acc[7];
#pragma unroll
  for (int d = 0; d < 7; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[d][i] = 0;
  const int ar = (wv & 1) * 32 + (lane & 31), br = (wv >> 1) * 32 + (lane & 31), hoff = (lane >> 5) * 64;
  auto multiply = [&](int buf) {
    const int8_t* A = &tl[buf][0][ar * kI8Ld + hoff];
    const int8_t* B = &tl[buf][1][br * kI8Ld + hoff];
#pragma unroll
    for (int cc = 0; cc < kI8Stage; ++cc) {
      i8x16_t a[4], bb[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        a[d] = *reinterpret_cast<const i8x16_t*>(A + cc * kI8ChunkB + d * 16);
        bb[d] = *reinterpret_cast<const i8x16_t*>(B + cc * kI8ChunkB + d * 16);
      }
#pragma unroll
      for (int d1 = 0; d1 < 4; ++d1)
#pragma unroll
        for (int d2 = 0; d2 < 4; ++d2)
          acc[d1 + d2] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[d1], bb[d2], acc[d1 + d2], 0, 0, 0);
    }
  };
  gload(ga, sb);
  gload(gb, sb + 1);
  lstore(ga, 0);
  __syncthreads();
  for (int64_t s = sb; s < se; s += 2) {
    gload(ga, s + 2);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the multiplies
    multiply(0);
    lstore(gb, 1);
    __syncthreads();
    gload(gb, s + 3);
    __builtin_amdgcn_sched_barrier(0);
    multiply(1);
    lstore(ga, 0);
    __syncthreads();
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the clamped loads of the last stages have landed
  int nu = 0;
  const int64_t e = e0 + (wv >> 1) * 32 + (lane & 31);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 + (wv & 1) * 32 + 8 * q + 4 * (lane >> 5) + i;
      if (t >= T || e >= E) continue;
      const int g = 4 * q + i;
      // sum_j D_j 2^(8 (6 - j)) = hi 2^48 + lo, both exact in int64
      const int64_t D0 = acc[0][g], D1 = acc[1][g], D2 = acc[2][g], D3 = acc[3][g];
      const int64_t hi = D0 + (D1 >> 8) + (D2 >> 16) + (D3 >> 24);
      const int64_t lo = (int64_t)acc[6][g] + ((int64_t)acc[5][g] << 8) + ((int64_t)acc[4][g] << 16) +
                         ((D3 & 0xFFFFFF) << 24) + ((D2 & 0xFFFF) << 32) + ((D1 & 0xFF) << 40);
      if constexpr (SPLIT) {
        int64_t* o = spart + 2 * (((int64_t)blockIdx.y * T + t) * E + e);
        o[0] = hi;
        o[1] = lo;
      } else {
        const float r = i8_round(hi, lo, rexp[t], rexp[T + e], rres[t], rres[T + e]);
        logits[t * E + e] = r;
        if (r != r) {
          ++nu;
          ulist[1 + atomicAdd(ulist, 1)] = (int)(t * E + e);
        }
      }
    }
  }
  if constexpr (!SPLIT) {
    if (nu) atomicAdd(&n_unc, nu);
    __syncthreads();
    if (tid == 0) blk[b] = n_unc;
  }
}

// Small batches: one thread per logit adds the K splits' exact partials (in
// int64: |hi| < 2^26 and |lo| < 2^51 per split, at most 2^10 splits) and
// rounds them; the unproven go to the list.
__global__ __launch_bounds__(256) void k_fin_i8(int64_t T, int64_t E, int64_t s8,
                                                const int64_t* __restrict__ spart, const int* __restrict__ rexp,
                                                const double* __restrict__ rres, float* __restrict__ logits,
                                                int* __restrict__ ulist, int* __restrict__ blk) {
  __shared__ int n_unc;
  const int tid = threadIdx.x;
  if (tid == 0) n_unc = 0;
  __syncthreads();
  const int64_t idx = (int64_t)blockIdx.x * 256 + tid;
  if (idx < T * E) {
    const int64_t t = idx / E, e = idx % E;
    int64_t hi = 0, lo = 0;
#pragma unroll 8
    for (int64_t z = 0; z < s8; ++z) {  // unrolled: the loads of 8 splits are in flight together
      const int64_t* pz = spart + 2 * (z * T * E + idx);
      hi += pz[0];
      lo += pz[1];
    }
    const float r = i8_round(hi, lo, rexp[t], rexp[T + e], rres[t], rres[T + e]);
    logits[idx] = r;
    if (r != r) {
      atomicAdd(&n_unc, 1);
      ulist[1 + atomicAdd(ulist, 1)] = (int)idx;
    }
  }
  __syncthreads();
  if (tid == 0) blk[blockIdx.x] = n_unc;
}

// The listed logits, exactly: each workgroup takes list entries blockIdx.x,
// blockIdx.x + gridDim.x, ... (the list order does not matter: every entry's
// value is exact).
template <bool XB, bool WB>
__global__ __launch_bounds__(128) void k_exact_list(const void* __restrict__ x, const void* __restrict__ w, int64_t E,
                                                    int64_t H, const double* __restrict__ norm, int64_t T,
                                                    const int* __restrict__ ulist, float* __restrict__ logits) {
  __shared__ ExactLds xl;
  const int n = ulist[0];
  for (int u = blockIdx.x; u < n; u += gridDim.x) {
    const int64_t i = ulist[1 + u], t = i / E, e = i % E;
    const float r = exact_logit_wg<XB, WB, 128>(x, w, t, e, H, abs_bound(norm[t], norm[T + e]), &xl);
    if (threadIdx.x == 0) logits[i] = r;
  }
}

// Wave-wide maximum of a 64-bit key, returned to every lane.  Data-parallel
// primitive moves: swaps within quads (lane ^ 1, lane ^ 2), mirrors within 8
// and 16 lanes (after the quad steps each mirror pairs lanes of different
// halves), then row broadcasts of lane 15 into rows 1 and 3 and of lane 31
// into rows 2 and 3, which leaves the maximum in lane 63; lanes a step does
// not write keep their own key (max with itself).
template <int CTRL, int ROWS>
__device__ inline uint64_t dpp_max_step(uint64_t v) {
  const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xF, false);
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xF, false);
  const uint64_t u = ((uint64_t)ohi << 32) | olo;
  return u > v ? u : v;
}

__device__ inline uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0xB1, 0xF>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_max_step<0x4E, 0xF>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_max_step<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max_step<0x140, 0xF>(v);  // row_mirror
  v = dpp_max_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

constexpr int kMaxE = 1024;
constexpr int kSelThreads = 256;

// One workgroup per token: exactly rounded sigmoid (binary64 certified,
// double-double fallback), group top-2 sums, group selection, iterative
// (score, index) argmax in wave 0, normalization.
__global__ __launch_bounds__(kSelThreads) void k_select(const float* __restrict__ logits, int64_t E, int n_group,
                                                        int topk_group, int topk, int32_t* __restrict__ ids,
                                                        float* __restrict__ wts, float* __restrict__ scores,
                                                        const int* __restrict__ blk, int64_t nblk,
                                                        int* __restrict__ diag) {
  __shared__ float s_lds[kMaxE];
  __shared__ unsigned long long keys[kMaxE];
  __shared__ float g_lds[64];
  __shared__ int kept[64];
  __shared__ int s_cnt;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  if (t == 0) {  // diagnostics: exact recomputations of all logits workgroups
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    int c = 0;
    for (int64_t i = tid; i < nblk; i += kSelThreads) c += blk[i];
    if (c) atomicAdd(&s_cnt, c);
    __syncthreads();
    if (tid == 0) diag[0] = s_cnt;
  }
  int nslow = 0;
  for (int64_t e = tid; e < E; e += kSelThreads) {
    bool fast;
    const float sv = sigmoid_f32_exact(logits[t * E + e], &fast);
    nslow += fast ? 0 : 1;
    s_lds[e] = sv;
    if (scores) scores[t * E + e] = sv;
  }
  if (nslow) atomicAdd(&diag[1], nslow);
  __syncthreads();
  const int gsz = (int)(E / n_group);
  if (tid < n_group) {
    float t1 = -1.0f, t2 = -1.0f;
    for (int i = 0; i < gsz; ++i) {
      const float v = s_lds[tid * gsz + i];
      if (v > t1) {
        t2 = t1;
        t1 = v;
      } else if (v > t2) {
        t2 = v;
      }
    }
    g_lds[tid] = t1 + t2;
  }
  __syncthreads();
  if (tid < n_group) {
    const float gj = g_lds[tid];
    int rank = 0;
    for (int i = 0; i < n_group; ++i) {
      const float gi = g_lds[i];
      rank += (gi > gj || (gi == gj && i < tid)) ? 1 : 0;
    }
    kept[tid] = rank < topk_group ? 1 : 0;
  }
  __syncthreads();
  // (score, index) keys: larger score first, then lower index; 0 = not a candidate
  for (int64_t e = tid; e < E; e += kSelThreads)
    keys[e] = kept[e / gsz] ? ((uint64_t)f2u(s_lds[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e) : 0ull;
  __syncthreads();
  if (tid >= 64) return;  // wave 0 selects; no barrier follows
  int my_id = 0;
  float my_s = 0.0f;
  float ssum = 0.0f;
  for (int r = 0; r < topk; ++r) {
    uint64_t m = 0;
    for (int64_t e = lane; e < E; e += 64) m = keys[e] > m ? keys[e] : m;
    m = wave_max_u64(m);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)m);
    const float sv = u2f((uint32_t)(m >> 32));
    if (lane == (e & 63)) keys[e] = 0ull;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    ssum = (r == 0) ? sv : ssum + sv;
    if (lane == r) {
      my_id = e;
      my_s = sv;
    }
  }
  if (lane < topk) {
    ids[t * topk + lane] = my_id;
    wts[t * topk + lane] = my_s / ssum;
  }
}

// 256 experts, groups of a multiple of 4: one wave per token, four
// consecutive experts per lane, so a group is gsz / 4 consecutive lanes.
// Same results as k_select (the same exactly rounded sigmoid, binary32 sum of
// the group's two best, (score, index) keys, binary32 running sum in output
// order), with shuffles in place of LDS and barriers.
constexpr int kSel4Tokens = 4;  // waves (tokens) per workgroup

__device__ inline void top2_merge(float& a1, float& a2, float b1, float b2) {
  // the two largest (as a multiset) of {a1 >= a2} and {b1 >= b2}
  const bool ah = a1 >= b1;
  const float n2 = ah ? (a2 >= b1 ? a2 : b1) : (a1 >= b2 ? a1 : b2);
  a1 = ah ? a1 : b1;
  a2 = n2;
}

// The selection of token t by one wave from its 256 logits, four consecutive experts per lane (l4).
__device__ inline void select256_wave(float4 l4, int64_t t, int lpg, int topk_group, int topk,
                                      int32_t* __restrict__ ids, float* __restrict__ wts, float* __restrict__ scores,
                                      int* __restrict__ diag) {
  constexpr int64_t E = 256;
  const int lane = threadIdx.x & 63;
  bool f0, f1, f2, f3;
  float sv[4] = {sigmoid_f32_exact(l4.x, &f0), sigmoid_f32_exact(l4.y, &f1), sigmoid_f32_exact(l4.z, &f2),
                 sigmoid_f32_exact(l4.w, &f3)};
  const int nslow = (f0 ? 0 : 1) + (f1 ? 0 : 1) + (f2 ? 0 : 1) + (f3 ? 0 : 1);
  if (nslow) atomicAdd(&diag[1], nslow);
  if (scores) *reinterpret_cast<float4*>(scores + t * E + 4 * lane) = make_float4(sv[0], sv[1], sv[2], sv[3]);
  // the group's two best: this lane's four, then a butterfly over the group's lanes
  float t1 = -1.0f, t2 = -1.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (sv[i] > t1) {
      t2 = t1;
      t1 = sv[i];
    } else if (sv[i] > t2) {
      t2 = sv[i];
    }
  }
  for (int o = 1; o < lpg; o <<= 1) {
    const float b1 = __shfl_xor(t1, o, 64), b2 = __shfl_xor(t2, o, 64);
    top2_merge(t1, t2, b1, b2);
  }
  const float gj = t1 + t2;
  const int ng = 64 / lpg, my_g = lane / lpg;
  int rank = 0;
  for (int i = 0; i < ng; ++i) {
    const float gi = __shfl(gj, i * lpg, 64);
    rank += (gi > gj || (gi == gj && i < my_g)) ? 1 : 0;
  }
  const bool kept = rank < topk_group;
  // (score, index) keys: larger score first, then lower index; 0 = not a candidate
  uint64_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    key[i] = kept ? ((uint64_t)f2u(sv[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(4 * lane + i)) : 0ull;
  int my_id = 0;
  float my_s = 0.0f, ssum = 0.0f;
  for (int r = 0; r < topk; ++r) {
    uint64_t m = key[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) m = key[i] > m ? key[i] : m;
    m = wave_max_u64(m);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)m);
    const float s = u2f((uint32_t)(m >> 32));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * lane + i == e) key[i] = 0ull;
    ssum = (r == 0) ? s : ssum + s;
    if (lane == r) {
      my_id = e;
      my_s = s;
    }
  }
  if (lane < topk) {
    ids[t * topk + lane] = my_id;
    wts[t * topk + lane] = my_s / ssum;
  }
}

__global__ __launch_bounds__(64 * kSel4Tokens) void k_select256(
    const float* __restrict__ logits, int64_t T, int lpg, int topk_group, int topk, int32_t* __restrict__ ids,
    float* __restrict__ wts, float* __restrict__ scores, const int* __restrict__ blk, int64_t nblk,
    int* __restrict__ diag) {
  constexpr int64_t E = 256;
  __shared__ int s_cnt;
  const int tid = threadIdx.x, lane = tid & 63;
  if (blockIdx.x == 0) {  // diagnostics: exact recomputations of all logits workgroups
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    int c = 0;
    for (int64_t i = tid; i < nblk; i += 64 * kSel4Tokens) c += blk[i];
    if (c) atomicAdd(&s_cnt, c);
    __syncthreads();
    if (tid == 0) diag[0] = s_cnt;
  }
  const int64_t t = (int64_t)blockIdx.x * kSel4Tokens + (tid >> 6);
  if (t >= T) return;  // whole waves leave; no barrier follows
  select256_wave(*reinterpret_cast<const float4*>(logits + t * E + 4 * lane), t, lpg, topk_group, topk, ids, wts,
                 scores, diag);
}

// bf16 router on the int8 matrix cores with K cut into splits (small batches), 256 experts: the
// selection kernel also finishes the logits, in place of the finalize and exact-list kernels.  One
// token per workgroup: thread e adds the splits' exact partials of logit (t, e) in int64 and rounds them
// once (the arithmetic of k_fin_i8).  Logits whose rounding the bound left unproven (NaN) are then
// recomputed exactly by the whole workgroup, one after another (exact_logit_wg), and counted in
// diag[0]; then wave 0 selects.  (At large batches the exact recomputation stays in k_exact_list: its
// slow path needs per-lane scratch, which would limit how many selection workgroups run at once.)
// xcodes (optional): the workgroup also quantizes its token's row of x to NVFP4 ("NVFP4 quantization"
// page, "Quantization scheme") while wave 0 selects: S_g = max|x| / 2688 from the row maxima of k_slice8
// (rowam, T of them, reduced by every workgroup: no atomics), s_b = E4M3(a_b / (6 S_g)),
// q = E2M1(fl32(x / (s_b S_g))) by the division itself; workgroup 0 writes S_g.
__global__ __launch_bounds__(256) void k_select256_fin(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int64_t T, int64_t H,
    const int64_t* __restrict__ spart, int64_t s8, const int* __restrict__ rexp, const double* __restrict__ rres,
    const double* __restrict__ norm, float* __restrict__ logits, int lpg, int topk_group, int topk,
    int32_t* __restrict__ ids, float* __restrict__ wts, float* __restrict__ scores, int* __restrict__ diag,
    const uint32_t* __restrict__ rowam, uint8_t* __restrict__ xcodes, uint8_t* __restrict__ xscales,
    float* __restrict__ xgs) {
  constexpr int64_t E = 256;
  __shared__ __attribute__((aligned(16))) float s_log[E];
  __shared__ int s_list[E];
  __shared__ int s_n;
  __shared__ uint32_t s_am[4];
  __shared__ ExactLds xl;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t t = blockIdx.x, e = tid;
  if (tid == 0) s_n = 0;
  if (xcodes) {  // max|x|: the largest of the row maxima (non-negative binary32 bits order as their values)
    uint32_t am = 0u;
    for (int64_t i = tid; i < T; i += 256) am = max(am, rowam[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, o, 64));
    if (lane == 0) s_am[tid >> 6] = am;
  }
  __syncthreads();
  int64_t hi = 0, lo = 0;
#pragma unroll 8
  for (int64_t z = 0; z < s8; ++z) {  // unrolled: the loads of 8 splits are in flight together
    const int64_t* pz = spart + 2 * ((z * T + t) * E + e);
    hi += pz[0];
    lo += pz[1];
  }
  const float r = i8_round(hi, lo, rexp[t], rexp[T + e], rres[t], rres[T + e]);
  s_log[e] = r;
  logits[t * E + e] = r;
  if (r != r) s_list[atomicAdd(&s_n, 1)] = (int)e;
  __syncthreads();
  const int n = s_n;  // the same in every thread
  for (int u = 0; u < n; ++u) {
    const int ee = s_list[u];
    const float v = exact_logit_wg<true, true, 256>(x, w, t, ee, H, abs_bound(norm[t], norm[T + ee]), &xl);
    if (tid == 0) {
      s_log[ee] = v;
      logits[t * E + ee] = v;
    }
  }
  if (n) {
    if (tid == 0) atomicAdd(&diag[0], n);
    __syncthreads();
  }
  if (tid >= 64) {  // waves 1-3 quantize the token's row while wave 0 selects; no barrier follows
    if (xcodes) {
      const float S = u2f(max(max(s_am[0], s_am[1]), max(s_am[2], s_am[3]))) / 2688.0f;
      if (t == 0 && tid == 64) *xgs = S;
      const float d1 = 6.0f * S;
      const int64_t nb = H / 16;
      for (int64_t j = tid - 64; j < nb; j += 192) {
        const int64_t f = t * nb + j;
        const uint4 q0 = *reinterpret_cast<const uint4*>(x + 16 * f);
        const uint4 q1 = *reinterpret_cast<const uint4*>(x + 16 * f + 8);
        const uint32_t u[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        float v[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[2 * i] = u2f(u[i] << 16);
          v[2 * i + 1] = u2f(u[i] & 0xFFFF0000u);
        }
        float ab = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) ab = fmaxf(ab, fabsf(v[i]));
        const uint32_t sc = S != 0.0f ? e4m3_code_mag(ab / d1) : 0u;
        const float sv = e4m3_value_mag(sc), d2 = sv * S;
        uint32_t c[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t q = ((f2u(v[i]) >> 31) << 3) | (sv != 0.0f ? e2m1_code_mag(fabsf(v[i]) / d2) : 0u);
          c[i >> 3] |= q << (4 * (i & 7));
        }
        *reinterpret_cast<uint2*>(xcodes + 8 * f) = make_uint2(c[0], c[1]);
        xscales[f] = (uint8_t)sc;
      }
    }
    return;
  }
  select256_wave(*reinterpret_cast<const float4*>(&s_log[4 * lane]), t, lpg, topk_group, topk, ids, wts, scores, diag);
}

// fewer rows than waves in flight on the chip: four waves per row
bool slice8_few(int64_t T, int64_t E) { return T + E < 4096; }

// rowam is taken with four waves per row only (slice8_few)
void launch_slice8(const uint16_t* x, const uint16_t* w, int64_t T, int64_t E, int64_t H, int64_t ncp, int8_t* dig,
                   int* rexp, double* rres, double* norm, int* ulist, int* diag, hipStream_t st,
                   uint32_t* rowam = nullptr) {
  const bool few = slice8_few(T, E);
  const unsigned g = (unsigned)(few ? T + E : (T + E + 3) / 4);
  const int64_t nc = (H / 16 + (few ? 255 : 63)) / (few ? 256 : 64);  // half chunks per lane
#define BSM_SLICE8(N, W) \
  k_slice8<N, W><<<g, 256, 0, st>>>(x, w, T, E, H, ncp, dig, rexp, rres, norm, ulist, diag, rowam)
#define BSM_SLICE8_NC(W)       \
  switch (nc) {                \
    case 1: BSM_SLICE8(1, W); break; \
    case 2: BSM_SLICE8(2, W); break; \
    case 3: BSM_SLICE8(3, W); break; \
    case 4: BSM_SLICE8(4, W); break; \
    case 5: BSM_SLICE8(5, W); break; \
    case 6: BSM_SLICE8(6, W); break; \
    case 7: BSM_SLICE8(7, W); break; \
    case 8: BSM_SLICE8(8, W); break; \
    default: BSM_SLICE8(0, W); break; \
  }
  if (few) {
    BSM_SLICE8_NC(4)
  } else {
    BSM_SLICE8_NC(1)
  }
#undef BSM_SLICE8_NC
#undef BSM_SLICE8
}

__global__ void k_copy_diag(const int* src, int32_t* dst) {
  if (threadIdx.x < 4) dst[threadIdx.x] = src[threadIdx.x];
}

}  // namespace

size_t route_ws(int64_t T, int64_t H, int64_t E) { return route_layout(T, H, E).total; }
size_t route_diag_offset(int64_t T, int64_t H, int64_t E) { return route_layout(T, H, E).diag; }

hipError_t launch_route(const void* x, bool xb, int64_t T, int64_t H, const void* w, bool wb, int64_t E, int n_group,
                        int topk_group, int topk, int32_t* ids, float* wts, float* scores, void* ws_, hipStream_t st,
                        uint32_t* rowam, uint8_t* xcodes, uint8_t* xscales, float* xgs, bool* x_done) {
  const RouteWs L = route_layout(T, H, E);
  uint8_t* ws = reinterpret_cast<uint8_t*>(ws_);
  float* logits = reinterpret_cast<float*>(ws + L.logits);
  int* blk = reinterpret_cast<int*>(ws + L.blk);
  int* diag = reinterpret_cast<int*>(ws + L.diag);
  double* norm = L.rb ? nullptr : reinterpret_cast<double*>(ws + L.norm);
  int* lsb = L.rb ? nullptr : reinterpret_cast<int*>(ws + L.lsb);
  double* part = L.rb ? nullptr : reinterpret_cast<double*>(ws + L.part);
  int* ulist = L.rb ? nullptr : reinterpret_cast<int*>(ws + L.ulist);
  if (x_done) *x_done = false;
  // the row maxima come with four waves per row; the selection kernel reads a row as 16-value blocks
  uint8_t* xc = slice8_few(T, E) && H % 16 == 0 ? xcodes : nullptr;
  if (T == 0) return hipSuccess;
  stage_mark(1, 0, st);
  const unsigned nrs = (unsigned)((T + E + 3) / 4);
  const bool vec = (H % 8) == 0;
  const unsigned nrb = (unsigned)(((T + kRbT - 1) / kRbT) * ((E + kRbE - 1) / kRbE));
  const dim3 gl((unsigned)((T + kTile - 1) / kTile), (unsigned)((E + kTile - 1) / kTile));
  const dim3 glz(gl.x, gl.y, (unsigned)L.ks);
  // bf16 x and w at large batches: exact integer dot products on the int8 matrix cores
  const bool i8 = L.i8ok && xb && wb;
  int8_t* dig = reinterpret_cast<int8_t*>(ws + L.dig);
  int64_t* spart = reinterpret_cast<int64_t*>(ws + L.spart);
  int* rexp = L.i8ok ? reinterpret_cast<int*>(ws + L.rexp) : nullptr;
  double* rres = L.i8ok ? reinterpret_cast<double*>(ws + L.rres) : nullptr;
  if (i8) {  // the small-batch int8 path needs the norms and the list too
    norm = reinterpret_cast<double*>(ws + L.norm);
    ulist = reinterpret_cast<int*>(ws + L.ulist);
  }
  // workgroups whose list counts the selection kernel adds up
  const int64_t nblk_used = i8 ? L.nblk8 : L.rb ? (int64_t)nrb : (int64_t)gl.x * gl.y;
  // one wave per token needs 256 experts, groups of a multiple of 4 and an aligned scores row
  const bool sel4 = E == 256 && (E / n_group) % 4 == 0 && topk <= 64 &&
                    ((uintptr_t)scores & 15) == 0;
#define BSM_ROUTE_DISPATCH(XB, WB)                                                                          \
  if (i8 && L.rb && sel4) { /* the selection kernel finishes the logits */                                  \
    launch_slice8(reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(w), T, E, H, L.ncp,  \
                  dig, rexp, rres, norm, ulist, diag, st, xc ? rowam : nullptr);                           \
    k_logits_i8<true><<<dim3(gl.x * gl.y, (unsigned)L.s8), 256, 0, st>>>(dig, T, E, L.ncp, L.sps8, rexp,     \
                                                                         rres, logits, ulist, blk, spart); \
    stage_mark(1, 1, st);                                                                                  \
    k_select256_fin<<<(unsigned)T, 256, 0, st>>>(reinterpret_cast<const uint16_t*>(x),                      \
                                                 reinterpret_cast<const uint16_t*>(w), T, H, spart, L.s8, rexp, \
                                                 rres, norm, logits, (int)(E / n_group) / 4, topk_group,   \
                                                 topk, ids, wts, scores, diag, rowam, xc, xscales, xgs);   \
    if (x_done) *x_done = xc != nullptr;                                                                   \
  } else {                                                                                                 \
  if (i8 && L.rb) {                                                                                        \
    launch_slice8(reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(w), T, E, H, L.ncp,  \
                  dig, rexp, rres, norm, ulist, diag, st);                                                 \
    k_logits_i8<true><<<dim3(gl.x * gl.y, (unsigned)L.s8), 256, 0, st>>>(dig, T, E, L.ncp, L.sps8, rexp,     \
                                                                         rres, logits, ulist, blk, spart); \
    k_fin_i8<<<(unsigned)L.nblk8, 256, 0, st>>>(T, E, L.s8, spart, rexp, rres, logits, ulist, blk);          \
  } else if (L.rb) {                                                                                       \
    k_logits_rb<XB, WB><<<nrb, 256, 0, st>>>(x, w, T, E, H, L.nadd, logits, blk, diag);                    \
  } else if (i8) {                                                                                         \
    launch_slice8(reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(w), T, E, H, L.ncp,  \
                  dig, rexp, rres, norm, ulist, diag, st);                                                 \
    k_logits_i8<false><<<gl.x * gl.y, 256, 0, st>>>(dig, T, E, L.ncp, L.sps8, rexp, rres, logits, ulist, blk, \
                                                     nullptr);                                              \
  } else {                                                                                                 \
    if (vec)                                                                                               \
      k_rowstats<XB, WB, true><<<nrs, 256, 0, st>>>(x, w, T, E, H, norm, lsb);                             \
    else                                                                                                   \
      k_rowstats<XB, WB, false><<<nrs, 256, 0, st>>>(x, w, T, E, H, norm, lsb);                            \
    if (H % kBK == 0)                                                                                      \
      k_logits<XB, WB, true><<<glz, 128, 0, st>>>(x, w, T, E, H, L.kslice, part, ulist);                   \
    else                                                                                                   \
      k_logits<XB, WB, false><<<glz, 128, 0, st>>>(x, w, T, E, H, L.kslice, part, ulist);                  \
    k_logits_fin<<<gl, 256, 0, st>>>(T, E, L.ks, part, norm, lsb, L.nadd, logits, ulist, blk, diag);        \
  }                                                                                                        \
  stage_mark(1, 1, st);                                                                                    \
  if (!L.rb || i8) k_exact_list<XB, WB><<<kExactWgs, 128, 0, st>>>(x, w, E, H, norm, T, ulist, logits);    \
  if (sel4)                                                                                                \
    k_select256<<<(unsigned)((T + kSel4Tokens - 1) / kSel4Tokens), 64 * kSel4Tokens, 0, st>>>(                \
        logits, T, (int)(E / n_group) / 4, topk_group, topk, ids, wts, scores, blk, nblk_used, diag);          \
  else                                                                                                     \
    k_select<<<(unsigned)T, kSelThreads, 0, st>>>(logits, E, n_group, topk_group, topk, ids, wts, scores,     \
                                                  blk, nblk_used, diag);                                    \
  }
  if (xb && wb) {
    BSM_ROUTE_DISPATCH(true, true)
  } else if (xb && !wb) {
    BSM_ROUTE_DISPATCH(true, false)
  } else if (!xb && wb) {
    BSM_ROUTE_DISPATCH(false, true)
  } else {
    BSM_ROUTE_DISPATCH(false, false)
  }
#undef BSM_ROUTE_DISPATCH
  stage_mark(1, 2, st);
  return hipGetLastError();
}

// Workspace of the routing + quantization call: the router's, then the row maxima of x (when the router's
// pass over x yields them), then the quantization's partial maxima (when it does not).
namespace {
struct RouteQWs {
  size_t rowam, parts, total;
};
RouteQWs route_q_layout(int64_t T, int64_t H, int64_t E) {
  RouteQWs L;
  L.rowam = align256(route_ws(T, H, E));
  L.parts = L.rowam + align256(sizeof(uint32_t) * (size_t)(T > 0 ? T : 1));
  L.total = L.parts + nvfp4_quant_ws(1, T, H);
  return L;
}
}  // namespace

size_t route_q_ws(int64_t T, int64_t H, int64_t E) { return route_q_layout(T, H, E).total; }

hipError_t launch_route_nvfp4_quantize(const void* x, bool xb, int64_t T, int64_t H, const void* w, bool wb,
                                       int64_t E, int n_group, int topk_group, int topk, int32_t* ids, float* wts,
                                       float* scores, uint8_t* codes, uint8_t* scales, float* gs, void* ws_,
                                       hipStream_t st) {
  const RouteQWs L = route_q_layout(T, H, E);
  uint8_t* ws = reinterpret_cast<uint8_t*>(ws_);
  bool fused = false;
  hipError_t err = launch_route(x, xb, T, H, w, wb, E, n_group, topk_group, topk, ids, wts, scores, ws_, st,
                                reinterpret_cast<uint32_t*>(ws + L.rowam), codes, scales, gs, &fused);
  if (err != hipSuccess || fused) return err;  // fused: the selection kernel quantized x
  return launch_nvfp4_quantize(x, xb, 1, T, H, codes, scales, gs, true, reinterpret_cast<float*>(ws + L.parts), st);
}

hipError_t launch_route_diag(const void* ws, int64_t T, int64_t H, int64_t E, int32_t* dst, hipStream_t st) {
  const int* src = reinterpret_cast<const int*>(reinterpret_cast<const uint8_t*>(ws) + route_layout(T, H, E).diag);
  k_copy_diag<<<1, 64, 0, st>>>(src, dst);
  return hipGetLastError();
}

}  // namespace bsm
