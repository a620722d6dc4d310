// bsm_ceil.hip -- measurement aids (not part of the method): the achievable
// ceilings of the GPU that the kernels' roofline fractions are also reported
// against.
//
//   k_ceil_read   streams a device buffer once with non-temporal 16-byte
//                 loads, four contiguous 4 KB pieces per workgroup and
//                 iteration, so every load instruction covers 8 whole 128-byte
//                 lines (the access pattern of the few-row GEMMs' weight
//                 streams; ordinary loads read about 15% slower), folding the
//                 words into one XOR per thread so the loads cannot be dropped
//   k_ceil_mfma   independent chains of FP16 MFMAs on register operands
//                 (32x32x16 or 16x16x32, FP32 accumulation): the matrix-core
//                 rate without any memory traffic

#include "bsm_internal.h"

namespace bsm {
namespace {

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

constexpr int kReadUnroll = 4;

__global__ __launch_bounds__(256) void k_ceil_read(const uint4* __restrict__ p, int64_t n16, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256 * kReadUnroll;
  for (int64_t base = (int64_t)blockIdx.x * 256 * kReadUnroll + threadIdx.x; base < n16; base += stride) {
    u4v v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      v[u] = i < n16 ? __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p) + i) : u4v{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

constexpr int kChains = 8;  // independent accumulator chains per wave

template <int SHAPE>  // 0: 32x32x16, 1: 16x16x32
__global__ __launch_bounds__(256) void k_ceil_mfma(int64_t iters, float* __restrict__ sink) {
  const _Float16 v = (_Float16)(float)(threadIdx.x & 7) * (_Float16)0.0009765625f;
  const h8v a = {v, v, v, v, v, v, v, v};
  const h8v b = {v, v, v, v, v, v, v, v};
  float s = 0.0f;
  if constexpr (SHAPE == 0) {
    f16v acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[c][q] = 0.0f;
    for (int64_t it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
      for (int q = 0; q < 16; ++q) s += acc[c][q];
  } else {
    f4v acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f4v{0.f, 0.f, 0.f, 0.f};
    for (int64_t it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) s += acc[c][q];
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_ceil_read(const void* buf, size_t bytes, uint32_t* sink, int wgs, hipStream_t st) {
  k_ceil_read<<<(unsigned)wgs, 256, 0, st>>>(reinterpret_cast<const uint4*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

hipError_t launch_ceil_mfma(int shape, int64_t iters, float* sink, int wgs, hipStream_t st) {
  if (shape == 0)
    k_ceil_mfma<0><<<(unsigned)wgs, 256, 0, st>>>(iters, sink);
  else
    k_ceil_mfma<1><<<(unsigned)wgs, 256, 0, st>>>(iters, sink);
  return hipGetLastError();
}

}  // namespace bsm
