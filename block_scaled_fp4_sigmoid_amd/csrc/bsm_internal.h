// bsm_internal.h -- declarations shared by the kernel translation units and
// the C ABI layer.  Launchers assume their arguments were validated by the
// ABI layer (shapes, alignment, workspace size) and return the HIP status of
// the enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bsm_numerics.h"

namespace bsm {

constexpr int kWave = 64;

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// ---- quantizers -----------------------------------------------------------
// per-tensor partial maxima of |x| (NVFP4 dynamic global scale)
constexpr int kAmaxMaxParts = 1024;
int nvfp4_amax_parts(int64_t R, int64_t C);
size_t nvfp4_quant_ws(int64_t B, int64_t R, int64_t C);
hipError_t launch_local_hessian(const void* x, bool x_bf16, int64_t N, int64_t C, double* out, hipStream_t st);
hipError_t launch_nvfp4_quantize_lh(const void* w, bool w_bf16, int64_t R, int64_t C, const double* hb, int radius,
                                    uint8_t* codes, uint8_t* scales, float* gs, float* parts, hipStream_t st);
hipError_t launch_nvfp4_quantize(const void* x, bool x_bf16, int64_t B, int64_t R, int64_t C, uint8_t* codes,
                                 uint8_t* scales, float* gs, bool dynamic, float* ws_partials,
                                 hipStream_t st);
// same, with the global amax already known (bits of a non-negative float at
// amax_bits, one per tensor) -- used for h whose amax comes from the GEMM epilogue
// dec16 (optional): also writes the exact FP16 values q * s_b (global scale not applied)
hipError_t launch_nvfp4_quantize_from_amax(const void* x, bool x_bf16, int64_t B, int64_t R, int64_t C,
                                           uint8_t* codes, uint8_t* scales, float* gs,
                                           const uint32_t* amax_bits, const float* static_gs,
                                           hipStream_t st, _Float16* dec16 = nullptr);
hipError_t launch_nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* gs, int64_t B,
                                   int64_t R, int64_t C, bool bf16_out, void* out, hipStream_t st);
// dec16 (optional): also writes the exact FP16 values of the E4M3 codes (row scale not applied)
hipError_t launch_fp8_quantize(const void* x, bool x_bf16, int64_t R, int64_t C, uint8_t* codes, float* scales,
                               hipStream_t st, _Float16* dec16 = nullptr);

// ---- router ---------------------------------------------------------------
size_t route_ws(int64_t T, int64_t H, int64_t E);
// rowam, xcodes, xscales, xgs (optional): when the path takes them (*x_done), the NVFP4 quantization of the
// same x (DYNAMIC global scale) into xcodes, xscales, xgs, with each x row's largest magnitude that is not
// NaN in rowam[T] (binary32 bits)
hipError_t launch_route(const void* x, bool x_bf16, int64_t T, int64_t H, const void* w, bool w_bf16, int64_t E,
                        int n_group, int topk_group, int topk, int32_t* ids, float* wts, float* scores, void* ws,
                        hipStream_t st, uint32_t* rowam = nullptr, uint8_t* xcodes = nullptr,
                        uint8_t* xscales = nullptr, float* xgs = nullptr, bool* x_done = nullptr);
// routing and NVFP4 quantization (DYNAMIC global scale) of the same x [T, H]
size_t route_q_ws(int64_t T, int64_t H, int64_t E);
hipError_t launch_route_nvfp4_quantize(const void* x, bool x_bf16, int64_t T, int64_t H, const void* w, bool w_bf16,
                                       int64_t E, int n_group, int topk_group, int topk, int32_t* ids, float* wts,
                                       float* scores, uint8_t* codes, uint8_t* scales, float* gs, void* ws,
                                       hipStream_t st);
size_t route_diag_offset(int64_t T, int64_t H, int64_t E);
hipError_t launch_route_diag(const void* ws, int64_t T, int64_t H, int64_t E, int32_t* dst, hipStream_t st);

// ---- expert MLP -----------------------------------------------------------
struct MoeLayout {
  size_t total, counts, offsets, row_pair, pair_row, tiles, h_f32, h_codes, h_scales, h_gs, y_f32, scratch;
  // scratch sub-buffers
  size_t sel_masks, chunk_cnt, chunk_base, ntiles, h_amax, act_f16, h_f16, tiles_w, ntiles_w, part;
  int64_t P, n_chunks, max_tiles, max_tiles_w;
};
MoeLayout moe_layout(bool nvfp4, int64_t E, int64_t H, int64_t I, int64_t T, int topk);

struct MoeArgs {
  bool nvfp4;
  bool a16 = false;  // weight-only W4A16: x_codes is BF16 x [T, H]; NVFP4 weights
  int64_t E, H, I, T;
  int topk;
  const uint8_t* w13_codes;
  const void* w13_scales;
  const float* w13_gs;
  const uint8_t* w2_codes;
  const void* w2_scales;
  const float* w2_gs;
  const uint8_t* x_codes;
  const void* x_scales;
  const float* x_gs;
  const int32_t* ids;
  const float* wts;
  bool pairs = false;  // weight codes in the pair layout (launch_codes_to_pairs)
  const uint8_t* w13_scales_lanes = nullptr;  // NVFP4 pairs: lane-ordered block scales (few-row GEMMs)
  const uint8_t* w2_scales_lanes = nullptr;
  float combine_scale;
  bool h_static;
  float* h_gs_user;
  float* out;
  uint8_t* ws;
};
hipError_t launch_moe(const MoeArgs& a, hipStream_t st);
// weight codes [rows, row_bytes] (rows % 16 == 0, row_bytes % 64 == 0) -> pair layout, out of place
hipError_t launch_codes_to_pairs(const uint8_t* in, uint8_t* out, int64_t rows, int64_t row_bytes, hipStream_t st);
// NVFP4 block scales [rows, row_bytes] (rows % 16 == 0, row_bytes % 32 == 0) -> lane order, out of place
hipError_t launch_scales_to_lanes(const uint8_t* in, uint8_t* out, int64_t rows, int64_t row_bytes, hipStream_t st);

// ---- dense FP8 linear ------------------------------------------------------
size_t fp8_linear_ws(int64_t T, int64_t K, int64_t N);
hipError_t launch_fp8_linear(const uint8_t* xc, const float* xs, const uint8_t* wc, const float* wsc, int64_t T,
                             int64_t K, int64_t N, float* out, uint8_t* ws, hipStream_t st);

// ---- stage events (profiling aid) -----------------------------------------
constexpr int kMaxStageEvents = 8;
struct StageEvents {
  hipEvent_t ev[kMaxStageEvents];
  int n = 0;
};
StageEvents& stage_events(int which);  // thread-local, which = 0 (moe) or 1 (route)
inline void stage_mark(int which, int i, hipStream_t st) {
  StageEvents& s = stage_events(which);
  if (i < s.n && s.ev[i]) (void)hipEventRecord(s.ev[i], st);
}

// ---- norm / residual ------------------------------------------------------
// measurement aids: HBM read and FP16 MFMA ceilings
hipError_t launch_ceil_read(const void* buf, size_t bytes, uint32_t* sink, int wgs, hipStream_t st);
hipError_t launch_ceil_mfma(int shape, int64_t iters, float* sink, int wgs, hipStream_t st);
hipError_t launch_rmsnorm(const float* x, int64_t T, int64_t H, float eps, const float* gamma, float* y,
                          hipStream_t st);
hipError_t launch_residual(float* x, const float* m, float a, float b, int64_t n, hipStream_t st);

}  // namespace bsm
