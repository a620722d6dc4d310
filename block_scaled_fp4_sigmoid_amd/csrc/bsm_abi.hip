// bsm_abi.hip -- extern "C" entry points declared in include/bsmoe.h:
// argument validation on the host, workspace sizing, kernel launches.
// Every check runs before anything is enqueued; on error nothing is launched.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/bsmoe.h"
#include "bsm_internal.h"

// Scratch of bsm_moe_expert_mlp_noalloc: a file-scope device array (each GPU the library runs on holds
// its own copy until the process ends).  Every call on a GPU shares that GPU's copy.
constexpr size_t kNoAllocScratchBytes = BSM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

thread_local char g_err[512] = {0};
thread_local bsm::StageEvents g_stage[2];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return BSM_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BSM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool dtype_ok(int d) { return d == BSM_BF16 || d == BSM_F32; }

int check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return BSM_OK;
  if (!ws) return fail(BSM_ERR_WORKSPACE, "workspace pointer is NULL (need %zu bytes)", need);
  if (!aligned(ws, 256)) return fail(BSM_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(BSM_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  return BSM_OK;
}

// Layout of the weight codes: the pair layout is read by the kernels that take a whole K step of the few-row
// GEMM (NVFP4 and W4A16: 512 values, FP8: 256) and by the many-row GEMM with I % 256 == 0, not by the
// fallbacks for other shapes or by the dense FP8 path (one expert, top-1, T <= 64).
static int check_layout(const bsm_moe_weights* w, bool nv, bool a16, int64_t T, int topk) {
  if (w->layout == BSM_LAYOUT_ROWS) return BSM_OK;
  if (w->layout != BSM_LAYOUT_PAIRS) return fail(BSM_ERR_INVALID_ARG, "bad weight layout %d", w->layout);
  const int64_t ks = nv ? 512 : 256;
  if (w->H % ks != 0 || w->I % ks != 0 || w->I % 256 != 0)
    return fail(BSM_ERR_UNSUPPORTED, "pair layout needs H and I multiples of %lld and I of 256", (long long)ks);
  if (!nv && !a16 && w->E == 1 && topk == 1 && T <= 64)
    return fail(BSM_ERR_UNSUPPORTED, "pair layout: not taken by the dense FP8 path (E = 1, topk = 1, T <= 64)");
  if (nv && T > 0 && (!w->w13_scales_lanes || !w->w2_scales_lanes))
    return fail(BSM_ERR_INVALID_ARG, "NVFP4 pair layout needs the lane-ordered scales");
  if (nv && T > 0 && (!aligned(w->w13_scales_lanes, 16) || !aligned(w->w2_scales_lanes, 16)))
    return fail(BSM_ERR_INVALID_ARG, "lane-ordered scales must be 16-byte aligned");
  return BSM_OK;
}

// Arguments of the routed-expert MLP, validated on the host (nothing is enqueued on error).  *empty:
// T == 0, nothing to do.
int moe_args(const bsm_moe_weights* w, const bsm_act_q* xq, int64_t T, const int32_t* topk_ids,
             const float* topk_weights, int topk, float combine_scale, int h_gs_mode, float* h_global_scale,
             float* out, bsm::MoeArgs* a, bool* empty) {
  if (!w || !xq) return fail(BSM_ERR_INVALID_ARG, "NULL weights / activation descriptor");
  if (w->format != BSM_FMT_NVFP4 && w->format != BSM_FMT_FP8) return fail(BSM_ERR_INVALID_ARG, "bad weight format");
  if (xq->format != w->format) return fail(BSM_ERR_INVALID_ARG, "activation and weight formats differ");
  const bool nv = w->format == BSM_FMT_NVFP4;
  const int64_t E = w->E, H = w->H, I = w->I;
  if (E <= 0 || H <= 0 || I <= 0 || T < 0) return fail(BSM_ERR_INVALID_ARG, "bad shape");
  if (H % 256 != 0 || I % 128 != 0) return fail(BSM_ERR_UNSUPPORTED, "H must be a multiple of 256 and I of 128");
  if (E > 1024) return fail(BSM_ERR_UNSUPPORTED, "E > 1024");
  if (topk < 1 || topk > 32 || topk > E) return fail(BSM_ERR_INVALID_ARG, "topk must be in [1, min(32, E)]");
  if (T * topk > 0x3FFFFFFF) return fail(BSM_ERR_UNSUPPORTED, "T * topk too large");
  if (h_gs_mode != BSM_GS_DYNAMIC && h_gs_mode != BSM_GS_STATIC) return fail(BSM_ERR_INVALID_ARG, "bad h_gs_mode");
  if (int r = check_layout(w, nv, false, T, topk)) return r;
  if (nv && h_gs_mode == BSM_GS_STATIC && !h_global_scale)
    return fail(BSM_ERR_INVALID_ARG, "STATIC h global scale needs h_global_scale");
  *empty = T == 0;
  if (*empty) return BSM_OK;
  if (!w->w13_codes || !w->w13_scales || !w->w2_codes || !w->w2_scales || !xq->codes || !xq->scales || !topk_ids ||
      !topk_weights || !out)
    return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  if (nv && (!w->w13_gs || !w->w2_gs || !xq->global_scale)) return fail(BSM_ERR_INVALID_ARG, "NULL global scale");
  if (!aligned(w->w13_codes, 16) || !aligned(w->w2_codes, 16) || !aligned(xq->codes, 16) || !aligned(out, 16))
    return fail(BSM_ERR_INVALID_ARG, "codes and out must be 16-byte aligned");
  if (nv && (!aligned(w->w13_scales, 2) || !aligned(w->w2_scales, 2) || !aligned(xq->scales, 2)))
    return fail(BSM_ERR_INVALID_ARG, "NVFP4 scales must be 2-byte aligned");
  a->nvfp4 = nv;
  a->E = E;
  a->H = H;
  a->I = I;
  a->T = T;
  a->topk = topk;
  a->w13_codes = w->w13_codes;
  a->w13_scales = w->w13_scales;
  a->w13_gs = w->w13_gs;
  a->w2_codes = w->w2_codes;
  a->w2_scales = w->w2_scales;
  a->w2_gs = w->w2_gs;
  a->x_codes = xq->codes;
  a->x_scales = xq->scales;
  a->x_gs = xq->global_scale;
  a->ids = topk_ids;
  a->wts = topk_weights;
  a->combine_scale = combine_scale;
  a->h_static = h_gs_mode == BSM_GS_STATIC;
  a->h_gs_user = h_global_scale;
  a->out = out;
  a->pairs = w->layout == BSM_LAYOUT_PAIRS;
  a->w13_scales_lanes = w->w13_scales_lanes;
  a->w2_scales_lanes = w->w2_scales_lanes;
  return BSM_OK;
}

// Device address of this GPU's copy of the static scratch (found once per device with that device
// current, then kept): host code uses this address, never the array's name, which on the host is only
// a stand-in for the symbol.
int noalloc_scratch(void** p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(BSM_ERR_HIP, "bsm_moe_expert_mlp_noalloc: no usable current device (%d)", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return fail(BSM_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *p = g_scratch_ptr[dev];
  return BSM_OK;
}

}  // namespace

namespace bsm {
StageEvents& stage_events(int which) { return g_stage[which]; }
}  // namespace bsm

extern "C" {

int bsm_abi_version(void) { return BSM_ABI_VERSION; }

const char* bsm_status_str(int s) {
  switch (s) {
    case BSM_OK: return "BSM_OK";
    case BSM_ERR_INVALID_ARG: return "BSM_ERR_INVALID_ARG";
    case BSM_ERR_UNSUPPORTED: return "BSM_ERR_UNSUPPORTED";
    case BSM_ERR_WORKSPACE: return "BSM_ERR_WORKSPACE";
    case BSM_ERR_HIP: return "BSM_ERR_HIP";
    default: return "BSM_ERR_UNKNOWN";
  }
}

const char* bsm_last_error(void) { return g_err; }

size_t bsm_nvfp4_quantize_workspace_size(int64_t B, int64_t R, int64_t C) {
  if (B < 0 || R < 0 || C < 0) return 0;
  return bsm::nvfp4_quant_ws(B, R, C);
}

int bsm_nvfp4_quantize(const void* x, int x_dtype, int64_t B, int64_t R, int64_t C, uint8_t* codes, uint8_t* scales,
                       float* global_scale, int gs_mode, void* ws, size_t ws_bytes, bsm_stream_t stream) {
  if (!dtype_ok(x_dtype)) return fail(BSM_ERR_INVALID_ARG, "x_dtype must be BSM_BF16 or BSM_F32");
  if (B < 0 || R < 0 || C < 0) return fail(BSM_ERR_INVALID_ARG, "negative shape");
  if (C % 16 != 0) return fail(BSM_ERR_INVALID_ARG, "C (%lld) must be a multiple of 16", (long long)C);
  if (B > 65535) return fail(BSM_ERR_UNSUPPORTED, "B (%lld) > 65535", (long long)B);
  if (gs_mode != BSM_GS_DYNAMIC && gs_mode != BSM_GS_STATIC) return fail(BSM_ERR_INVALID_ARG, "bad gs_mode");
  if (B * R * C == 0) return ok();
  if (!x || !codes || !scales || !global_scale) return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(x, 32) || !aligned(codes, 8)) return fail(BSM_ERR_INVALID_ARG, "x must be 32-byte and codes 8-byte aligned");
  const size_t need = gs_mode == BSM_GS_DYNAMIC ? bsm::nvfp4_quant_ws(B, R, C) : 0;
  if (int r = check_ws(ws, ws_bytes, need)) return r;
  return hip_status(bsm::launch_nvfp4_quantize(x, x_dtype == BSM_BF16, B, R, C, codes, scales, global_scale,
                                               gs_mode == BSM_GS_DYNAMIC, (float*)ws, (hipStream_t)stream),
                    "bsm_nvfp4_quantize");
}

int bsm_local_hessian_blocks(const void* x, int x_dtype, int64_t N, int64_t C, double* hess_blocks,
                             bsm_stream_t stream) {
  if (!dtype_ok(x_dtype)) return fail(BSM_ERR_INVALID_ARG, "x_dtype must be BSM_BF16 or BSM_F32");
  if (N < 0 || C < 0) return fail(BSM_ERR_INVALID_ARG, "negative shape");
  if (C % 16 != 0) return fail(BSM_ERR_INVALID_ARG, "C (%lld) must be a multiple of 16", (long long)C);
  if (C == 0) return ok();
  if (!hess_blocks || (N > 0 && !x)) return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(hess_blocks, 8)) return fail(BSM_ERR_INVALID_ARG, "hess_blocks must be 8-byte aligned");
  return hip_status(bsm::launch_local_hessian(x, x_dtype == BSM_BF16, N, C, hess_blocks, (hipStream_t)stream),
                    "bsm_local_hessian_blocks");
}

int bsm_nvfp4_quantize_local_hessian(const void* w, int w_dtype, int64_t R, int64_t C, const double* hess_blocks,
                                     int radius, uint8_t* codes, uint8_t* scales, float* global_scale, void* ws,
                                     size_t ws_bytes, bsm_stream_t stream) {
  if (!dtype_ok(w_dtype)) return fail(BSM_ERR_INVALID_ARG, "w_dtype must be BSM_BF16 or BSM_F32");
  if (R < 0 || C < 0) return fail(BSM_ERR_INVALID_ARG, "negative shape");
  if (C % 16 != 0) return fail(BSM_ERR_INVALID_ARG, "C (%lld) must be a multiple of 16", (long long)C);
  if (radius < 0 || radius > 125) return fail(BSM_ERR_INVALID_ARG, "radius must be in [0, 125]");
  if (R * C == 0) return ok();
  if (!w || !hess_blocks || !codes || !scales || !global_scale) return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(w, 32) || !aligned(codes, 8) || !aligned(hess_blocks, 8))
    return fail(BSM_ERR_INVALID_ARG, "w 32-byte, codes and hess_blocks 8-byte alignment");
  if (int r = check_ws(ws, ws_bytes, bsm::nvfp4_quant_ws(1, R, C))) return r;
  return hip_status(bsm::launch_nvfp4_quantize_lh(w, w_dtype == BSM_BF16, R, C, hess_blocks, radius, codes, scales,
                                                  global_scale, (float*)ws, (hipStream_t)stream),
                    "bsm_nvfp4_quantize_local_hessian");
}

int bsm_nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* global_scale, int64_t B, int64_t R,
                         int64_t C, int out_dtype, void* out, bsm_stream_t stream) {
  if (!dtype_ok(out_dtype)) return fail(BSM_ERR_INVALID_ARG, "out_dtype must be BSM_BF16 or BSM_F32");
  if (B < 0 || R < 0 || C < 0) return fail(BSM_ERR_INVALID_ARG, "negative shape");
  if (C % 16 != 0) return fail(BSM_ERR_INVALID_ARG, "C (%lld) must be a multiple of 16", (long long)C);
  if (B > 65535) return fail(BSM_ERR_UNSUPPORTED, "B (%lld) > 65535", (long long)B);
  if (B * R * C == 0) return ok();
  if (!codes || !scales || !global_scale || !out) return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(codes, 8) || !aligned(out, 16)) return fail(BSM_ERR_INVALID_ARG, "codes 8-byte / out 16-byte alignment");
  return hip_status(bsm::launch_nvfp4_dequantize(codes, scales, global_scale, B, R, C, out_dtype == BSM_BF16, out,
                                                 (hipStream_t)stream),
                    "bsm_nvfp4_dequantize");
}

int bsm_fp8_quantize(const void* x, int x_dtype, int64_t R, int64_t C, uint8_t* codes, float* scales,
                     bsm_stream_t stream) {
  if (!dtype_ok(x_dtype)) return fail(BSM_ERR_INVALID_ARG, "x_dtype must be BSM_BF16 or BSM_F32");
  if (R < 0 || C < 0) return fail(BSM_ERR_INVALID_ARG, "negative shape");
  if (C % 4 != 0) return fail(BSM_ERR_INVALID_ARG, "C (%lld) must be a multiple of 4", (long long)C);
  if (R > 0x7FFFFFFF) return fail(BSM_ERR_UNSUPPORTED, "R too large");
  if (R * C == 0) {
    if (R > 0 && C == 0) return fail(BSM_ERR_INVALID_ARG, "C must be positive");
    return ok();
  }
  if (!x || !codes || !scales) return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(x, 16) || !aligned(codes, 4)) return fail(BSM_ERR_INVALID_ARG, "x 16-byte / codes 4-byte alignment");
  return hip_status(bsm::launch_fp8_quantize(x, x_dtype == BSM_BF16, R, C, codes, scales, (hipStream_t)stream),
                    "bsm_fp8_quantize");
}

size_t bsm_route_workspace_size(int64_t T, int64_t H, int64_t E) {
  if (T < 0 || H <= 0 || E <= 0) return 0;
  return bsm::route_ws(T, H, E);
}

static int route_checks(int64_t T, int64_t H, int64_t E, int n_group, int topk_group, int topk) {
  if (T < 0 || H <= 0 || E <= 0) return fail(BSM_ERR_INVALID_ARG, "T >= 0, H > 0, E > 0 required");
  if (E > 1024) return fail(BSM_ERR_UNSUPPORTED, "E (%lld) > 1024", (long long)E);
  if (n_group < 1 || n_group > 64) return fail(BSM_ERR_INVALID_ARG, "n_group must be in [1, 64]");
  if (E % n_group != 0) return fail(BSM_ERR_INVALID_ARG, "E %% n_group != 0");
  if (E / n_group < 2) return fail(BSM_ERR_INVALID_ARG, "groups need at least 2 experts");
  if (topk_group < 1 || topk_group > n_group) return fail(BSM_ERR_INVALID_ARG, "topk_group must be in [1, n_group]");
  if (topk < 1 || topk > 32) return fail(BSM_ERR_INVALID_ARG, "topk must be in [1, 32]");
  if ((int64_t)topk > (int64_t)topk_group * (E / n_group))
    return fail(BSM_ERR_INVALID_ARG, "topk > topk_group * E / n_group");
  if (T * E > 0x7FFFFFFF) return fail(BSM_ERR_UNSUPPORTED, "T * E too large");
  return BSM_OK;
}

int bsm_route(const void* x, int x_dtype, int64_t T, int64_t H, const void* w_router, int w_dtype, int64_t E,
              int n_group, int topk_group, int topk, int32_t* topk_ids, float* topk_weights, float* scores, void* ws,
              size_t ws_bytes, bsm_stream_t stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(w_dtype)) return fail(BSM_ERR_INVALID_ARG, "dtype must be BSM_BF16 or BSM_F32");
  if (int r = route_checks(T, H, E, n_group, topk_group, topk)) return r;
  if (T == 0) return ok();
  if (!x || !w_router || !topk_ids || !topk_weights) return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  if (int r = check_ws(ws, ws_bytes, bsm::route_ws(T, H, E))) return r;
  return hip_status(bsm::launch_route(x, x_dtype == BSM_BF16, T, H, w_router, w_dtype == BSM_BF16, E, n_group,
                                      topk_group, topk, topk_ids, topk_weights, scores, ws, (hipStream_t)stream),
                    "bsm_route");
}

size_t bsm_route_nvfp4_quantize_workspace_size(int64_t T, int64_t H, int64_t E) {
  if (T < 0 || H <= 0 || E <= 0) return 0;
  return bsm::route_q_ws(T, H, E);
}

int bsm_route_nvfp4_quantize(const void* x, int x_dtype, int64_t T, int64_t H, const void* w_router, int w_dtype,
                             int64_t E, int n_group, int topk_group, int topk, int32_t* topk_ids,
                             float* topk_weights, float* scores, uint8_t* codes, uint8_t* scales,
                             float* global_scale, void* ws, size_t ws_bytes, bsm_stream_t stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(w_dtype)) return fail(BSM_ERR_INVALID_ARG, "dtype must be BSM_BF16 or BSM_F32");
  if (int r = route_checks(T, H, E, n_group, topk_group, topk)) return r;
  if (H % 16 != 0) return fail(BSM_ERR_INVALID_ARG, "H (%lld) must be a multiple of 16", (long long)H);
  if (T == 0) return ok();
  if (!x || !w_router || !topk_ids || !topk_weights || !codes || !scales || !global_scale)
    return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(x, 32) || !aligned(codes, 8)) return fail(BSM_ERR_INVALID_ARG, "x must be 32-byte and codes 8-byte aligned");
  if (int r = check_ws(ws, ws_bytes, bsm::route_q_ws(T, H, E))) return r;
  return hip_status(bsm::launch_route_nvfp4_quantize(x, x_dtype == BSM_BF16, T, H, w_router, w_dtype == BSM_BF16, E,
                                                     n_group, topk_group, topk, topk_ids, topk_weights, scores,
                                                     codes, scales, global_scale, ws, (hipStream_t)stream),
                    "bsm_route_nvfp4_quantize");
}

int bsm_route_diagnostics(const void* ws, int64_t T, int64_t H, int64_t E, int32_t* diag, bsm_stream_t stream) {
  if (T < 0 || H <= 0 || E <= 0) return fail(BSM_ERR_INVALID_ARG, "bad shape");
  if (!ws || !diag) return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  return hip_status(bsm::launch_route_diag(ws, T, H, E, diag, (hipStream_t)stream), "bsm_route_diagnostics");
}

static bool known_format(int f) { return f == BSM_FMT_NVFP4 || f == BSM_FMT_FP8 || f == BSM_FMT_W4A16; }

size_t bsm_moe_workspace_size(int format, int64_t E, int64_t H, int64_t I, int64_t T, int topk) {
  if (!known_format(format) || E <= 0 || H <= 0 || I <= 0 || T < 0 || topk <= 0) return 0;
  return bsm::moe_layout(format != BSM_FMT_FP8, E, H, I, T, topk).total;
}

int bsm_moe_workspace_layout(int format, int64_t E, int64_t H, int64_t I, int64_t T, int topk,
                             bsm_moe_ws_layout* out) {
  if (!known_format(format) || E <= 0 || H <= 0 || I <= 0 || T < 0 || topk <= 0 || !out)
    return fail(BSM_ERR_INVALID_ARG, "bad arguments");
  const bsm::MoeLayout L = bsm::moe_layout(format != BSM_FMT_FP8, E, H, I, T, topk);
  out->total = L.total;
  out->counts = L.counts;
  out->offsets = L.offsets;
  out->row_pair = L.row_pair;
  out->pair_row = L.pair_row;
  out->tiles = L.tiles;
  out->h_f32 = L.h_f32;
  out->h_codes = L.h_codes;
  out->h_scales = L.h_scales;
  out->h_gs = L.h_gs;
  out->y_f32 = L.y_f32;
  out->scratch = L.scratch;
  return ok();
}

int bsm_moe_expert_mlp(const bsm_moe_weights* w, const bsm_act_q* xq, int64_t T, const int32_t* topk_ids,
                       const float* topk_weights, int topk, float combine_scale, int h_gs_mode, float* h_global_scale,
                       float* out, void* ws, size_t ws_bytes, bsm_stream_t stream) {
  bsm::MoeArgs a;
  bool empty = false;
  if (int r = moe_args(w, xq, T, topk_ids, topk_weights, topk, combine_scale, h_gs_mode, h_global_scale, out, &a,
                       &empty))
    return r;
  if (empty) return ok();
  if (int r = check_ws(ws, ws_bytes, bsm::moe_layout(a.nvfp4, a.E, a.H, a.I, T, topk).total)) return r;
  a.ws = (uint8_t*)ws;
  return hip_status(bsm::launch_moe(a, (hipStream_t)stream), "bsm_moe_expert_mlp");
}

int bsm_moe_expert_mlp_noalloc(const bsm_moe_weights* w, const bsm_act_q* xq, int64_t T, const int32_t* topk_ids,
                               const float* topk_weights, int topk, float combine_scale, int h_gs_mode,
                               float* h_global_scale, float* out, bsm_stream_t stream) {
  bsm::MoeArgs a;
  bool empty = false;
  if (int r = moe_args(w, xq, T, topk_ids, topk_weights, topk, combine_scale, h_gs_mode, h_global_scale, out, &a,
                       &empty))
    return r;
  if (empty) return ok();
  const size_t need = bsm::moe_layout(a.nvfp4, a.E, a.H, a.I, T, topk).total;
  if (need > kNoAllocScratchBytes)
    return fail(BSM_ERR_UNSUPPORTED,
                "bsm_moe_expert_mlp_noalloc: this call needs %zu bytes of scratch, the static scratch holds %zu "
                "(use bsm_moe_expert_mlp with a workspace)",
                need, kNoAllocScratchBytes);
  void* sp = nullptr;
  if (int r = noalloc_scratch(&sp)) return r;
  a.ws = (uint8_t*)sp;
  return hip_status(bsm::launch_moe(a, (hipStream_t)stream), "bsm_moe_expert_mlp_noalloc");
}

int bsm_moe_expert_mlp_w4a16(const bsm_moe_weights* w, const void* x, int64_t T, const int32_t* topk_ids,
                             const float* topk_weights, int topk, float combine_scale, float* out, void* ws,
                             size_t ws_bytes, bsm_stream_t stream) {
  if (!w) return fail(BSM_ERR_INVALID_ARG, "NULL weights");
  if (w->format != BSM_FMT_NVFP4) return fail(BSM_ERR_INVALID_ARG, "weight-only path needs NVFP4 weights");
  const int64_t E = w->E, H = w->H, I = w->I;
  if (E <= 0 || H <= 0 || I <= 0 || T < 0) return fail(BSM_ERR_INVALID_ARG, "bad shape");
  if (H % 256 != 0 || I % 128 != 0) return fail(BSM_ERR_UNSUPPORTED, "H must be a multiple of 256 and I of 128");
  if (E > 1024) return fail(BSM_ERR_UNSUPPORTED, "E > 1024");
  if (topk < 1 || topk > 32 || topk > E) return fail(BSM_ERR_INVALID_ARG, "topk must be in [1, min(32, E)]");
  if (T * topk > 0x3FFFFFFF) return fail(BSM_ERR_UNSUPPORTED, "T * topk too large");
  if (int r = check_layout(w, true, true, T, topk)) return r;
  if (T == 0) return ok();
  if (!w->w13_codes || !w->w13_scales || !w->w2_codes || !w->w2_scales || !w->w13_gs || !w->w2_gs || !x ||
      !topk_ids || !topk_weights || !out)
    return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(w->w13_codes, 16) || !aligned(w->w2_codes, 16) || !aligned(x, 16) || !aligned(out, 16))
    return fail(BSM_ERR_INVALID_ARG, "codes, x and out must be 16-byte aligned");
  if (!aligned(w->w13_scales, 2) || !aligned(w->w2_scales, 2))
    return fail(BSM_ERR_INVALID_ARG, "NVFP4 scales must be 2-byte aligned");
  if (int r = check_ws(ws, ws_bytes, bsm::moe_layout(true, E, H, I, T, topk).total)) return r;
  bsm::MoeArgs a;
  a.nvfp4 = true;
  a.a16 = true;
  a.E = E;
  a.H = H;
  a.I = I;
  a.T = T;
  a.topk = topk;
  a.w13_codes = w->w13_codes;
  a.w13_scales = w->w13_scales;
  a.w13_gs = w->w13_gs;
  a.w2_codes = w->w2_codes;
  a.w2_scales = w->w2_scales;
  a.w2_gs = w->w2_gs;
  a.x_codes = reinterpret_cast<const uint8_t*>(x);
  a.x_scales = nullptr;
  a.x_gs = nullptr;
  a.ids = topk_ids;
  a.wts = topk_weights;
  a.combine_scale = combine_scale;
  a.h_static = false;
  a.h_gs_user = nullptr;
  a.out = out;
  a.pairs = w->layout == BSM_LAYOUT_PAIRS;
  a.w13_scales_lanes = w->w13_scales_lanes;
  a.w2_scales_lanes = w->w2_scales_lanes;
  a.ws = reinterpret_cast<uint8_t*>(ws);
  return hip_status(bsm::launch_moe(a, (hipStream_t)stream), "bsm_moe_expert_mlp_w4a16");
}

int bsm_scales_to_lanes(const uint8_t* in, uint8_t* out, int64_t rows, int64_t row_bytes, bsm_stream_t stream) {
  if (rows < 0 || row_bytes < 0 || rows % 16 != 0 || row_bytes % 32 != 0)
    return fail(BSM_ERR_INVALID_ARG, "rows must be a multiple of 16 and row_bytes of 32");
  if (rows == 0 || row_bytes == 0) return ok();
  if (!in || !out) return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(in, 16) || !aligned(out, 16)) return fail(BSM_ERR_INVALID_ARG, "in and out must be 16-byte aligned");
  const uint8_t *ie = in + rows * row_bytes, *oe = out + rows * row_bytes;
  if (in < oe && out < ie) return fail(BSM_ERR_INVALID_ARG, "in and out overlap");
  return hip_status(bsm::launch_scales_to_lanes(in, out, rows, row_bytes, (hipStream_t)stream), "bsm_scales_to_lanes");
}

int bsm_codes_to_pairs(const uint8_t* in, uint8_t* out, int64_t rows, int64_t row_bytes, bsm_stream_t stream) {
  if (rows < 0 || row_bytes < 0 || rows % 16 != 0 || row_bytes % 64 != 0)
    return fail(BSM_ERR_INVALID_ARG, "rows must be a multiple of 16 and row_bytes of 64");
  if (rows == 0 || row_bytes == 0) return ok();
  if (!in || !out) return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(in, 16) || !aligned(out, 16)) return fail(BSM_ERR_INVALID_ARG, "in and out must be 16-byte aligned");
  const uint8_t *ie = in + rows * row_bytes, *oe = out + rows * row_bytes;
  if (in < oe && out < ie) return fail(BSM_ERR_INVALID_ARG, "in and out overlap");
  return hip_status(bsm::launch_codes_to_pairs(in, out, rows, row_bytes, (hipStream_t)stream), "bsm_codes_to_pairs");
}

size_t bsm_fp8_linear_workspace_size(int64_t T, int64_t K, int64_t N) {
  if (T < 0 || K <= 0 || N <= 0) return 0;
  return bsm::fp8_linear_ws(T, K, N);
}

int bsm_fp8_linear(const uint8_t* x_codes, const float* x_scales, const uint8_t* w_codes, const float* w_scales,
                   int64_t T, int64_t K, int64_t N, float* out, void* ws, size_t ws_bytes, bsm_stream_t stream) {
  if (T < 0 || K <= 0 || N <= 0) return fail(BSM_ERR_INVALID_ARG, "bad shape");
  if (K % 128 != 0 || N % 128 != 0) return fail(BSM_ERR_UNSUPPORTED, "K and N must be multiples of 128");
  if (T > 0x3FFFFFFF || K > 0x3FFFFFFF || N > 0x3FFFFFFF) return fail(BSM_ERR_UNSUPPORTED, "shape too large");
  if (T == 0) return ok();
  if (!x_codes || !x_scales || !w_codes || !w_scales || !out) return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(x_codes, 16) || !aligned(w_codes, 16) || !aligned(out, 16))
    return fail(BSM_ERR_INVALID_ARG, "codes and out must be 16-byte aligned");
  if (int r = check_ws(ws, ws_bytes, bsm::fp8_linear_ws(T, K, N))) return r;
  return hip_status(bsm::launch_fp8_linear(x_codes, x_scales, w_codes, w_scales, T, K, N, out,
                                           reinterpret_cast<uint8_t*>(ws), (hipStream_t)stream),
                    "bsm_fp8_linear");
}

int bsm_set_stage_events(int which, void* const* events, int n) {
  if (which != 0 && which != 1) return fail(BSM_ERR_INVALID_ARG, "which must be 0 (moe) or 1 (route)");
  const int need = which == 0 ? 6 : 3;
  if (n != 0 && n != need) return fail(BSM_ERR_INVALID_ARG, "n must be 0 or %d", need);
  if (n && !events) return fail(BSM_ERR_INVALID_ARG, "NULL events");
  bsm::StageEvents& s = bsm::stage_events(which);
  for (int i = 0; i < n; ++i) s.ev[i] = (hipEvent_t)events[i];
  s.n = n;
  return ok();
}

int bsm_ceiling_hbm_read(const void* buf, size_t bytes, uint32_t* sink, int wgs, bsm_stream_t stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || !aligned(buf, 16) || wgs < 1 || wgs > (1 << 20))
    return fail(BSM_ERR_INVALID_ARG, "bsm_ceiling_hbm_read: buf 16-byte aligned, bytes a positive multiple of 16, "
                                     "wgs in [1, 2^20], sink non-NULL");
  return hip_status(bsm::launch_ceil_read(buf, bytes, sink, wgs, (hipStream_t)stream), "bsm_ceiling_hbm_read");
}

int bsm_ceiling_mfma_f16(int shape, int64_t iters, float* sink, int wgs, bsm_stream_t stream) {
  if ((shape != 0 && shape != 1) || iters < 1 || !sink || wgs < 1 || wgs > (1 << 20))
    return fail(BSM_ERR_INVALID_ARG, "bsm_ceiling_mfma_f16: shape 0 or 1, iters >= 1, wgs in [1, 2^20], sink "
                                     "non-NULL");
  return hip_status(bsm::launch_ceil_mfma(shape, iters, sink, wgs, (hipStream_t)stream), "bsm_ceiling_mfma_f16");
}

int bsm_rmsnorm_f32(const float* x, int64_t T, int64_t H, float eps, const float* gamma, float* y,
                    bsm_stream_t stream) {
  if (T < 0 || H <= 0) return fail(BSM_ERR_INVALID_ARG, "bad shape");
  if (!(eps >= 0.0f)) return fail(BSM_ERR_INVALID_ARG, "eps must be >= 0");
  if (T == 0) return ok();
  if (!x || !y) return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  return hip_status(bsm::launch_rmsnorm(x, T, H, eps, gamma, y, (hipStream_t)stream), "bsm_rmsnorm_f32");
}

int bsm_residual_step_weights(int64_t k, float* a, float* b) {
  if (k < 2) return fail(BSM_ERR_INVALID_ARG, "residual step k must be >= 2 (the embedding is step 1)");
  if (!a || !b) return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  *a = (float)sqrt((double)(k - 1) / (double)k);
  *b = (float)(1.0 / sqrt((double)k));
  return ok();
}

int bsm_scaled_residual_f32(float* x, const float* m, float a, float b, int64_t T, int64_t H, bsm_stream_t stream) {
  if (T < 0 || H <= 0) return fail(BSM_ERR_INVALID_ARG, "bad shape");
  if (T == 0) return ok();
  if (!x || !m) return fail(BSM_ERR_INVALID_ARG, "NULL pointer argument");
  return hip_status(bsm::launch_residual(x, m, a, b, T * H, (hipStream_t)stream), "bsm_scaled_residual_f32");
}

}  // extern "C"
