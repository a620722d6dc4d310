/*
 * bsmoe.h -- C ABI of the MI355X (gfx950) NVFP4 / FP8_DYNAMIC routed-expert
 * MoE path: group-limited sigmoid routing, block-scaled activation
 * quantization, expert-grouped gate/up/down GEMMs with a SwiGLU product, and
 * the normalized-weight combine.
 *
 * Method sources (cited per function below):
 *   [NVFP4]  "NVFP4 quantization" page, section "Quantization scheme":
 *            W4A4; values are held as 4-bit E2M1 codes, every run of 16
 *            values along a row carries its own FP8 E4M3 scale, and the
 *            tensor as a whole one FP32 scale on top; only the
 *            routed experts' gate/up/down projections are quantized, router
 *            input and weights stay unquantized.
 *   [FP8]    "FP8 quantization" page, sections "Quantization scheme" and
 *            "Quantization method": FP8_DYNAMIC (W8A8), E4M3 codes; a weight
 *            row (output channel) has one fixed scale, an activation row
 *            (token) one scale found at run time; each quotient
 *            value / scale becomes the closest E4M3 value (RTN).
 *   [MOE]    "Reflection releases Beam" news page, section
 *            "Mixture-of-Experts details": sigmoid scores over 256 experts,
 *            8 groups of 32, keep the 4 groups with the largest sum of their
 *            two best scores, top 8 experts within them, SwiGLU experts with
 *            intermediate 2560; the chosen experts' outputs are weighted by
 *            their scores renormalized to sum to one, added, and the total
 *            multiplied by 2.5.
 *   [WO]     "Beam-1.0 auf 4x NVIDIA RTX PRO 6000 Blackwell Server Edition"
 *            page, section "NVFP4 auf Blackwell gegen FP8 auf Hopper" (and
 *            the H100 line of the [NVFP4] page's "Hardware compatibility and
 *            serving"): without FP4 arithmetic the NVFP4 experts run
 *            weight-only, FP4 weights with BF16 activations (W4A16).
 *   [NUM]    same page as [MOE], section "Residual stream and numerical decisions":
 *            router, SwiGLU product and norms in FP32; the embedding is
 *            step 1, and step k scales the stream by sqrt((k-1)/k) before
 *            adding the sublayer output scaled by 1/sqrt(k).
 *
 * Conventions (all functions):
 *   - Pointers named x, w*, codes, scales, out, ws ... are DEVICE pointers
 *     owned by the caller; arrays are dense row-major; the library never
 *     allocates or frees and keeps no pointer after a call returns.
 *   - Work is enqueued on `stream` (hipStream_t, 0 = null stream) and is
 *     asynchronous; no function synchronizes the host.
 *   - Scratch memory is a caller-provided (ws, ws_bytes) pair, at least the
 *     size the matching *_workspace_size() returns, 256-byte aligned.  Its
 *     contents need no initialization and are clobbered.
 *   - Return value: BSM_OK or an error code.  Arguments are validated on the
 *     host before anything is enqueued; on error nothing is enqueued and no
 *     output is touched.  bsm_last_error() returns a thread-local message
 *     describing the most recent error of the calling thread.
 *   - Inputs must be finite; non-finite inputs give unspecified output values
 *     (never an out-of-range access).  Results are deterministic: the same
 *     inputs give bit-identical outputs on every run.
 *   - Element dtypes: BSM_BF16 (bfloat16) or BSM_F32 (IEEE binary32).
 *   - E4M3 means OCP FP8 E4M3FN (bias 7, max finite 448, no infinities).
 */
#ifndef BSMOE_H
#define BSMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSM_ABI_VERSION 5

typedef struct ihipStream_t* bsm_stream_t; /* identical to hipStream_t */

enum bsm_status {
  BSM_OK = 0,
  BSM_ERR_INVALID_ARG = 1, /* null pointer, bad shape, bad enum value */
  BSM_ERR_UNSUPPORTED = 2, /* valid request this build does not implement */
  BSM_ERR_WORKSPACE = 3,   /* ws missing, misaligned or too small */
  BSM_ERR_HIP = 4          /* a HIP runtime call failed (message in bsm_last_error) */
};

enum bsm_dtype { BSM_BF16 = 1, BSM_F32 = 2 };
enum bsm_format { BSM_FMT_NVFP4 = 1, BSM_FMT_FP8 = 2, BSM_FMT_W4A16 = 3 /* workspace sizing only */ };
enum bsm_gs_mode { BSM_GS_DYNAMIC = 0, BSM_GS_STATIC = 1 };
/* Order of the expert weight codes in memory (bsm_moe_weights.layout); the codes themselves are the same. */
enum bsm_layout {
  BSM_LAYOUT_ROWS = 0, /* canonical, row-major */
  BSM_LAYOUT_PAIRS = 1 /* codes from bsm_codes_to_pairs (NVFP4: and lane-ordered copies of the block scales) */
};

/* Library version (BSM_ABI_VERSION). */
int bsm_abi_version(void);

/* Static string naming a status code. */
const char* bsm_status_str(int status);

/* Thread-local description of the calling thread's most recent error ("" if none). */
const char* bsm_last_error(void);

/* ------------------------------------------------------------------------
 * NVFP4 quantization [NVFP4]
 *
 * Quantizes B independent tensors x[b] of shape [R, C] (C % 16 == 0, blocks of
 * 16 consecutive values along C) to
 *   codes  uint8 [B, R, C/2]   E2M1 codes, element 2j in the low nibble of byte j
 *   scales uint8 [B, R, C/16]  E4M3 block scales
 *   global_scale float [B]     per-tensor decode multiplier S_g
 * with, per tensor (IEEE binary32 arithmetic, round to nearest even):
 *   S_g = amax / 2688                       (DYNAMIC: written; STATIC: read)
 *   s_b = E4M3(a_b / (6*S_g)), a_b = max |x| over the block  (0 if S_g == 0)
 *   q   = E2M1(x / (s_b*S_g)), sign = sign of x; a zero scale gives +-0 codes
 * E4M3/E2M1 conversions round to nearest, ties to even, saturating at 448/6.
 * Decoded value: q * s_b * S_g.  B = 1 for activations; B = n_experts for one
 * projection of every expert (each expert's gate, up and down get their own
 * S_g).  x: bf16 or f32 per x_dtype.  Workspace: see the size function.
 * ------------------------------------------------------------------------ */
size_t bsm_nvfp4_quantize_workspace_size(int64_t B, int64_t R, int64_t C);
int bsm_nvfp4_quantize(const void* x, int x_dtype, int64_t B, int64_t R, int64_t C,
                       uint8_t* codes, uint8_t* scales, float* global_scale, int gs_mode,
                       void* ws, size_t ws_bytes, bsm_stream_t stream);

/* ------------------------------------------------------------------------
 * Local-Hessian block-scale search (offline weight quantizer) [NVFP4]
 * ("NVFP4 quantization" page, "Quantization method": each block's scale is
 * the candidate with the smallest error dW^T H dW, where H comes from the
 * inputs of the tokens that the router sends to that expert).
 *
 * bsm_local_hessian_blocks: x [N, C] (the inputs the weight multiplies, bf16
 *   or f32) -> hess_blocks double [C/16][16][16], block b = the 16 x 16
 *   diagonal block of x^T x over input features 16b..16b+15 (binary64, tokens
 *   summed in order).
 * bsm_nvfp4_quantize_local_hessian: one tensor w [R, C] -> codes [R, C/2],
 *   scales [R, C/16], global_scale [1] like bsm_nvfp4_quantize (DYNAMIC global
 *   scale), except that each block's E4M3 scale is the code among
 *   c0 - radius .. c0 + radius (c0 = the round-to-nearest code, admissible
 *   codes 1..126; a zero block keeps 0) minimizing dw^T H_b dw with
 *   dw = w - q * s * S_g, evaluated in binary64 as t_i = sum_j H_ij dw_j
 *   (j ascending), e = sum_i dw_i t_i (i ascending); ties go to the lower
 *   code.  radius 0 is round-to-nearest.  w 32-byte, codes and hess_blocks
 *   8-byte aligned.  Workspace: bsm_nvfp4_quantize_workspace_size(1, R, C).
 * ------------------------------------------------------------------------ */
int bsm_local_hessian_blocks(const void* x, int x_dtype, int64_t N, int64_t C, double* hess_blocks,
                             bsm_stream_t stream);
int bsm_nvfp4_quantize_local_hessian(const void* w, int w_dtype, int64_t R, int64_t C, const double* hess_blocks,
                                     int radius, uint8_t* codes, uint8_t* scales, float* global_scale, void* ws,
                                     size_t ws_bytes, bsm_stream_t stream);

/* Dequantize [NVFP4]: out[b,r,c] = the exact value q * s_b * S_g[b] rounded once to out_dtype
 * (nearest, ties to even): BSM_F32 gives fl32(fl32(q*s_b) * S_g) (q*s_b is exact in binary32),
 * BSM_BF16 rounds the exact product (at most 30 significant bits) straight to BF16.
 * codes [B,R,C/2], scales [B,R,C/16], global_scale [B] float, out [B,R,C] of out_dtype;
 * C % 16 == 0; codes 8-byte and out 16-byte aligned. */
int bsm_nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                         int64_t B, int64_t R, int64_t C, int out_dtype, void* out, bsm_stream_t stream);

/* ------------------------------------------------------------------------
 * FP8_DYNAMIC quantization, one scale per row [FP8]
 *
 * x [R, C] -> codes uint8 [R, C] (E4M3), scales float [R]:
 *   s = amax_row / 448 ; q = E4M3(x / s) (nearest, ties to even, saturating)
 * A row with amax == 0 gets s = 0 and +-0 codes.  Rows are tokens for
 * activations and output channels for weights.  Decoded value q * s.
 * ------------------------------------------------------------------------ */
int bsm_fp8_quantize(const void* x, int x_dtype, int64_t R, int64_t C, uint8_t* codes, float* scales,
                     bsm_stream_t stream);

/* ------------------------------------------------------------------------
 * Group-limited sigmoid router [MOE], FP32 [NUM], unquantized [NVFP4]
 *
 * x [T, H] (bf16 or f32), w_router [E, H] (bf16 or f32).  Per token:
 *   l_e = exactly rounded binary32 value of the exact dot product x . w_e
 *   s_e = exactly rounded binary32 value of 1 / (1 + exp(-l_e))
 *   group score g_j = s(1) + s(2) (binary32 add of the group's two best)
 *   keep the topk_group groups with the largest g (ties: lower group index)
 *   select the topk experts with the largest s inside kept groups (ties: lower
 *   expert index); topk_ids [T, topk] int32 ordered by (s desc, id asc)
 *   topk_weights [T, topk] = s_j / S, S = binary32 running sum of the
 *   selected s in output order (the combine scale is applied later).
 * scores [T, E] (float) receives s when non-NULL.
 * Requirements: E % n_group == 0, E/n_group >= 2, 1 <= topk_group <= n_group,
 * 1 <= topk <= min(32, topk_group * E/n_group), E <= 1024, n_group <= 64.
 * ------------------------------------------------------------------------ */
size_t bsm_route_workspace_size(int64_t T, int64_t H, int64_t E);
int bsm_route(const void* x, int x_dtype, int64_t T, int64_t H, const void* w_router, int w_dtype, int64_t E,
              int n_group, int topk_group, int topk, int32_t* topk_ids, float* topk_weights, float* scores,
              void* ws, size_t ws_bytes, bsm_stream_t stream);

/* Routing and NVFP4 quantization of the same activations in one call [MOE] [NVFP4]: the outputs of
 * bsm_route(x, ..., topk_ids, topk_weights, scores) and of
 * bsm_nvfp4_quantize(x, x_dtype, 1, T, H, codes, scales, global_scale, BSM_GS_DYNAMIC), bit for bit (the
 * router's definition above; the quantization's in "NVFP4 quantization" page, "Quantization scheme").
 * Where the router takes its int8 path for small batches (bf16 x and w_router, E = 256), its pass over x
 * also yields max|x| (NaN excluded, as the quantization takes it) and its selection kernel quantizes each
 * token's row while it selects, so the quantization launches nothing of its own.  Arguments and requirements: those of both calls (x 32-byte aligned, H % 16 == 0, codes [T, H/2]
 * 8-byte aligned, scales [T, H/16], global_scale one float); ws of
 * bsm_route_nvfp4_quantize_workspace_size bytes, 256-byte aligned.  Enqueued on stream; T == 0 does nothing. */
size_t bsm_route_nvfp4_quantize_workspace_size(int64_t T, int64_t H, int64_t E);
int bsm_route_nvfp4_quantize(const void* x, int x_dtype, int64_t T, int64_t H, const void* w_router, int w_dtype,
                             int64_t E, int n_group, int topk_group, int topk, int32_t* topk_ids,
                             float* topk_weights, float* scores, uint8_t* codes, uint8_t* scales,
                             float* global_scale, void* ws, size_t ws_bytes, bsm_stream_t stream);

/* Route diagnostics read back from the workspace of the last bsm_route call
 * enqueued with it: number of logits and scores that needed the exact
 * fallback evaluation.  Copies 4 int32 from device ws to `diag` (device
 * pointer) on `stream`. */
int bsm_route_diagnostics(const void* ws, int64_t T, int64_t H, int64_t E, int32_t* diag, bsm_stream_t stream);

/* ------------------------------------------------------------------------
 * Routed-expert MLP [MOE] [NVFP4] [FP8] [NUM]
 *
 * Weights (canonical layout, consumed directly):
 *   NVFP4: w13_codes uint8 [E, 2I, H/2], w13_scales uint8 [E, 2I, H/16],
 *          w13_gs float [E, 2] (gate, up);  rows 0..I-1 gate, I..2I-1 up.
 *          w2_codes uint8 [E, H, I/2], w2_scales uint8 [E, H, I/16], w2_gs float [E].
 *   FP8:   w13_codes uint8 [E, 2I, H], w13_scales float [E, 2I];
 *          w2_codes uint8 [E, H, I],   w2_scales float [E, H]; *_gs unused (NULL).
 * Activations xq: NVFP4 codes [T, H/2] + scales [T, H/16] + global_scale
 *   (device float*), or FP8 codes [T, H] + scales float [T].
 * For every pair (t, j), e = topk_ids[t, j]:
 *   g, u = binary32-accumulated products of the decoded x[t] with gate/up of e
 *   h    = silu(g) * u in binary32
 *   h is re-quantized (NVFP4: one global scale over all T*topk rows, DYNAMIC
 *   or STATIC via h_gs_mode / h_global_scale; FP8: one scale per row)
 *   y    = decoded h times down of e
 *   out[t] = combine_scale * sum_j topk_weights[t, j] * y(t, j)   (float [T, H])
 * Requirements: H % 256 == 0, I % 128 == 0,
 * topk <= 32, ids in [0, E) and distinct within a token (a pair whose id lies
 * outside [0, E) is dropped: it gets no row and adds nothing to out, so no
 * out-of-range access follows from it; the pair_row of a dropped pair reads -1;
 * repeated ids within a token give unspecified values).  h_global_scale: NVFP4 STATIC -> read; DYNAMIC ->
 * written when non-NULL.  The layout of the workspace (stage buffers) is
 * reported by bsm_moe_workspace_layout for inspection.
 * ------------------------------------------------------------------------ */
typedef struct bsm_moe_weights {
  int format;
  int64_t E, H, I;
  const uint8_t* w13_codes;
  const void* w13_scales;
  const float* w13_gs;
  const uint8_t* w2_codes;
  const void* w2_scales;
  const float* w2_gs;
  int layout; /* BSM_LAYOUT_ROWS, or BSM_LAYOUT_PAIRS for w13_codes and w2_codes from bsm_codes_to_pairs
                 (the scales above stay as they are).  PAIRS needs H and I multiples of the few-row GEMM's
                 K step (NVFP4 and W4A16: 512 values, FP8: 256) and I a multiple of 256, and is not taken
                 by the dense FP8 path (E = 1, topk = 1, T <= 64): BSM_ERR_UNSUPPORTED otherwise. */
  /* NVFP4 with BSM_LAYOUT_PAIRS only (else ignored): w13_scales and w2_scales through bsm_scales_to_lanes,
     same shapes, 16-byte aligned, read by the GEMM of experts with few rows (the one of experts with many
     rows reads the row-major scales); NULL or misaligned -> BSM_ERR_INVALID_ARG. */
  const uint8_t* w13_scales_lanes;
  const uint8_t* w2_scales_lanes;
} bsm_moe_weights;

typedef struct bsm_act_q {
  int format;
  const uint8_t* codes;
  const void* scales;
  const float* global_scale;
} bsm_act_q;

/* Byte offsets of the stage buffers inside the expert-MLP workspace. */
typedef struct bsm_moe_ws_layout {
  size_t total;
  size_t counts;      /* int32 [E]        pairs per expert                                  */
  size_t offsets;     /* int32 [E+1]      first row of each expert (rows sorted by (e, t, j)) */
  size_t row_pair;    /* int32 [P]        pair index t*topk+j of each sorted row             */
  size_t pair_row;    /* int32 [P]        sorted row of each pair                            */
  size_t tiles;       /* int32 [..]       row-tile work list                                 */
  size_t h_f32;       /* float [P, I]     h of each sorted row                               */
  size_t h_codes;     /* uint8 [P, I/2] (NVFP4) or [P, I] (FP8)                              */
  size_t h_scales;    /* uint8 [P, I/16] (NVFP4) or float [P] (FP8)                          */
  size_t h_gs;        /* float [1]        NVFP4 global scale of h                            */
  size_t y_f32;       /* float [P, H]     down-projection output of each sorted row          */
  size_t scratch;     /* internal                                                            */
} bsm_moe_ws_layout;

size_t bsm_moe_workspace_size(int format, int64_t E, int64_t H, int64_t I, int64_t T, int topk);
int bsm_moe_workspace_layout(int format, int64_t E, int64_t H, int64_t I, int64_t T, int topk,
                             bsm_moe_ws_layout* layout /* host pointer */);
int bsm_moe_expert_mlp(const bsm_moe_weights* w /* host */, const bsm_act_q* xq /* host */, int64_t T,
                       const int32_t* topk_ids, const float* topk_weights, int topk, float combine_scale,
                       int h_gs_mode, float* h_global_scale, float* out, void* ws, size_t ws_bytes,
                       bsm_stream_t stream);

/* ------------------------------------------------------------------------
 * Routed-expert MLP without allocation or workspace argument
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, semantics, validation and results (bit-identical) as
 * bsm_moe_expert_mlp, minus the workspace: the call uses a static device
 * array of BSM_NOALLOC_SCRATCH_BYTES (32 MiB) that every GPU the library
 * runs on holds until the process ends (a Beam decode layer of 64 tokens
 * needs about 19.4 MiB in either format).  A call whose
 * bsm_moe_workspace_size exceeds it returns BSM_ERR_UNSUPPORTED and enqueues
 * nothing.  The call allocates nothing (no hipMalloc, no library allocation);
 * the first call on a device looks up that device's copy of the array with
 * the device current.  Every call on one GPU shares its scratch, which keeps
 * the last call's contents (whatever must start at zero is cleared on the
 * stream by the call's own kernels): calls that overlap on one GPU (on
 * different streams, or from several threads without ordering) race.
 * ------------------------------------------------------------------------ */
#define BSM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int bsm_moe_expert_mlp_noalloc(const bsm_moe_weights* w /* host */, const bsm_act_q* xq /* host */, int64_t T,
                               const int32_t* topk_ids, const float* topk_weights, int topk, float combine_scale,
                               int h_gs_mode, float* h_global_scale, float* out, bsm_stream_t stream);

/* ------------------------------------------------------------------------
 * Weight-only W4A16 routed-expert MLP [WO] [MOE] [NUM]
 *
 * w: NVFP4 weights in the canonical layout above (format BSM_FMT_NVFP4).
 * x: BF16 [T, H] (device), the layer input itself; no activation
 * quantization.  For every pair (t, j), e = topk_ids[t, j]:
 *   g, u = binary32-accumulated products of x[t] with the exactly decoded
 *          gate / up rows (q * s_b * S_g; q * s_b is exact in BF16)
 *   h    = silu(g) * u in binary32, rounded to BF16 (nearest, ties to even)
 *   y    = binary32-accumulated products of h with the decoded down rows
 *   out[t] = combine_scale * sum_j topk_weights[t, j] * y(t, j)  (float [T, H])
 * Requirements as bsm_moe_expert_mlp (H % 256 == 0, I % 128 == 0, topk <= 32,
 * ids in [0, E) and distinct within a token); x 16-byte aligned.  Workspace:
 * bsm_moe_workspace_size(BSM_FMT_W4A16, ...); its layout
 * (bsm_moe_workspace_layout with BSM_FMT_W4A16) has h_f32 as above, h_codes
 * and h_scales unused.
 * ------------------------------------------------------------------------ */
int bsm_moe_expert_mlp_w4a16(const bsm_moe_weights* w /* host */, const void* x, int64_t T,
                             const int32_t* topk_ids, const float* topk_weights, int topk, float combine_scale,
                             float* out, void* ws, size_t ws_bytes, bsm_stream_t stream);

/* Pair layout of routed-expert weight codes (BSM_LAYOUT_PAIRS), out of place.  The codes are those of the
 * canonical layout (NVFP4: E2M1 pairs per byte; FP8: E4M3 bytes; "NVFP4 quantization" and "FP8
 * quantization" pages, "Quantization scheme"); only their order changes: in every block of 16 rows, rows
 * p and p + 8 (p < 8) become one double row of 2 * row_bytes bytes whose 128-byte lines hold 64 bytes of
 * row p, then the same 64 bytes of row p + 8.  The few-row expert GEMM then loads each lane's operand
 * pieces directly while every load instruction still reads whole cache lines.
 * in, out: device pointers to [rows, row_bytes] bytes (w13_codes: rows = E * 2I; w2_codes: rows = E * H),
 * 16-byte aligned, not overlapping; rows % 16 == 0, row_bytes % 64 == 0 (BSM_ERR_INVALID_ARG otherwise).
 * Enqueued on stream; the caller owns both buffers. */
int bsm_codes_to_pairs(const uint8_t* in, uint8_t* out, int64_t rows, int64_t row_bytes, bsm_stream_t stream);

/* Lane order of NVFP4 block scales (the E4M3 scale of each block of 16 values, "NVFP4 quantization" page,
 * "Quantization scheme"), out of place, for the *_scales_lanes copies of BSM_LAYOUT_PAIRS weights: the same
 * bytes, reordered.  Row r's
 * 32 scale bytes of each span of 512 values (super-step st) go to 16-row block r / 16, super-step st,
 * row r % 16 (32 bytes each, so a block's super-step is 512 contiguous bytes), block b of the span to
 * byte ((b >> 1) & 3) * 8 + (b >> 3) * 2 + (b & 1): each lane of the few-row GEMM finds its 8 scale bytes
 * of a super-step together, and each 128-byte line holds 4 rows' bytes of one super-step only.
 * in, out: device pointers to [rows, row_bytes] bytes (w13_scales: rows = E * 2I, row_bytes = H / 16;
 * w2_scales: rows = E * H, row_bytes = I / 16), 16-byte aligned, not overlapping; rows % 16 == 0,
 * row_bytes % 32 == 0 (BSM_ERR_INVALID_ARG otherwise).  Enqueued on stream; the caller owns both. */
int bsm_scales_to_lanes(const uint8_t* in, uint8_t* out, int64_t rows, int64_t row_bytes, bsm_stream_t stream);

/* ------------------------------------------------------------------------
 * Dense FP8_DYNAMIC (W8A8) linear projection [FP8]
 *
 * In the FP8 checkpoint the projections of attention (q, k, v, o and the
 * head gate) and of the dense MLPs are FP8 as well ([FP8] "Quantization
 * scheme").
 *   x_codes uint8 [T, K] E4M3, x_scales float [T]   (bsm_fp8_quantize of x)
 *   w_codes uint8 [N, K] E4M3, w_scales float [N]   (bsm_fp8_quantize of W)
 *   out[t, n] = x_scales[t] * w_scales[n] * sum_k q_x[t,k] q_w[n,k]
 *               (binary32 accumulation of exactly decoded operands), float [T, N]
 * Requirements: K % 128 == 0, N % 128 == 0; codes and out 16-byte aligned.
 * Workspace: bsm_fp8_linear_workspace_size(T, K, N) bytes.  A dense FP8
 * SwiGLU MLP is bsm_moe_expert_mlp with one expert (E = 1), every token's id
 * 0 with weight 1 (topk = 1) and combine_scale 1.
 * ------------------------------------------------------------------------ */
size_t bsm_fp8_linear_workspace_size(int64_t T, int64_t K, int64_t N);
int bsm_fp8_linear(const uint8_t* x_codes, const float* x_scales, const uint8_t* w_codes, const float* w_scales,
                   int64_t T, int64_t K, int64_t N, float* out, void* ws, size_t ws_bytes, bsm_stream_t stream);

/* ------------------------------------------------------------------------
 * Profiling aid (not part of the method): stage-boundary events.
 *
 * After bsm_set_stage_events(which, events, n) with n > 0, every later call
 * made by the calling thread records events[i] (hipEvent_t handles created and
 * owned by the caller) on the call's stream at its stage boundaries, so the
 * caller can time individual kernels with hipEventElapsedTime:
 *   which = 0, bsm_moe_expert_mlp / _w4a16 (n = 6): [0] start, [1] after
 *     the permutation, [2] after the gate/up GEMM + SwiGLU, [3] after the h
 *     quantization (W4A16: BF16 rounding), [4] after the down GEMM, [5]
 *     after the combine;
 *   which = 1, bsm_route (n = 3): [0] start, [1] after the logits kernel
 *     (row statistics, dot products, rounding proofs), [2] after the exact
 *     fallback of unproven logits, sigmoid and selection.
 * A NULL entry skips its boundary (each recorded event costs GPU time).
 * n = 0 (events may be NULL) stops recording.  The library keeps the handle
 * values, not the events; they must stay valid while recording is on.
 * ------------------------------------------------------------------------ */
int bsm_set_stage_events(int which, void* const* events, int n);

/* ------------------------------------------------------------------------
 * Measurement aids (not part of the method): this GPU's achievable ceilings.
 *
 * bsm_ceiling_hbm_read: reads bytes (a multiple of 16, buf 16-byte aligned)
 *   of buf once, non-temporal 16-byte loads in 4 KB pieces per workgroup
 *   (each load instruction covers 8 whole 128-byte lines), with wgs
 *   workgroups of 256 threads; writes one word per thread to sink (wgs * 256
 *   uint32).  Bytes / time = the streaming read ceiling.
 * bsm_ceiling_mfma_f16: wgs workgroups of 4 waves, each wave running iters
 *   rounds of 8 independent FP16 MFMAs with FP32 accumulation on register
 *   operands (shape 0: 32x32x16, 32768 flop each; shape 1: 16x16x32, 16384
 *   flop each); writes one float per thread to sink (wgs * 256 floats).
 * Both validate their arguments (BSM_ERR_INVALID_ARG) and enqueue on stream.
 * ------------------------------------------------------------------------ */
int bsm_ceiling_hbm_read(const void* buf, size_t bytes, uint32_t* sink, int wgs, bsm_stream_t stream);
int bsm_ceiling_mfma_f16(int shape, int64_t iters, float* sink, int wgs, bsm_stream_t stream);

/* ------------------------------------------------------------------------
 * FP32 RMSNorm and depth-scaled residual [NUM]
 *
 * bsm_rmsnorm_f32: y[t] = fl32(fl32(x[t] * r) * gamma), r = fl32(1/sqrt(fl32(mean(x[t]^2)) + eps)),
 *   mean and root in float64; gamma: device float [H], or NULL for gain 1 (the reading taken for the
 *   synthetic stack: y = fl32(x[t] * r)).
 * bsm_scaled_residual_f32: x <- fl32(a*x + b*m) in place (float64 evaluation).
 * bsm_residual_step_weights: the weights of residual step k >= 2 (the embedding is step 1, MoE layer i
 *   of a stack is step i + 1): *a = fl32(sqrt((k-1)/k)), *b = fl32(1/sqrt(k)), square roots in
 *   float64; a and b are host pointers; no device work.
 * ------------------------------------------------------------------------ */
int bsm_rmsnorm_f32(const float* x, int64_t T, int64_t H, float eps, const float* gamma, float* y,
                    bsm_stream_t stream);
int bsm_residual_step_weights(int64_t k, float* a /* host */, float* b /* host */);
int bsm_scaled_residual_f32(float* x, const float* m, float a, float b, int64_t T, int64_t H,
                            bsm_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BSMOE_H */
