"""Python binding of the MI355X NVFP4 / FP8_DYNAMIC routed-expert MoE library.

Argument marshalling only: every computation runs in the HIP kernels of
``libbsmoe.so`` (C ABI declared in ``include/bsmoe.h``).  Tensors are torch
CUDA tensors (device memory on the MI355X); work is enqueued on torch's current
stream.  There is no CPU fallback: if the library is missing or no GPU is
visible, calls raise.

Exported names follow the C ABI: ``nvfp4_quantize``, ``nvfp4_dequantize``,
``fp8_quantize``, ``route``, ``moe_expert_mlp`` (plus ``rmsnorm``,
``scaled_residual_``, and the convenience ``quantize_expert_weights`` and
``moe_layer`` built from those calls).
"""

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsmoe.so")

BSM_OK = 0
BSM_BF16, BSM_F32 = 1, 2
FMT_NVFP4, FMT_FP8, FMT_W4A16 = 1, 2, 3
GS_DYNAMIC, GS_STATIC = 0, 1
LAYOUT_ROWS, LAYOUT_PAIRS = 0, 1

_lib = None


class BsmError(RuntimeError):
    pass


class _MoeWeights(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int), ("E", ctypes.c_int64), ("H", ctypes.c_int64), ("I", ctypes.c_int64),
                ("w13_codes", ctypes.c_void_p), ("w13_scales", ctypes.c_void_p), ("w13_gs", ctypes.c_void_p),
                ("w2_codes", ctypes.c_void_p), ("w2_scales", ctypes.c_void_p), ("w2_gs", ctypes.c_void_p),
                ("layout", ctypes.c_int), ("w13_scales_lanes", ctypes.c_void_p), ("w2_scales_lanes", ctypes.c_void_p)]


class _ActQ(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("global_scale", ctypes.c_void_p)]


class _WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("total", "counts", "offsets", "row_pair", "pair_row", "tiles", "h_f32",
                                                "h_codes", "h_scales", "h_gs", "y_f32", "scratch")]


def load():
    """Load ``libbsmoe.so`` (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise BsmError(f"HIP library not built: {LIB_PATH} missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, sz, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
    sig = {
        "bsm_abi_version": (i32, []),
        "bsm_status_str": (ctypes.c_char_p, [i32]),
        "bsm_last_error": (ctypes.c_char_p, []),
        "bsm_nvfp4_quantize_workspace_size": (sz, [i64, i64, i64]),
        "bsm_nvfp4_quantize": (i32, [vp, i32, i64, i64, i64, vp, vp, vp, i32, vp, sz, vp]),
        "bsm_nvfp4_dequantize": (i32, [vp, vp, vp, i64, i64, i64, i32, vp, vp]),
        "bsm_local_hessian_blocks": (i32, [vp, i32, i64, i64, vp, vp]),
        "bsm_nvfp4_quantize_local_hessian": (i32, [vp, i32, i64, i64, vp, i32, vp, vp, vp, vp, sz, vp]),
        "bsm_fp8_quantize": (i32, [vp, i32, i64, i64, vp, vp, vp]),
        "bsm_route_workspace_size": (sz, [i64, i64, i64]),
        "bsm_route": (i32, [vp, i32, i64, i64, vp, i32, i64, i32, i32, i32, vp, vp, vp, vp, sz, vp]),
        "bsm_route_nvfp4_quantize_workspace_size": (sz, [i64, i64, i64]),
        "bsm_route_nvfp4_quantize": (i32, [vp, i32, i64, i64, vp, i32, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                           vp, sz, vp]),
        "bsm_route_diagnostics": (i32, [vp, i64, i64, i64, vp, vp]),
        "bsm_moe_workspace_size": (sz, [i32, i64, i64, i64, i64, i32]),
        "bsm_moe_workspace_layout": (i32, [i32, i64, i64, i64, i64, i32, ctypes.POINTER(_WsLayout)]),
        "bsm_moe_expert_mlp": (i32, [ctypes.POINTER(_MoeWeights), ctypes.POINTER(_ActQ), i64, vp, vp, i32, f32, i32,
                                     vp, vp, vp, sz, vp]),
        "bsm_moe_expert_mlp_noalloc": (i32, [ctypes.POINTER(_MoeWeights), ctypes.POINTER(_ActQ), i64, vp, vp, i32,
                                             f32, i32, vp, vp, vp]),
        "bsm_moe_expert_mlp_w4a16": (i32, [ctypes.POINTER(_MoeWeights), vp, i64, vp, vp, i32, f32, vp, vp, sz, vp]),
        "bsm_codes_to_pairs": (i32, [vp, vp, i64, i64, vp]),
        "bsm_scales_to_lanes": (i32, [vp, vp, i64, i64, vp]),
        "bsm_fp8_linear_workspace_size": (sz, [i64, i64, i64]),
        "bsm_fp8_linear": (i32, [vp, vp, vp, vp, i64, i64, i64, vp, vp, sz, vp]),
        "bsm_set_stage_events": (i32, [i32, ctypes.POINTER(vp), i32]),
        "bsm_rmsnorm_f32": (i32, [vp, i64, i64, f32, vp, vp, vp]),
        "bsm_residual_step_weights": (i32, [i64, ctypes.POINTER(f32), ctypes.POINTER(f32)]),
        "bsm_ceiling_hbm_read": (i32, [vp, sz, vp, i32, vp]),
        "bsm_ceiling_mfma_f16": (i32, [i32, i64, vp, i32, vp]),
        "bsm_scaled_residual_f32": (i32, [vp, vp, f32, f32, i64, i64, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status):
    if status != BSM_OK:
        lib = load()
        raise BsmError(f"{lib.bsm_status_str(status).decode()}: {lib.bsm_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BSM_BF16
    if t.dtype == torch.float32:
        return BSM_F32
    raise BsmError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _dev(t, name):
    if not t.is_cuda:
        raise BsmError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise BsmError(f"{name} must be contiguous")
    return t


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# quantizers
# ---------------------------------------------------------------------------


def nvfp4_quantize(x: torch.Tensor, global_scale: Optional[torch.Tensor] = None):
    """NVFP4 of B tensors x[B, R, C] (or one tensor [R, C]).

    Returns (codes uint8 [..., R, C/2], scales uint8 [..., R, C/16], global_scale f32 [B]).
    ``global_scale`` given (f32 [B] on the device) -> static mode.
    """
    lib = load()
    _dev(x, "x")
    squeeze = x.dim() == 2
    x3 = x.unsqueeze(0) if squeeze else x
    B, R, C = x3.shape
    codes = torch.empty((B, R, C // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((B, R, C // 16), dtype=torch.uint8, device=x.device)
    if global_scale is None:
        gs = torch.empty(B, dtype=torch.float32, device=x.device)
        mode = GS_DYNAMIC
        ws = _ws(lib.bsm_nvfp4_quantize_workspace_size(B, R, C), x.device)
    else:
        gs = _dev(global_scale.reshape(-1).to(torch.float32), "global_scale")
        mode = GS_STATIC
        ws = None
    _check(lib.bsm_nvfp4_quantize(_ptr(x3), _dtype_code(x), B, R, C, _ptr(codes), _ptr(scales), _ptr(gs), mode,
                                  _ptr(ws), 0 if ws is None else ws.numel(), _stream()))
    if squeeze:
        return codes[0], scales[0], gs
    return codes, scales, gs


def nvfp4_quantize_into(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, gs: torch.Tensor,
                        ws: Optional[torch.Tensor] = None):
    """Dynamic NVFP4 of one tensor x [R, C] into caller buffers codes [R, C/2], scales [R, C/16], gs [1];
    ``ws`` (returned) is reused when large enough."""
    lib = load()
    for t, n in ((x, "x"), (codes, "codes"), (scales, "scales"), (gs, "gs")):
        _dev(t, n)
    R, C = x.shape
    if tuple(codes.shape) != (R, C // 2) or tuple(scales.shape) != (R, C // 16) or gs.numel() != 1:
        raise BsmError("codes [R, C/2], scales [R, C/16] and gs [1] buffers required")
    need = lib.bsm_nvfp4_quantize_workspace_size(1, R, C)
    if ws is None or ws.numel() < need:
        ws = _ws(need, x.device)
    _check(lib.bsm_nvfp4_quantize(_ptr(x), _dtype_code(x), 1, R, C, _ptr(codes), _ptr(scales), _ptr(gs), GS_DYNAMIC,
                                  _ptr(ws), ws.numel(), _stream()))
    return ws


def nvfp4_dequantize(codes: torch.Tensor, scales: torch.Tensor, global_scale: torch.Tensor,
                     out_dtype: torch.dtype = torch.float32):
    """Values q * s_b * S_g of NVFP4 tensors, rounded once to ``out_dtype`` (float32 or bfloat16)."""
    lib = load()
    _dev(codes, "codes")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise BsmError("out_dtype must be torch.float32 or torch.bfloat16")
    squeeze = codes.dim() == 2
    c3 = codes.unsqueeze(0) if squeeze else codes
    B, R, C2 = c3.shape
    out = torch.empty((B, R, C2 * 2), dtype=out_dtype, device=codes.device)
    _check(lib.bsm_nvfp4_dequantize(_ptr(c3), _ptr(_dev(scales, "scales")), _ptr(_dev(global_scale, "gs")), B, R,
                                    C2 * 2, _dtype_code(out), _ptr(out), _stream()))
    return out[0] if squeeze else out


def local_hessian_blocks(x: torch.Tensor):
    """x [N, C] -> [C/16, 16, 16] float64 diagonal blocks of x^T x (the local Hessians of a weight's blocks)."""
    lib = load()
    _dev(x, "x")
    N, C = x.shape
    out = torch.empty((C // 16, 16, 16), dtype=torch.float64, device=x.device)
    _check(lib.bsm_local_hessian_blocks(_ptr(x), _dtype_code(x), N, C, _ptr(out), _stream()))
    return out


def nvfp4_quantize_local_hessian(w: torch.Tensor, hess_blocks: torch.Tensor, radius: int = 8):
    """Offline NVFP4 quantization of w [R, C] with the Local-Hessian block-scale search -> (codes, scales, gs[1])."""
    lib = load()
    _dev(w, "w")
    _dev(hess_blocks, "hess_blocks")
    R, C = w.shape
    if hess_blocks.dtype != torch.float64 or tuple(hess_blocks.shape) != (C // 16, 16, 16):
        raise BsmError("hess_blocks must be float64 [C/16, 16, 16]")
    codes = torch.empty((R, C // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((R, C // 16), dtype=torch.uint8, device=w.device)
    gs = torch.empty(1, dtype=torch.float32, device=w.device)
    ws = _ws(lib.bsm_nvfp4_quantize_workspace_size(1, R, C), w.device)
    _check(lib.bsm_nvfp4_quantize_local_hessian(_ptr(w), _dtype_code(w), R, C, _ptr(hess_blocks), int(radius),
                                                _ptr(codes), _ptr(scales), _ptr(gs), _ptr(ws), ws.numel(),
                                                _stream()))
    return codes, scales, gs


def fp8_quantize(x: torch.Tensor):
    """Per-row FP8 E4M3 quantization of x[R, C] -> (codes uint8 [R, C], scales f32 [R])."""
    lib = load()
    _dev(x, "x")
    R, C = x.shape
    codes = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    scales = torch.empty(R, dtype=torch.float32, device=x.device)
    _check(lib.bsm_fp8_quantize(_ptr(x), _dtype_code(x), R, C, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------


def route(x, w_router, n_group, topk_group, topk, return_scores=False, return_workspace=False):
    """Group-limited sigmoid routing -> (ids int32 [T, k], weights f32 [T, k][, scores f32 [T, E]])."""
    lib = load()
    _dev(x, "x")
    _dev(w_router, "w_router")
    T, H = x.shape
    E = w_router.shape[0]
    ids = torch.empty((T, topk), dtype=torch.int32, device=x.device)
    wts = torch.empty((T, topk), dtype=torch.float32, device=x.device)
    scores = torch.empty((T, E), dtype=torch.float32, device=x.device) if return_scores else None
    ws = _ws(lib.bsm_route_workspace_size(T, H, E), x.device)
    _check(lib.bsm_route(_ptr(x), _dtype_code(x), T, H, _ptr(w_router), _dtype_code(w_router), E, n_group, topk_group,
                         topk, _ptr(ids), _ptr(wts), _ptr(scores), _ptr(ws), ws.numel(), _stream()))
    out = [ids, wts]
    if return_scores:
        out.append(scores)
    if return_workspace:
        out.append(ws)
    return tuple(out)


def route_nvfp4_quantize(x, w_router, n_group, topk_group, topk, return_scores=False, ws=None):
    """Routing and NVFP4 quantization of the same x in one call -> (ids, weights, (codes, scales, gs[1])[, scores]);
    the same values as ``route`` and ``nvfp4_quantize``."""
    lib = load()
    _dev(x, "x")
    _dev(w_router, "w_router")
    T, H = x.shape
    E = w_router.shape[0]
    ids = torch.empty((T, topk), dtype=torch.int32, device=x.device)
    wts = torch.empty((T, topk), dtype=torch.float32, device=x.device)
    scores = torch.empty((T, E), dtype=torch.float32, device=x.device) if return_scores else None
    codes = torch.empty((T, H // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((T, H // 16), dtype=torch.uint8, device=x.device)
    gs = torch.empty(1, dtype=torch.float32, device=x.device)
    need = lib.bsm_route_nvfp4_quantize_workspace_size(T, H, E)
    if ws is None or ws.numel() < need:
        ws = _ws(need, x.device)
    _check(lib.bsm_route_nvfp4_quantize(_ptr(x), _dtype_code(x), T, H, _ptr(w_router), _dtype_code(w_router), E,
                                        n_group, topk_group, topk, _ptr(ids), _ptr(wts), _ptr(scores), _ptr(codes),
                                        _ptr(scales), _ptr(gs), _ptr(ws), ws.numel(), _stream()))
    out = [ids, wts, (codes, scales, gs)]
    if return_scores:
        out.append(scores)
    return tuple(out)


def route_diagnostics(ws, T, H, E):
    """[exact-fallback logits, double-double sigmoids, 0, 0] of the last route call using ``ws``."""
    lib = load()
    d = torch.zeros(4, dtype=torch.int32, device=ws.device)
    _check(lib.bsm_route_diagnostics(_ptr(ws), T, H, E, _ptr(d), _stream()))
    return d


# ---------------------------------------------------------------------------
# expert MLP
# ---------------------------------------------------------------------------


@dataclass
class ExpertWeights:
    """Quantized routed-expert weights: codes in the canonical row-major layout (``LAYOUT_ROWS``) or in the
    pair layout (``LAYOUT_PAIRS``, from ``to_pair_layout``); the scales are row-major either way, and NVFP4
    pair-layout weights also carry lane-ordered copies of the block scales (``*_scales_lanes``)."""
    format: int
    E: int
    H: int
    I: int
    w13_codes: torch.Tensor
    w13_scales: torch.Tensor
    w13_gs: Optional[torch.Tensor]
    w2_codes: torch.Tensor
    w2_scales: torch.Tensor
    w2_gs: Optional[torch.Tensor]
    layout: int = LAYOUT_ROWS
    w13_scales_lanes: Optional[torch.Tensor] = None
    w2_scales_lanes: Optional[torch.Tensor] = None

    def _struct(self):
        return _MoeWeights(self.format, self.E, self.H, self.I, self.w13_codes.data_ptr(), self.w13_scales.data_ptr(),
                           None if self.w13_gs is None else self.w13_gs.data_ptr(), self.w2_codes.data_ptr(),
                           self.w2_scales.data_ptr(), None if self.w2_gs is None else self.w2_gs.data_ptr(),
                           self.layout, None if self.w13_scales_lanes is None else self.w13_scales_lanes.data_ptr(),
                           None if self.w2_scales_lanes is None else self.w2_scales_lanes.data_ptr())


def codes_to_pairs(codes: torch.Tensor) -> torch.Tensor:
    """Pair layout of weight codes [..., rows, row_bytes] (uint8; rows a multiple of 16 in total, row_bytes of 64),
    out of place: in every block of 16 rows, rows p and p + 8 share each 128-byte line, 64 bytes each."""
    lib = load()
    _dev(codes, "codes")
    if codes.dtype != torch.uint8:
        raise BsmError("codes must be uint8")
    rb = codes.shape[-1]
    rows = codes.numel() // rb if rb else 0
    out = torch.empty_like(codes)
    _check(lib.bsm_codes_to_pairs(_ptr(codes), _ptr(out), rows, rb, _stream()))
    return out


def scales_to_lanes(scales: torch.Tensor) -> torch.Tensor:
    """Lane order of NVFP4 block scales [..., rows, row_bytes] (uint8; rows a multiple of 16 in total, row_bytes
    of 32), out of place: per 16-row block and 512-value span, each row's 32 bytes reordered for the lanes."""
    lib = load()
    _dev(scales, "scales")
    if scales.dtype != torch.uint8:
        raise BsmError("scales must be uint8")
    rb = scales.shape[-1]
    rows = scales.numel() // rb if rb else 0
    out = torch.empty_like(scales)
    _check(lib.bsm_scales_to_lanes(_ptr(scales), _ptr(out), rows, rb, _stream()))
    return out


def to_pair_layout(w: "ExpertWeights") -> "ExpertWeights":
    """The same weights in the pair layout: both code tensors through codes_to_pairs (new tensors; the scales
    are shared) and, for NVFP4, lane-ordered copies of both block-scale tensors through scales_to_lanes."""
    if w.layout == LAYOUT_PAIRS:
        return w
    nv = w.format == FMT_NVFP4
    return ExpertWeights(w.format, w.E, w.H, w.I, codes_to_pairs(w.w13_codes), w.w13_scales, w.w13_gs,
                         codes_to_pairs(w.w2_codes), w.w2_scales, w.w2_gs, LAYOUT_PAIRS,
                         scales_to_lanes(w.w13_scales) if nv else None, scales_to_lanes(w.w2_scales) if nv else None)


def quantize_expert_weights(w13: torch.Tensor, w2: torch.Tensor, fmt: str) -> ExpertWeights:
    """Offline RTN quantization of bf16 masters W13 [E, 2I, H] (gate rows then up rows) and W2 [E, H, I].

    NVFP4: every expert's gate, up and down is its own tensor with its own global scale.
    FP8: one scale per output channel (row).
    """
    E, I2, H = w13.shape
    I = I2 // 2
    if fmt == "nvfp4":
        c13, s13, g13 = nvfp4_quantize(w13.reshape(2 * E, I, H))
        c2, s2, g2 = nvfp4_quantize(w2)
        return ExpertWeights(FMT_NVFP4, E, H, I, c13.reshape(E, 2 * I, H // 2), s13.reshape(E, 2 * I, H // 16),
                             g13.reshape(E, 2), c2, s2, g2)
    if fmt == "fp8":
        c13, s13 = fp8_quantize(w13.reshape(E * 2 * I, H))
        c2, s2 = fp8_quantize(w2.reshape(E * H, I))
        return ExpertWeights(FMT_FP8, E, H, I, c13.reshape(E, 2 * I, H), s13.reshape(E, 2 * I), None,
                             c2.reshape(E, H, I), s2.reshape(E, H), None)
    raise BsmError(f"unknown format {fmt}")


def quantize_activations(x: torch.Tensor, fmt: str):
    """NVFP4 (codes, scales, gs[1]) or FP8 (codes, scales[T]) of the expert input."""
    if fmt == "nvfp4":
        return nvfp4_quantize(x)
    return fp8_quantize(x)


def moe_workspace_layout(fmt, E, H, I, T, topk):
    lib = load()
    lay = _WsLayout()
    code = {"nvfp4": FMT_NVFP4, "fp8": FMT_FP8, "w4a16": FMT_W4A16}[fmt]
    _check(lib.bsm_moe_workspace_layout(code, E, H, I, T, topk, ctypes.byref(lay)))
    return {n: getattr(lay, n) for n, _ in _WsLayout._fields_}


def _routing_args(ids, wts):
    _dev(ids, "ids")
    _dev(wts, "wts")
    if ids.dtype != torch.int32 or ids.dim() != 2:
        raise BsmError("ids must be int32 [T, topk]")
    if wts.dtype != torch.float32 or tuple(wts.shape) != tuple(ids.shape):
        raise BsmError("wts must be float32 with the shape of ids")
    return ids.shape


def _act_struct(weights, xq, T):
    fmt = weights.format
    H = weights.H
    if fmt == FMT_NVFP4:
        codes, scales, gs = xq
        if tuple(codes.shape) != (T, H // 2) or codes.dtype != torch.uint8:
            raise BsmError(f"NVFP4 activation codes must be uint8 [{T}, {H // 2}]")
        if tuple(scales.shape) != (T, H // 16) or scales.dtype != torch.uint8:
            raise BsmError(f"NVFP4 activation scales must be uint8 [{T}, {H // 16}]")
        if gs.numel() != 1 or gs.dtype != torch.float32:
            raise BsmError("NVFP4 activation global scale must be one float32")
        for t, n in ((codes, "codes"), (scales, "scales"), (gs, "global scale")):
            _dev(t, n)
        return _ActQ(fmt, codes.data_ptr(), scales.data_ptr(), gs.data_ptr())
    codes, scales = xq
    if tuple(codes.shape) != (T, H) or codes.dtype != torch.uint8:
        raise BsmError(f"FP8 activation codes must be uint8 [{T}, {H}]")
    if tuple(scales.shape) != (T,) or scales.dtype != torch.float32:
        raise BsmError(f"FP8 activation scales must be float32 [{T}]")
    _dev(codes, "codes")
    _dev(scales, "scales")
    return _ActQ(fmt, codes.data_ptr(), scales.data_ptr(), None)


def moe_expert_mlp(weights: ExpertWeights, xq, ids, wts, combine_scale=2.5, h_global_scale=None, out=None, ws=None,
                   return_workspace=False):
    """Routed-expert MLP on quantized activations ``xq`` -> out f32 [T, H]."""
    lib = load()
    T, topk = _routing_args(ids, wts)
    act = _act_struct(weights, xq, T)
    fmt = weights.format
    if out is None:
        out = torch.empty((T, weights.H), dtype=torch.float32, device=ids.device)
    need = lib.bsm_moe_workspace_size(fmt, weights.E, weights.H, weights.I, T, topk)
    if ws is None or ws.numel() < need:
        ws = _ws(need, ids.device)
    mode = GS_STATIC if h_global_scale is not None else GS_DYNAMIC
    wstruct = weights._struct()
    _check(lib.bsm_moe_expert_mlp(ctypes.byref(wstruct), ctypes.byref(act), T, _ptr(ids), _ptr(wts), topk,
                                  float(combine_scale), mode, _ptr(h_global_scale), _ptr(out), _ptr(ws), ws.numel(),
                                  _stream()))
    return (out, ws) if return_workspace else out


def moe_expert_mlp_noalloc(weights: ExpertWeights, xq, ids, wts, out: torch.Tensor, combine_scale=2.5,
                           h_global_scale=None):
    """``moe_expert_mlp`` into the caller's ``out`` (f32 [T, H]) without any allocation: the library's static
    per-GPU scratch replaces the workspace (calls on one GPU share it and must not overlap)."""
    lib = load()
    T, topk = _routing_args(ids, wts)
    act = _act_struct(weights, xq, T)
    _dev(out, "out")
    if out.dtype != torch.float32 or tuple(out.shape) != (T, weights.H):
        raise BsmError(f"out must be float32 [{T}, {weights.H}]")
    mode = GS_STATIC if h_global_scale is not None else GS_DYNAMIC
    wstruct = weights._struct()
    _check(lib.bsm_moe_expert_mlp_noalloc(ctypes.byref(wstruct), ctypes.byref(act), T, _ptr(ids), _ptr(wts), topk,
                                          float(combine_scale), mode, _ptr(h_global_scale), _ptr(out), _stream()))
    return out


def moe_expert_mlp_w4a16(weights: ExpertWeights, x, ids, wts, combine_scale=2.5, out=None, ws=None,
                         return_workspace=False):
    """Weight-only routed-expert MLP: NVFP4 ``weights``, BF16 activations ``x`` [T, H] -> out f32 [T, H]."""
    lib = load()
    _dev(x, "x")
    T, topk = _routing_args(ids, wts)
    if x.dtype != torch.bfloat16 or tuple(x.shape) != (T, weights.H):
        raise BsmError(f"the weight-only path takes BF16 activations [{T}, {weights.H}]")
    if weights.format != FMT_NVFP4:
        raise BsmError("the weight-only path takes NVFP4 weights")
    if out is None:
        out = torch.empty((T, weights.H), dtype=torch.float32, device=ids.device)
    need = lib.bsm_moe_workspace_size(FMT_W4A16, weights.E, weights.H, weights.I, T, topk)
    if ws is None or ws.numel() < need:
        ws = _ws(need, ids.device)
    wstruct = weights._struct()
    _check(lib.bsm_moe_expert_mlp_w4a16(ctypes.byref(wstruct), _ptr(x), T, _ptr(ids), _ptr(wts), topk,
                                        float(combine_scale), _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return (out, ws) if return_workspace else out


def fp8_linear(xq, wq, out=None, ws=None):
    """Dense FP8_DYNAMIC linear: xq = fp8_quantize(x [T, K]), wq = fp8_quantize(W [N, K]) -> out f32 [T, N]."""
    lib = load()
    xc, xs = xq
    wc, wsc = wq
    for t, n in ((xc, "x codes"), (xs, "x scales"), (wc, "w codes"), (wsc, "w scales")):
        _dev(t, n)
    T, K = xc.shape
    N = wc.shape[0]
    if wc.shape[1] != K:
        raise BsmError("x and W disagree on K")
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=xc.device)
    need = lib.bsm_fp8_linear_workspace_size(T, K, N)
    if ws is None or ws.numel() < need:
        ws = _ws(need, xc.device)
    _check(lib.bsm_fp8_linear(_ptr(xc), _ptr(xs), _ptr(wc), _ptr(wsc), T, K, N, _ptr(out), _ptr(ws), ws.numel(),
                              _stream()))
    return out


def fp8_dense_mlp(weights: ExpertWeights, x, out=None):
    """Dense FP8 SwiGLU MLP: one-expert weights (E = 1), every token routed to it with weight 1, scale 1."""
    if weights.format != FMT_FP8 or weights.E != 1:
        raise BsmError("dense MLP weights: FP8 with E = 1")
    T = x.shape[0]
    ids = torch.zeros((T, 1), dtype=torch.int32, device=x.device)
    wts = torch.ones((T, 1), dtype=torch.float32, device=x.device)
    return moe_expert_mlp(weights, quantize_activations(x, "fp8"), ids, wts, combine_scale=1.0, out=out)


def moe_layer(x, w_router, weights: ExpertWeights, n_group, topk_group, topk, combine_scale=2.5):
    """Route -> quantize activations (NVFP4: in the same call) -> expert MLP.  Returns (out, ids, wts)."""
    if weights.format == FMT_NVFP4:
        ids, wts, xq = route_nvfp4_quantize(x, w_router, n_group, topk_group, topk)
    else:
        ids, wts = route(x, w_router, n_group, topk_group, topk)
        xq = quantize_activations(x, "fp8")
    out = moe_expert_mlp(weights, xq, ids, wts, combine_scale)
    return out, ids, wts


def set_stage_events(which: int, handles):
    """Record caller-owned hipEvent_t ``handles`` at stage boundaries (see bsmoe.h); None skips one; [] stops."""
    lib = load()
    n = len(handles)
    arr = (ctypes.c_void_p * max(n, 1))(*[ctypes.c_void_p(h) for h in handles])
    _check(lib.bsm_set_stage_events(which, arr if n else None, n))


# ---------------------------------------------------------------------------
# norm / residual
# ---------------------------------------------------------------------------


def residual_step_weights(k: int):
    """(a_k, b_k) of residual step k >= 2, from the library (fl32 of sqrt((k-1)/k) and 1/sqrt(k))."""
    lib = load()
    a, b = ctypes.c_float(), ctypes.c_float()
    _check(lib.bsm_residual_step_weights(int(k), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def moe_stack(x1: torch.Tensor, layers, n_group, topk_group, topk, eps=1e-6, combine_scale=2.5, keep=False):
    """Stack of MoE layers on an FP32 residual stream whose input is residual step 1.

    Layer i (1-based) is residual step k = i + 1:  n = RMSNorm(x);  m = MoE_i(n);
    x <- fl32(a_k * x + b_k * m) with (a_k, b_k) = residual_step_weights(k).  ``layers``: list of
    (w_router, ExpertWeights).  Returns the final stream (and, with keep=True, the
    per-layer (stream input, normed, ids, weights, moe output)).
    """
    x = x1.clone().float().contiguous()
    trace = []
    for i, (wr, weights) in enumerate(layers, start=1):
        n = rmsnorm(x, eps)
        m, ids, wts = moe_layer(n, wr, weights, n_group, topk_group, topk, combine_scale)
        if keep:
            trace.append((x.clone(), n, ids, wts, m))
        a, b = residual_step_weights(i + 1)
        scaled_residual_(x, m, a, b)
    return (x, trace) if keep else x


def rmsnorm(x: torch.Tensor, eps=1e-6, gamma: Optional[torch.Tensor] = None):
    """FP32 RMSNorm of the rows of x, times the gain ``gamma`` [H] if given (else gain 1)."""
    lib = load()
    _dev(x, "x")
    if gamma is not None:
        _dev(gamma, "gamma")
        if gamma.dtype != torch.float32 or tuple(gamma.shape) != (x.shape[1],):
            raise BsmError(f"gamma must be float32 [{x.shape[1]}]")
    y = torch.empty_like(x)
    _check(lib.bsm_rmsnorm_f32(_ptr(x), x.shape[0], x.shape[1], float(eps), _ptr(gamma), _ptr(y), _stream()))
    return y


def scaled_residual_(x: torch.Tensor, m: torch.Tensor, a: float, b: float):
    """x <- fl32(a*x + b*m) in place."""
    lib = load()
    _dev(x, "x")
    _dev(m, "m")
    _check(lib.bsm_scaled_residual_f32(_ptr(x), _ptr(m), float(a), float(b), x.shape[0], x.shape[1], _stream()))
    return x


# ---------------------------------------------------------------------------
# measurement aids
# ---------------------------------------------------------------------------


def ceiling_hbm_read(buf: torch.Tensor, wgs: int, sink: torch.Tensor):
    """Enqueue one streaming read of ``buf`` (see bsm_ceiling_hbm_read); ``sink`` holds wgs * 256 words."""
    lib = load()
    _check(lib.bsm_ceiling_hbm_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), int(wgs), _stream()))


def ceiling_mfma_f16(shape: int, iters: int, wgs: int, sink: torch.Tensor):
    """Enqueue the FP16 MFMA loop (shape 0: 32x32x16, 1: 16x16x32); ``sink`` holds wgs * 256 floats."""
    lib = load()
    _check(lib.bsm_ceiling_mfma_f16(int(shape), int(iters), _ptr(sink), int(wgs), _stream()))
