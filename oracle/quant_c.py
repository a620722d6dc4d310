"""The oracle's quantizers through their C transcription (``quant_c.c``), for full-size tensors.

TEST INFRASTRUCTURE ONLY -- part of the CPU oracle; never used by the product path.

Same functions, arguments and results as ``oracle.quant`` (whose NumPy code is
the readable definition); the C loops make a 39.3 M-weight Beam expert a matter
of milliseconds instead of seconds.  Inputs are float32 arrays, or bf16 values
given as their uint16 bit patterns (exact in float32).  Pinned bit-exactly
against ``oracle.quant`` in ``tests/test_oracle_quant_c.py``.
"""

import ctypes
import os

import numpy as np

from .build_c import LIB, build

_lib = None


def load():
    """The C library; built with gcc on first use when it is missing (``python -m oracle.build_c``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        lib.orq_nvfp4_quantize.argtypes = [vp, i32, i64, i64, i32, f32, vp, vp, vp]
        lib.orq_nvfp4_dequantize.argtypes = [vp, vp, f32, i64, i64, vp]
        lib.orq_fp8_quantize.argtypes = [vp, i32, i64, i64, vp, vp]
        lib.orq_fp8_dequantize.argtypes = [vp, vp, i64, i64, vp]
        for f in (lib.orq_nvfp4_quantize, lib.orq_nvfp4_dequantize, lib.orq_fp8_quantize, lib.orq_fp8_dequantize):
            f.restype = None
        _lib = lib
    return _lib


def _input(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, 1
    if x.dtype != np.float32:
        x32 = x.astype(np.float32)
        assert np.array_equal(x32.astype(x.dtype), x), "input not float32-exact"
        x = np.ascontiguousarray(x32)
    return x, 0


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def nvfp4_quantize(x, global_scale=None):
    """x[R, C] -> (codes uint8 [R, C/2], scales uint8 [R, C/16], S_g float32); static if global_scale given."""
    x, bf = _input(x)
    assert x.ndim == 2 and x.shape[1] % 16 == 0
    R, C = x.shape
    codes = np.empty((R, C // 2), np.uint8)
    scales = np.empty((R, C // 16), np.uint8)
    gs = np.zeros(1, np.float32)
    st = global_scale is not None
    load().orq_nvfp4_quantize(_p(x), bf, R, C, int(st), float(np.float32(global_scale)) if st else 0.0,
                              _p(codes), _p(scales), _p(gs))
    return codes, scales, np.float32(gs[0])


def nvfp4_dequantize_exact(codes, scales, S_g):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    R, C = codes.shape[0], codes.shape[1] * 2
    out = np.empty((R, C), np.float64)
    load().orq_nvfp4_dequantize(_p(codes), _p(scales), float(np.float32(S_g)), R, C, _p(out))
    return out


def fp8_quantize(x):
    """Per-row FP8_DYNAMIC quantization of x[R, C] -> (codes uint8 [R, C], scales f32 [R])."""
    x, bf = _input(x)
    assert x.ndim == 2
    R, C = x.shape
    codes = np.empty((R, C), np.uint8)
    scales = np.empty(R, np.float32)
    load().orq_fp8_quantize(_p(x), bf, R, C, _p(codes), _p(scales))
    return codes, scales


def fp8_dequantize_exact(codes, scales):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.float32)
    R, C = codes.shape
    out = np.empty((R, C), np.float64)
    load().orq_fp8_dequantize(_p(codes), _p(scales), R, C, _p(out))
    return out
