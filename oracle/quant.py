"""NVFP4 and FP8_DYNAMIC quantizers, written from the method's definition.

TEST INFRASTRUCTURE ONLY -- part of the CPU oracle; never used by the product path.

NVFP4 ("NVFP4 quantization" page, "Quantization scheme"): 4-bit E2M1 elements,
one FP8 E4M3 scale per block of 16 values, one more global scale per tensor.
FP8_DYNAMIC ("FP8 quantization" page, "Quantization scheme" and "Quantization
method"): E4M3 elements, one scale per row (output channel for weights, token
for activations); each quotient value / scale becomes the closest E4M3
value.

Readings taken where the pages are silent (each one is a choice, listed with
the others in the design notes):
* global scale S_g = fl32(amax / (6*448)): the decode multiplier that maps the
  largest block scale onto E4M3's largest finite value; S_g = 0 for amax = 0.
* block scale s_b = E4M3(fl32(a_b / fl32(6*S_g))), a_b = max |x| in the block.
* element code q = E2M1(fl32(x / fl32(s_b*S_g))), IEEE single division; a
  block whose scale decodes to 0 gets +-0 codes; the sign bit is the sign of x.
* blocks run along the last (reduction) axis; element 2j goes in the low
  nibble and 2j+1 in the high nibble of byte j.
* FP8 row scale s = fl32(amax_row / 448); a row with amax 0 gets +-0 codes.
All arithmetic on float32 values below is numpy float32 arithmetic, i.e. one
IEEE round-to-nearest-even per operation, in the order written.

Parity: the codecs are pinned (see formats.py); the quantizers are pinned by
invariants that hold for any correct implementation of this reading
(power-of-two scaling, sign symmetry, the block maximum encoding as +-6, error
bounds, brute-force recomputation of single blocks).  The constants 6*448 and
448 themselves are the reading above, not values printed on the pages.
"""

import numpy as np

from . import formats
from .formats import (
    e2m1_decode,
    e2m1_encode,
    e4m3_decode,
    e4m3_encode,
    e4m3_encode_magnitude,
)

F32 = np.float32
NVFP4_BLOCK = 16
NVFP4_GS_DIVISOR = F32(6.0 * 448.0)  # 2688
FP8_MAX = F32(448.0)


def _as_f32_exact(x):
    x = np.asarray(x)
    x32 = x.astype(np.float32)
    if x.dtype != np.float32:
        assert np.array_equal(x32.astype(x.dtype), x, equal_nan=True), "input not float32-exact"
    return x32


def nvfp4_global_scale(x):
    """S_g = fl32(max|x| / 2688) for one tensor (dynamic global scale)."""
    x32 = _as_f32_exact(x)
    amax = F32(np.max(np.abs(x32))) if x32.size else F32(0.0)
    return F32(amax / NVFP4_GS_DIVISOR)


def nvfp4_quantize(x, global_scale=None, row_chunk=4096):
    """Quantize one tensor x[R, C] to NVFP4.

    Returns (codes uint8 [R, C/2], scales uint8 [R, C/16] (E4M3 codes),
    S_g float32).  ``global_scale`` given -> static mode (S_g is that value).
    """
    x32 = _as_f32_exact(x)
    assert x32.ndim == 2 and x32.shape[1] % NVFP4_BLOCK == 0
    R, C = x32.shape
    S_g = nvfp4_global_scale(x32) if global_scale is None else F32(global_scale)
    codes = np.empty((R, C // 2), np.uint8)
    scales = np.empty((R, C // NVFP4_BLOCK), np.uint8)
    d1 = F32(F32(6.0) * S_g)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore", under="ignore"):
        for r0 in range(0, R, row_chunk):
            blk = x32[r0:r0 + row_chunk].reshape(-1, C // NVFP4_BLOCK, NVFP4_BLOCK)
            a_b = np.max(np.abs(blk), axis=-1)
            if S_g == 0:
                sb_code = np.zeros(a_b.shape, np.uint8)
            else:
                sb_code = e4m3_encode_magnitude(a_b / d1)
            sb = e4m3_decode(sb_code).astype(np.float32)
            d2 = sb * S_g
            r = blk / d2[..., None]
            q = e2m1_encode(r, sign_src=blk)
            q = np.where((sb == 0)[..., None], (np.signbit(blk).astype(np.uint8) << 3), q)
            q = q.reshape(blk.shape[0], C).astype(np.uint8)
            codes[r0:r0 + row_chunk] = q[:, 0::2] | (q[:, 1::2] << 4)
            scales[r0:r0 + row_chunk] = sb_code
    return codes, scales, S_g


def unpack_e2m1(codes):
    """[R, C/2] packed bytes -> [R, C] 4-bit codes (low nibble = even element)."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out


def nvfp4_dequantize_exact(codes, scales, S_g):
    """Exact decoded values q * s_b * S_g as float64 (no rounding: <= 30 bits)."""
    q = e2m1_decode(unpack_e2m1(codes))
    sb = e4m3_decode(scales)
    R, C = q.shape
    v = (q.reshape(R, C // NVFP4_BLOCK, NVFP4_BLOCK) * sb[..., None]).reshape(R, C)
    return v * np.float64(S_g)


def nvfp4_dequantize_f32(codes, scales, S_g):
    """Standalone dequantize: fl32(fl32(q*s_b) * S_g); q*s_b is exact in float32."""
    q = e2m1_decode(unpack_e2m1(codes)).astype(np.float32)
    sb = e4m3_decode(scales).astype(np.float32)
    R, C = q.shape
    v = (q.reshape(R, C // NVFP4_BLOCK, NVFP4_BLOCK) * sb[..., None]).reshape(R, C)
    return (v * F32(S_g)).astype(np.float32)


def nvfp4_dequantize_bf16(codes, scales, S_g):
    """Standalone dequantize to BF16: the exact q * s_b * S_g rounded once to BF16 (nearest, ties to even),
    returned as float32 (BF16 values are exact in float32)."""
    return formats.bf16_round_exact(nvfp4_dequantize_exact(codes, scales, S_g)).astype(np.float32)


def fp8_quantize(x):
    """Per-row FP8_DYNAMIC quantization of x[R, C] -> (codes uint8 [R, C], scales f32 [R])."""
    x32 = _as_f32_exact(x)
    assert x32.ndim == 2
    amax = np.max(np.abs(x32), axis=1) if x32.shape[1] else np.zeros(x32.shape[0], np.float32)
    s = (amax / FP8_MAX).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = x32 / s[:, None]
    q = e4m3_encode(r, sign_src=x32)
    q = np.where((s == 0)[:, None], (np.signbit(x32).astype(np.uint8) << 7), q).astype(np.uint8)
    return q, s


def fp8_dequantize_exact(codes, scales):
    """Exact decoded values q * s as float64 (4 + 24 significant bits)."""
    return e4m3_decode(codes) * np.asarray(scales, np.float64)[:, None]
