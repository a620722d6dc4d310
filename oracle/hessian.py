"""NVFP4 block-scale search weighted by the local Hessian (offline weight quantizer).

TEST INFRASTRUCTURE ONLY -- part of the CPU oracle; never used by the product path.

Source: "NVFP4 quantization" page, "Quantization method": post-training
quantization calibrated with a Local Hessian -- each block's scale is the
candidate with the smallest error dW^T H dW, where H comes from the inputs of
the tokens that the router sends to that expert.  "Quantization scheme": E2M1
elements, one E4M3 scale per 16 values, one global scale per tensor.

Readings (the page names the objective, not the search):
* H is the Gram matrix X^T X of the inputs X [N, C] the weight multiplies
  (for gate/up: the tokens routed to the expert; for down: their h).  "Local":
  a block of 16 weights of one row only sees its own 16 input features, so the
  objective of block b is dw^T H_b dw with H_b = H[16b:16b+16, 16b:16b+16];
* the global scale stays the round-to-nearest one, S_g = fl32(amax / 2688);
* candidates: the round-to-nearest block-scale code c0 (as in the RTN
  quantizer) and the E4M3 codes c0 - radius .. c0 + radius (radius 8 = one
  binade either way), restricted to 1..126; a zero block keeps code 0;
* for a candidate scale s the block quantizes exactly as in RTN
  (q = E2M1(fl32(w / fl32(s * S_g)))); dw = w - q * s * S_g in binary64;
* the objective is evaluated in binary64 in a fixed order, each product and
  sum rounded once: t_i = sum_j H_b[i, j] * dw_j (j ascending), then
  e = sum_i dw_i * t_i (i ascending); the smallest e wins, ties go to the lower
  code.  The GPU evaluates the same operations in the same order, so both
  sides reach the same decision.

Parity: pinned in tests by closed forms -- radius 0 reproduces RTN; with
H = I the objective is the squared error and the pick is its brute-force
minimum; every pick is at most the RTN error; the pick is invariant under
scaling H by a power of two.  Local Hessian blocks: against X^T X.
"""

import numpy as np

from .formats import e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode_magnitude
from .quant import NVFP4_BLOCK, _as_f32_exact, nvfp4_global_scale

F32 = np.float32


def local_hessian_blocks(x):
    """x [N, C] -> [C/16, 16, 16] float64 diagonal blocks of x^T x."""
    x64 = np.asarray(x, np.float64)
    N, C = x64.shape
    xb = x64.reshape(N, C // NVFP4_BLOCK, NVFP4_BLOCK)
    return np.einsum("tbi,tbj->bij", xb, xb)


def _objective(dw, hb):
    """dw [..., nb, 16], hb [nb, 16, 16] -> e [..., nb] in the fixed binary64 order."""
    e = np.zeros(dw.shape[:-1])
    for i in range(NVFP4_BLOCK):
        t = np.zeros(dw.shape[:-1])
        for j in range(NVFP4_BLOCK):
            t = t + hb[:, i, j] * dw[..., j]
        e = e + dw[..., i] * t
    return e


def _quantize_block(blk, sb, S_g):
    """RTN element encoding of blocks with given block scales; returns (codes 4-bit, exact decode float64)."""
    d2 = (sb * S_g).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (blk / d2[..., None]).astype(np.float32)
    q = e2m1_encode(r, sign_src=blk)
    q = np.where((sb == 0)[..., None], (np.signbit(blk).astype(np.uint8) << 3), q).astype(np.uint8)
    mag = e2m1_decode(q & 7).astype(np.float64)
    val = np.where(q & 8, -mag, mag) * sb.astype(np.float64)[..., None] * np.float64(S_g)
    return q, val


def nvfp4_quantize_local_hessian(w, hblocks, radius=8, global_scale=None):
    """w [R, C], hblocks [C/16, 16, 16] -> (codes [R, C/2], scales [R, C/16], S_g, objective of the pick).

    ``global_scale``: the tensor's S_g when w holds only some of its rows (rows quantize independently).
    """
    w32 = _as_f32_exact(w)
    R, C = w32.shape
    nb = C // NVFP4_BLOCK
    hb = np.asarray(hblocks, np.float64)
    assert hb.shape == (nb, NVFP4_BLOCK, NVFP4_BLOCK)
    S_g = nvfp4_global_scale(w32) if global_scale is None else F32(global_scale)
    blk = w32.reshape(R, nb, NVFP4_BLOCK)
    a_b = np.max(np.abs(blk), axis=-1)
    d1 = F32(F32(6.0) * S_g)
    with np.errstate(divide="ignore", invalid="ignore"):
        c0 = np.zeros(a_b.shape, np.int64) if S_g == 0 else e4m3_encode_magnitude(a_b / d1).astype(np.int64)
    best_code = c0.copy()
    best_err = np.full(a_b.shape, np.inf)
    blk64 = blk.astype(np.float64)
    for delta in range(-radius, radius + 1):
        c = c0 + delta
        valid = (c0 > 0) & (c >= 1) & (c <= 126)
        sb = e4m3_decode(np.clip(c, 0, 126)).astype(np.float32)
        _, val = _quantize_block(blk, sb, S_g)
        err = _objective(blk64 - val, hb)
        better = valid & (err < best_err)
        best_code = np.where(better, c, best_code)
        best_err = np.where(better, err, best_err)
    sb = e4m3_decode(best_code).astype(np.float32)
    q, _ = _quantize_block(blk, sb, S_g)
    q = q.reshape(R, C)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    best_err = np.where(c0 > 0, best_err, 0.0)
    return codes, best_code.astype(np.uint8), S_g, best_err


def weighted_error(w, codes, scales, S_g, hblocks):
    """Objective dw^T H_b dw of every block of an NVFP4 encoding of w (same fixed order)."""
    from .quant import nvfp4_dequantize_exact
    w64 = _as_f32_exact(w).astype(np.float64)
    R, C = w64.shape
    dw = (w64 - nvfp4_dequantize_exact(codes, scales, S_g)).reshape(R, C // NVFP4_BLOCK, NVFP4_BLOCK)
    return _objective(dw, np.asarray(hblocks, np.float64))
