"""C-ABI library: loads on the host, exports every declared symbol, and rejects bad arguments
before touching the GPU (no kernel is launched by any call in this file)."""

import ctypes
import os
import re

import numpy as np
import pytest

import block_scaled_fp4_sigmoid_amd as bsm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return bsm.load()


def _declared():
    src = open(os.path.join(ROOT, "include", "bsmoe.h")).read()
    return sorted(set(re.findall(r"\b(bsm_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_function(lib):
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.bsm_abi_version() == 5
    assert lib.bsm_status_str(0) == b"BSM_OK"
    assert lib.bsm_status_str(3) == b"BSM_ERR_WORKSPACE"


def _err(lib):
    return lib.bsm_last_error().decode()


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails validation


def test_nvfp4_quantize_validation(lib):
    assert lib.bsm_nvfp4_quantize(FAKE, 7, 1, 4, 32, FAKE, FAKE, FAKE, 0, None, 0, None) == 1
    assert lib.bsm_nvfp4_quantize(FAKE, 1, 1, 4, 40, FAKE, FAKE, FAKE, 0, None, 0, None) == 1
    assert "multiple of 16" in _err(lib)
    assert lib.bsm_nvfp4_quantize(None, 1, 1, 4, 32, FAKE, FAKE, FAKE, 0, None, 0, None) == 1
    assert lib.bsm_nvfp4_quantize(FAKE, 1, 1, 4, 32, FAKE, FAKE, FAKE, 5, None, 0, None) == 1
    assert lib.bsm_nvfp4_quantize(FAKE, 1, 1, 4, 32, FAKE, FAKE, FAKE, 0, None, 0, None) == 3
    assert lib.bsm_nvfp4_quantize(FAKE, 1, 1, 4, 32, FAKE, FAKE, FAKE, 0, ctypes.c_void_p(0x100010), 1 << 20,
                                  None) == 3  # misaligned workspace
    assert lib.bsm_nvfp4_quantize(FAKE, 1, 1, 4, 32, FAKE, FAKE, FAKE, 0, FAKE, 16, None) == 3
    # empty tensors are a successful no-op
    assert lib.bsm_nvfp4_quantize(None, 1, 1, 0, 32, None, None, None, 0, None, 0, None) == 0
    assert lib.bsm_nvfp4_quantize_workspace_size(1, 4, 32) >= 256


def test_fp8_and_dequant_validation(lib):
    assert lib.bsm_fp8_quantize(FAKE, 1, 4, 30, FAKE, FAKE, None) == 1
    assert lib.bsm_fp8_quantize(FAKE, 3, 4, 32, FAKE, FAKE, None) == 1
    assert lib.bsm_fp8_quantize(None, 1, 0, 32, None, None, None) == 0
    assert lib.bsm_nvfp4_dequantize(FAKE, FAKE, FAKE, 1, 4, 24, 2, FAKE, None) == 1
    assert lib.bsm_nvfp4_dequantize(None, FAKE, FAKE, 1, 4, 32, 2, FAKE, None) == 1
    assert lib.bsm_nvfp4_dequantize(FAKE, FAKE, FAKE, 1, 4, 32, 7, FAKE, None) == 1  # out_dtype


@pytest.mark.parametrize("E,G,kg,k,code", [
    (256, 8, 4, 8, 3),     # valid shape, missing workspace
    (256, 7, 4, 8, 1),     # E % n_group
    (256, 8, 9, 8, 1),     # topk_group > n_group
    (256, 8, 4, 33, 1),    # topk > 32
    (16, 8, 1, 3, 1),      # topk > topk_group * group size
    (2048, 8, 4, 8, 2),    # E > 1024 unsupported
    (16, 16, 4, 2, 1),     # group size 1
])
def test_route_validation(lib, E, G, kg, k, code):
    r = lib.bsm_route(FAKE, 1, 64, 5120, FAKE, 1, E, G, kg, k, FAKE, FAKE, None, None, 0, None)
    assert r == code, _err(lib)


def test_route_nvfp4_quantize_validation(lib):
    """The routing + quantization call takes both calls' rules, checked before anything is enqueued."""
    f = lib.bsm_route_nvfp4_quantize
    args = lambda T=64, H=5120, x=FAKE, E=256, G=8, codes=FAKE, ws=None, wsb=0: (
        x, 1, T, H, FAKE, 1, E, G, 4, 8, FAKE, FAKE, None, codes, FAKE, FAKE, ws, wsb, None)
    assert f(*args()) == 3  # valid, missing workspace
    assert f(*args(G=7)) == 1  # E % n_group
    assert f(*args(H=5128)) == 1  # H % 16
    assert f(*args(x=ctypes.c_void_p(0x100010))) == 1  # x not 32-byte aligned
    assert f(*args(codes=None)) == 1
    need = lib.bsm_route_nvfp4_quantize_workspace_size(64, 5120, 256)
    assert need >= lib.bsm_route_workspace_size(64, 5120, 256) + lib.bsm_nvfp4_quantize_workspace_size(1, 64, 5120)
    assert f(*args(ws=ctypes.c_void_p(0x200000), wsb=need - 1)) == 3
    assert f(*args(T=0)) == 0


def test_moe_validation(lib):
    w = bsm._MoeWeights(1, 256, 5120, 2560, 0x100000, 0x100000, 0x100000, 0x100000, 0x100000, 0x100000)
    a = bsm._ActQ(1, 0x100000, 0x100000, 0x100000)
    ref = ctypes.byref
    assert lib.bsm_moe_expert_mlp(ref(w), ref(a), 64, FAKE, FAKE, 8, 2.5, 0, None, FAKE, None, 0, None) == 3
    bad = bsm._MoeWeights(1, 256, 5120, 2500, 0x100000, 0x100000, 0x100000, 0x100000, 0x100000, 0x100000)
    assert lib.bsm_moe_expert_mlp(ref(bad), ref(a), 64, FAKE, FAKE, 8, 2.5, 0, None, FAKE, None, 0, None) == 2
    a8 = bsm._ActQ(2, 0x100000, 0x100000, None)
    assert lib.bsm_moe_expert_mlp(ref(w), ref(a8), 64, FAKE, FAKE, 8, 2.5, 0, None, FAKE, None, 0, None) == 1
    assert lib.bsm_moe_expert_mlp(ref(w), ref(a), 64, FAKE, FAKE, 0, 2.5, 0, None, FAKE, None, 0, None) == 1
    assert lib.bsm_moe_expert_mlp(ref(w), ref(a), 64, FAKE, FAKE, 8, 2.5, 1, None, FAKE, None, 0, None) == 1
    assert lib.bsm_moe_expert_mlp(None, ref(a), 64, FAKE, FAKE, 8, 2.5, 0, None, FAKE, None, 0, None) == 1
    assert lib.bsm_moe_expert_mlp(ref(w), ref(a), 0, None, None, 8, 2.5, 0, None, None, None, 0, None) == 0
    lay = bsm._WsLayout()
    assert lib.bsm_moe_workspace_layout(1, 256, 5120, 2560, 64, 8, ctypes.byref(lay)) == 0
    assert lay.total == lib.bsm_moe_workspace_size(1, 256, 5120, 2560, 64, 8)
    assert lay.y_f32 >= lay.h_f32 + 512 * 2560 * 4
    assert all(getattr(lay, f) % 256 == 0 for f, _ in bsm._WsLayout._fields_)


def test_moe_weight_layout_validation(lib):
    """The pair layout of the weight codes is checked on the host: an unknown layout, shapes its kernels do not
    take, and the dense FP8 path are refused before any device call."""
    ref = ctypes.byref
    a = bsm._ActQ(1, 0x100000, 0x100000, 0x100000)
    P = 0x100000
    unknown = bsm._MoeWeights(1, 256, 5120, 2560, P, P, P, P, P, P, 7)
    assert lib.bsm_moe_expert_mlp(ref(unknown), ref(a), 64, FAKE, FAKE, 8, 2.5, 0, None, FAKE, None, 0, None) == 1
    assert "layout" in _err(lib)
    # NVFP4 pairs need H and I multiples of 512 (I = 384: fine for rows, not for pairs)
    odd = bsm._MoeWeights(1, 256, 5120, 384, P, P, P, P, P, P, bsm.LAYOUT_PAIRS)
    assert lib.bsm_moe_expert_mlp(ref(odd), ref(a), 64, FAKE, FAKE, 8, 2.5, 0, None, FAKE, None, 0, None) == 2
    assert "pair layout" in _err(lib)
    rows = bsm._MoeWeights(1, 256, 5120, 384, P, P, P, P, P, P, bsm.LAYOUT_ROWS)
    assert lib.bsm_moe_expert_mlp(ref(rows), ref(a), 64, FAKE, FAKE, 8, 2.5, 0, None, FAKE, None, 0, None) == 3
    # FP8 dense path (one expert, top-1, at most 64 tokens) reads the canonical layout only
    dense = bsm._MoeWeights(2, 1, 5120, 2560, P, P, None, P, P, None, bsm.LAYOUT_PAIRS)
    a8 = bsm._ActQ(2, 0x100000, 0x100000, None)
    assert lib.bsm_moe_expert_mlp(ref(dense), ref(a8), 64, FAKE, FAKE, 1, 1.0, 0, None, FAKE, None, 0, None) == 2
    # W4A16 takes the same rule
    assert lib.bsm_moe_expert_mlp_w4a16(ref(odd), FAKE, 64, FAKE, FAKE, 8, 2.5, FAKE, None, 0, None) == 2
    # NVFP4 pairs need the lane-ordered copies of the block scales, 16-byte aligned (FP8 pairs do not)
    bare = bsm._MoeWeights(1, 256, 5120, 2560, P, P, P, P, P, P, bsm.LAYOUT_PAIRS)
    assert lib.bsm_moe_expert_mlp(ref(bare), ref(a), 64, FAKE, FAKE, 8, 2.5, 0, None, FAKE, None, 0, None) == 1
    assert "lane-ordered" in _err(lib)
    assert lib.bsm_moe_expert_mlp_w4a16(ref(bare), FAKE, 64, FAKE, FAKE, 8, 2.5, FAKE, None, 0, None) == 1
    skew = bsm._MoeWeights(1, 256, 5120, 2560, P, P, P, P, P, P, bsm.LAYOUT_PAIRS, P, P + 8)
    assert lib.bsm_moe_expert_mlp(ref(skew), ref(a), 64, FAKE, FAKE, 8, 2.5, 0, None, FAKE, None, 0, None) == 1
    full = bsm._MoeWeights(1, 256, 5120, 2560, P, P, P, P, P, P, bsm.LAYOUT_PAIRS, P, P)
    assert lib.bsm_moe_expert_mlp(ref(full), ref(a), 64, FAKE, FAKE, 8, 2.5, 0, None, FAKE, None, 0, None) == 3
    fp8 = bsm._MoeWeights(2, 256, 5120, 2560, P, P, None, P, P, None, bsm.LAYOUT_PAIRS)
    assert lib.bsm_moe_expert_mlp(ref(fp8), ref(a8), 64, FAKE, FAKE, 8, 2.5, 0, None, FAKE, None, 0, None) == 3


def test_codes_to_pairs_validation(lib):
    f = lib.bsm_codes_to_pairs
    assert f(FAKE, ctypes.c_void_p(0x200000), 24, 64, None) == 1  # rows % 16
    assert f(FAKE, ctypes.c_void_p(0x200000), 32, 96, None) == 1  # row_bytes % 64
    assert f(None, ctypes.c_void_p(0x200000), 32, 64, None) == 1
    assert f(FAKE, ctypes.c_void_p(0x100010), 32, 64, None) == 1  # out overlaps in
    assert f(FAKE, ctypes.c_void_p(0x200008), 32, 64, None) == 1  # misaligned
    assert f(None, None, 0, 64, None) == 0
    g = lib.bsm_scales_to_lanes
    assert g(FAKE, ctypes.c_void_p(0x200000), 24, 32, None) == 1  # rows % 16
    assert g(FAKE, ctypes.c_void_p(0x200000), 32, 48, None) == 1  # row_bytes % 32
    assert g(None, ctypes.c_void_p(0x200000), 32, 32, None) == 1
    assert g(FAKE, ctypes.c_void_p(0x100010), 32, 32, None) == 1  # out overlaps in
    assert g(None, None, 0, 32, None) == 0


def test_moe_noalloc_validation(lib):
    """The allocation-free MLP validates like the workspace one and refuses calls beyond its static scratch
    (all of these fail before any device call)."""
    w = bsm._MoeWeights(1, 256, 5120, 2560, 0x100000, 0x100000, 0x100000, 0x100000, 0x100000, 0x100000)
    a = bsm._ActQ(1, 0x100000, 0x100000, 0x100000)
    ref = ctypes.byref
    f = lib.bsm_moe_expert_mlp_noalloc
    assert lib.bsm_moe_workspace_size(1, 256, 5120, 2560, 64, 8) <= 32 << 20  # a Beam decode layer fits
    assert f(ref(w), ref(a), 4096, FAKE, FAKE, 8, 2.5, 0, None, FAKE, None) == 2  # 1.2 GB of scratch needed
    assert "static scratch" in _err(lib)
    bad = bsm._MoeWeights(1, 256, 5120, 2500, 0x100000, 0x100000, 0x100000, 0x100000, 0x100000, 0x100000)
    assert f(ref(bad), ref(a), 64, FAKE, FAKE, 8, 2.5, 0, None, FAKE, None) == 2
    assert f(None, ref(a), 64, FAKE, FAKE, 8, 2.5, 0, None, FAKE, None) == 1
    assert f(ref(w), ref(a), 64, FAKE, FAKE, 8, 2.5, 1, None, FAKE, None) == 1  # STATIC without a scale
    assert f(ref(w), ref(a), 64, FAKE, FAKE, 8, 2.5, 0, None, None, None) == 1  # NULL out
    assert f(ref(w), ref(a), 0, None, None, 8, 2.5, 0, None, None, None) == 0   # empty batch


def test_norm_validation(lib):
    assert lib.bsm_rmsnorm_f32(FAKE, 4, 0, 1e-6, None, FAKE, None) == 1
    assert lib.bsm_rmsnorm_f32(FAKE, 4, 16, -1.0, None, FAKE, None) == 1
    assert lib.bsm_scaled_residual_f32(None, FAKE, 1.0, 1.0, 4, 16, None) == 1
    assert lib.bsm_rmsnorm_f32(None, 0, 16, 1e-6, None, None, None) == 0


def test_residual_step_weights_match_the_oracle(lib):
    """The library's residual weights are the oracle's, bit for bit (host computation, no device work)."""
    from oracle import moe as OM

    a, b = ctypes.c_float(), ctypes.c_float()
    for k in range(2, 200):
        assert lib.bsm_residual_step_weights(k, ctypes.byref(a), ctypes.byref(b)) == 0
        ra, rb = OM.residual_weights(k)
        assert np.float32(a.value).view(np.uint32) == ra.view(np.uint32)
        assert np.float32(b.value).view(np.uint32) == rb.view(np.uint32)
    assert lib.bsm_residual_step_weights(1, ctypes.byref(a), ctypes.byref(b)) == 1
    assert lib.bsm_residual_step_weights(3, None, ctypes.byref(b)) == 1


def test_ceiling_validation(lib):
    assert lib.bsm_ceiling_hbm_read(FAKE, 24, FAKE, 8, None) == 1        # bytes % 16
    assert lib.bsm_ceiling_hbm_read(None, 4096, FAKE, 8, None) == 1
    assert lib.bsm_ceiling_mfma_f16(2, 10, FAKE, 8, None) == 1           # shape
    assert lib.bsm_ceiling_mfma_f16(0, 0, FAKE, 8, None) == 1            # iters


def test_weight_only_moe_validation(lib):
    w = bsm._MoeWeights(1, 256, 5120, 2560, 0x100000, 0x100000, 0x100000, 0x100000, 0x100000, 0x100000)
    ref = ctypes.byref
    f = lib.bsm_moe_expert_mlp_w4a16
    assert f(ref(w), FAKE, 64, FAKE, FAKE, 8, 2.5, FAKE, None, 0, None) == 3   # no workspace
    w8 = bsm._MoeWeights(2, 256, 5120, 2560, 0x100000, 0x100000, None, 0x100000, 0x100000, None)
    assert f(ref(w8), FAKE, 64, FAKE, FAKE, 8, 2.5, FAKE, None, 0, None) == 1  # FP8 weights
    bad = bsm._MoeWeights(1, 256, 5120, 2500, 0x100000, 0x100000, 0x100000, 0x100000, 0x100000, 0x100000)
    assert f(ref(bad), FAKE, 64, FAKE, FAKE, 8, 2.5, FAKE, None, 0, None) == 2  # I % 128
    assert f(ref(w), None, 64, FAKE, FAKE, 8, 2.5, FAKE, None, 0, None) == 1     # NULL x
    assert f(ref(w), 0x100008, 64, FAKE, FAKE, 8, 2.5, FAKE, None, 0, None) == 1  # x misaligned
    assert f(ref(w), FAKE, 64, FAKE, FAKE, 33, 2.5, FAKE, None, 0, None) == 1   # topk > 32
    assert f(ref(w), FAKE, 0, None, None, 8, 2.5, None, None, 0, None) == 0     # empty batch
    assert lib.bsm_moe_workspace_size(3, 256, 5120, 2560, 64, 8) == lib.bsm_moe_workspace_size(1, 256, 5120, 2560,
                                                                                             64, 8)
    assert lib.bsm_moe_workspace_size(4, 256, 5120, 2560, 64, 8) == 0


def test_local_hessian_validation(lib):
    f = lib.bsm_nvfp4_quantize_local_hessian
    assert f(FAKE, 1, 64, 250, FAKE, 8, FAKE, FAKE, FAKE, None, 0, None) == 1     # C % 16
    assert f(FAKE, 1, 64, 256, FAKE, -1, FAKE, FAKE, FAKE, None, 0, None) == 1    # radius < 0
    assert f(FAKE, 1, 64, 256, FAKE, 126, FAKE, FAKE, FAKE, None, 0, None) == 1   # radius > 125
    assert f(FAKE, 3, 64, 256, FAKE, 8, FAKE, FAKE, FAKE, None, 0, None) == 1     # dtype
    assert f(FAKE, 1, 64, 256, None, 8, FAKE, FAKE, FAKE, None, 0, None) == 1     # NULL H
    assert f(FAKE, 1, 64, 256, FAKE, 8, FAKE, FAKE, FAKE, None, 0, None) == 3     # no workspace
    assert f(None, 1, 0, 256, None, 8, None, None, None, None, 0, None) == 0      # empty
    h = lib.bsm_local_hessian_blocks
    assert h(FAKE, 1, 100, 250, FAKE, None) == 1
    assert h(FAKE, 1, 100, 256, None, None) == 1
    assert h(FAKE, 1, 100, 256, ctypes.c_void_p(0x100004), None) == 1            # misaligned output
