"""C-ABI library: loads on the host, exports every declared symbol, and rejects bad arguments
before touching the GPU (no kernel is launched by any call in this file)."""

import ctypes
import os
import re

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
    assert lib.bsm_abi_version() == 1
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
    assert lib.bsm_nvfp4_dequantize(FAKE, FAKE, FAKE, 1, 4, 24, FAKE, None) == 1
    assert lib.bsm_nvfp4_dequantize(None, FAKE, FAKE, 1, 4, 32, FAKE, None) == 1


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


def test_norm_validation(lib):
    assert lib.bsm_rmsnorm_f32(FAKE, 4, 0, 1e-6, FAKE, None) == 1
    assert lib.bsm_rmsnorm_f32(FAKE, 4, 16, -1.0, FAKE, None) == 1
    assert lib.bsm_scaled_residual_f32(None, FAKE, 1.0, 1.0, 4, 16, None) == 1
    assert lib.bsm_rmsnorm_f32(None, 0, 16, 1e-6, None, None) == 0


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
