"""GPU parity: dense FP8_DYNAMIC linear projections and the dense FP8 SwiGLU MLP."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import linear as OL
from oracle import quant_c as QC
from tests.fullsize import bf16_bits
from tests.helpers import np_, rel_l2, to_dev_bf16, weights_match

pytestmark = pytest.mark.gpu

TOL = 1e-5  # FP32 accumulation of exactly decoded E4M3 products (about sqrt(K) * 2^-24 per element)

# Beam attention projections: hidden 5120, 8 KV heads and 48 query heads of 128 dimensions, a per-channel head gate
SHAPES = {"q": (5120, 6144), "kv": (5120, 1024), "o": (6144, 5120), "gate": (5120, 6144)}


def _bf16(rng, shape, std):
    return torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("proj,T", [("q", 64), ("kv", 64), ("o", 64), ("gate", 1), ("kv", 37), ("kv", 300)])
def test_fp8_linear_projection(gpu_lib, proj, T):
    K, N = SHAPES[proj]
    rng = np.random.default_rng(hash((proj, T)) % 2 ** 32)
    x = _bf16(rng, (T, K), 1.0)
    w = _bf16(rng, (N, K), 0.02)
    xq = gpu_lib.fp8_quantize(to_dev_bf16(x))
    wq = gpu_lib.fp8_quantize(to_dev_bf16(w))
    out = gpu_lib.fp8_linear(xq, wq)
    torch.cuda.synchronize()
    oxq, owq, y = OL.fp8_linear(x, w)
    assert np.array_equal(np_(xq[0]), oxq[0]) and np.array_equal(np_(xq[1]), oxq[1])
    assert np.array_equal(np_(wq[0]), owq[0]) and np.array_equal(np_(wq[1]), owq[1])
    err = rel_l2(np_(out), y)
    print(f"fp8 linear {proj} T={T} K={K} N={N}: rel L2 {err:.3e}")
    assert err <= TOL


def test_fp8_linear_rejects_bad_shapes(gpu_lib):
    x = torch.zeros((4, 200), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((128, 200), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu_lib.BsmError):
        gpu_lib.fp8_linear(gpu_lib.fp8_quantize(x), gpu_lib.fp8_quantize(w))


@pytest.mark.parametrize("T", [64, 300])
def test_fp8_dense_mlp_reduced_shape(gpu_lib, T):
    """Dense MLP at a reduced shape (hidden 512, intermediate 1024), every token checked."""
    H, I = 512, 1024
    rng = np.random.default_rng(T)
    x = _bf16(rng, (T, H), 1.0)
    wg, wu, wd = _bf16(rng, (I, H), 0.02), _bf16(rng, (I, H), 0.02), _bf16(rng, (H, I), 0.02)
    w13 = to_dev_bf16(np.concatenate([wg, wu])[None])
    w2 = to_dev_bf16(wd[None])
    gw = gpu_lib.quantize_expert_weights(w13, w2, "fp8")
    out = gpu_lib.fp8_dense_mlp(gw, to_dev_bf16(x))
    torch.cuda.synchronize()
    ref = OL.fp8_dense_mlp(x, wg, wu, wd)
    err = rel_l2(np_(out), ref["out"])
    print(f"fp8 dense MLP T={T}: end-to-end rel L2 {err:.3e}")
    assert err <= 1e-3


@pytest.mark.slow
def test_fp8_dense_mlp_full_shape(gpu_lib):
    """Beam dense MLP shape (hidden 5120, intermediate 20480, 64 tokens): every token and stage.

    The oracle quantizes the same bf16 masters itself (its codes and scales must equal the GPU's) and runs
    the whole MLP; h of every token within 1e-5, the oracle's quantizer on the GPU's h reproduces its codes,
    output within 1e-3."""
    H, I, T = 5120, 20480, 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20480)
    w13 = (torch.randn((1, 2 * I, H), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    w2 = (torch.randn((1, H, I), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    x = W.activations(W.DECODE)
    gw = gpu_lib.quantize_expert_weights(w13, w2, "fp8")
    ids = torch.zeros((T, 1), dtype=torch.int32, device="cuda")
    wts = torch.ones((T, 1), dtype=torch.float32, device="cuda")
    xq = gpu_lib.quantize_activations(to_dev_bf16(x), "fp8")
    out, ws = gpu_lib.moe_expert_mlp(gw, xq, ids, wts, combine_scale=1.0, return_workspace=True)
    torch.cuda.synchronize()
    lay = gpu_lib.moe_workspace_layout("fp8", 1, H, I, T, 1)
    h_gpu = np_(ws[lay["h_f32"]:lay["h_f32"] + T * I * 4].view(torch.float32).reshape(T, I))
    hc_gpu = np_(ws[lay["h_codes"]:lay["h_codes"] + T * I].reshape(T, I))
    ref = OL.fp8_dense_mlp(x, bf16_bits(w13[0, :I]), bf16_bits(w13[0, I:]), bf16_bits(w2[0]), q=QC)
    weights_match(gw, {0: ref["expert"]}, "fp8", [0])
    assert np.array_equal(np_(xq[0]), ref["xq"][0]) and np.array_equal(np_(xq[1]), ref["xq"][1])
    h_err = rel_l2(h_gpu, ref["h"])
    assert h_err <= TOL
    assert np.array_equal(hc_gpu, QC.fp8_quantize(h_gpu)[0])
    err = rel_l2(np_(out), ref["out"])
    print(f"fp8 dense MLP full shape: h rel L2 {h_err:.3e}, end-to-end rel L2 {err:.3e}")
    assert err <= 1e-3
