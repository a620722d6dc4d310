"""GPU parity: local Hessian blocks and the Local-Hessian NVFP4 block-scale search (offline quantizer)."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import hessian as LH
from oracle import moe as OM
from oracle import quant as Q
from oracle import route as OR
from tests.helpers import np_, to_dev_bf16

pytestmark = pytest.mark.gpu


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def test_local_hessian_blocks_match_oracle(gpu_lib):
    rng = np.random.default_rng(0)
    x = _bf16(rng.standard_normal((300, 256)) * (1 + 3 * rng.random(256)))
    hb = np_(gpu_lib.local_hessian_blocks(to_dev_bf16(x)))
    ref = LH.local_hessian_blocks(x)
    assert np.allclose(hb, ref, rtol=1e-12, atol=0)


@pytest.mark.parametrize("radius", [0, 3, 8])
def test_local_hessian_quantize_bitexact_small(gpu_lib, radius):
    """Tiny expert gate matrix (128 x 256) with H from the tokens the tiny router sends to it."""
    cfg = W.TINY
    x, wr = W.activations(cfg, T=400), W.router_weights(cfg)
    ids, _, _, _ = OR.route(x, wr, cfg.n_group, cfg.topk_group, cfg.topk)
    e = int(np.bincount(ids.ravel(), minlength=cfg.E).argmax())
    xe = x[(ids == e).any(1)]
    wg = W.expert_weights_host(cfg, e)[0]
    hb = LH.local_hessian_blocks(xe)
    codes, scales, gs = gpu_lib.nvfp4_quantize_local_hessian(to_dev_bf16(wg), torch.from_numpy(hb).cuda(), radius)
    torch.cuda.synchronize()
    oc, os_, og, oerr = LH.nvfp4_quantize_local_hessian(wg, hb, radius)
    assert np_(gs)[0] == og
    assert np.array_equal(np_(scales), os_) and np.array_equal(np_(codes), oc)
    if radius == 0:
        rc, rs, _ = Q.nvfp4_quantize(wg)
        assert np.array_equal(np_(codes), rc) and np.array_equal(np_(scales), rs)
    else:
        changed = (np_(scales) != Q.nvfp4_quantize(wg)[1]).mean()
        print(f"radius {radius}: {changed:.1%} of block scales differ from round-to-nearest")


def test_local_hessian_quantize_beam_expert_sampled_rows(gpu_lib):
    """Beam expert gate projection (2560 x 5120) with H from 256 synthetic tokens; 128 sampled rows checked."""
    cfg = W.DECODE
    x = W.activations(cfg, T=256)
    w13, _ = W.expert_weights_device(cfg, experts=[7])
    wg = w13[0, :cfg.I].contiguous()
    hb_dev = gpu_lib.local_hessian_blocks(to_dev_bf16(x))
    codes, scales, gs = gpu_lib.nvfp4_quantize_local_hessian(wg, hb_dev, 8)
    torch.cuda.synchronize()
    hb = np_(hb_dev)
    assert np.allclose(hb, LH.local_hessian_blocks(x), rtol=1e-12, atol=0)
    wg_h = wg.float().cpu().numpy()
    assert np_(gs)[0] == Q.nvfp4_global_scale(wg_h)
    rows = np.random.default_rng(1).choice(cfg.I, 128, replace=False)
    oc, os_, _, oerr = LH.nvfp4_quantize_local_hessian(wg_h[rows], hb, 8, global_scale=np_(gs)[0])
    assert np.array_equal(np_(scales)[rows], os_) and np.array_equal(np_(codes)[rows], oc)
    # the search lowers the Hessian-weighted error of these rows below round-to-nearest
    rc, rs, rg = Q.nvfp4_quantize(wg_h[rows], global_scale=np_(gs)[0])
    e_rtn = LH.weighted_error(wg_h[rows], rc, rs, rg, hb).sum()
    print(f"Beam expert rows: weighted error {oerr.sum() / e_rtn:.4f} of round-to-nearest")
    assert oerr.sum() < e_rtn
