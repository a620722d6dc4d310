"""Pins of the Local-Hessian NVFP4 block-scale search against closed forms and brute force."""

import numpy as np

from oracle import formats as F
from oracle import hessian as LH
from oracle import quant as Q


def _bf16(a):
    import torch
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _case(seed, R=24, C=64, N=200):
    rng = np.random.default_rng(seed)
    w = _bf16(rng.standard_normal((R, C)) * 0.02)
    x = _bf16(rng.standard_normal((N, C)) * (1 + 3 * rng.random(C)))  # uneven feature scales
    return w, x


def test_local_blocks_are_the_diagonal_of_the_gram_matrix():
    _, x = _case(0)
    hb = LH.local_hessian_blocks(x)
    g = x.astype(np.float64).T @ x.astype(np.float64)
    for b in range(hb.shape[0]):
        assert np.allclose(hb[b], g[16 * b:16 * b + 16, 16 * b:16 * b + 16], rtol=1e-12, atol=0)


def test_radius_zero_is_round_to_nearest():
    w, x = _case(1)
    codes, scales, sg, _ = LH.nvfp4_quantize_local_hessian(w, LH.local_hessian_blocks(x), radius=0)
    rc, rs, rg = Q.nvfp4_quantize(w)
    assert np.array_equal(codes, rc) and np.array_equal(scales, rs) and sg == rg


def test_identity_hessian_picks_the_squared_error_minimum():
    w, _ = _case(2)
    nb = w.shape[1] // 16
    eye = np.broadcast_to(np.eye(16), (nb, 16, 16)).copy()
    codes, scales, sg, err = LH.nvfp4_quantize_local_hessian(w, eye, radius=8)
    # brute force: every admissible code of every block, plain squared error
    rc, rs, _ = Q.nvfp4_quantize(w)
    blk = w.reshape(w.shape[0], nb, 16).astype(np.float64)
    for r in range(w.shape[0]):
        for b in range(nb):
            c0 = int(rs[r, b])
            errs = {}
            for c in range(max(1, c0 - 8), min(126, c0 + 8) + 1):
                s = F.e4m3_decode(np.array([c])).astype(np.float32)[0]
                q = F.e2m1_encode((blk[r, b].astype(np.float32) / np.float32(s * sg)).astype(np.float32),
                                  sign_src=blk[r, b].astype(np.float32))
                mag = F.e2m1_decode(q & 7)
                val = np.where(q & 8, -mag, mag) * np.float64(s) * np.float64(sg)
                errs[c] = float(np.sum((blk[r, b] - val) ** 2))
            best = min(errs.values())
            assert errs[int(scales[r, b])] <= best * (1 + 1e-12)
            # ties go to the lower code
            assert int(scales[r, b]) == min(c for c, e in errs.items() if e <= best * (1 + 1e-12))


def test_pick_never_worse_than_round_to_nearest_and_scale_invariant():
    w, x = _case(3)
    hb = LH.local_hessian_blocks(x)
    codes, scales, sg, err = LH.nvfp4_quantize_local_hessian(w, hb)
    rc, rs, rg = Q.nvfp4_quantize(w)
    e_rtn = LH.weighted_error(w, rc, rs, rg, hb)
    e_lh = LH.weighted_error(w, codes, scales, sg, hb)
    assert np.array_equal(e_lh, err)
    assert np.all(e_lh <= e_rtn)
    assert e_lh.sum() < e_rtn.sum()  # the search does find better scales on these inputs
    c2, s2, _, _ = LH.nvfp4_quantize_local_hessian(w, hb * 8.0)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_zero_blocks_and_zero_tensor():
    w, x = _case(4)
    w[3, 16:32] = 0.0
    codes, scales, sg, _ = LH.nvfp4_quantize_local_hessian(w, LH.local_hessian_blocks(x))
    assert scales[3, 1] == 0
    z = np.zeros((4, 32), np.float32)
    c, s, g, e = LH.nvfp4_quantize_local_hessian(z, np.ones((2, 16, 16)))
    assert g == 0 and not c.any() and not s.any() and not e.any()
