"""Group-limited sigmoid router, written from the method's definition.

TEST INFRASTRUCTURE ONLY -- part of the CPU oracle; never used by the product path.

Source: "Reflection releases Beam" news page, "Mixture-of-Experts details":
every expert gets a sigmoid score, the experts form 8 groups of 32 each, the 4
groups with the largest sum of their two best scores are kept, the top 8
experts inside the kept groups are selected, and each chosen expert's weight is
its score over the sum of the chosen scores (the x2.5 is applied at the
combine, see moe.py).  "Residual stream and numerical decisions": the router runs in FP32.
The "NVFP4 quantization" page, "Quantization scheme", keeps router input and
weights unquantized.

Readings taken where the pages are silent:
* logits are the exactly rounded FP32 value of the exact dot product x.w
  (an FP32 result independent of summation order);
* scores are the exactly rounded FP32 value of 1/(1+exp(-l));
* group score = fl32(best + second best) of the group;
* ties (groups, experts) go to the lower index; selected ids are ordered by
  (score descending, index ascending);
* normalized weight w_j = fl32(s_j / S), S the float32 running sum of the
  selected scores in output order; no bias or correction term, no epsilon.

Parity: pinned by brute force on tiny inputs (a pairwise-dominance
formulation of the selection), the textbook special case (all groups kept ==
plain top-k), hand-built ties, sum(w) == 1 within float32 rounding, exact
rational recomputation of logits, and decimal-precision recomputation of the
sigmoid.
"""

import decimal
import math
from fractions import Fraction

import numpy as np

from .formats import f32_rounding_certified, round_fraction_to_f32

F32 = np.float32


def logits_exact_f32(x, w):
    """l[t, e] = fl32(sum_i x[t, i] * w[e, i]) with the sum taken exactly.

    Products of float32-exact inputs are exact in float64.  A float64 GEMM
    gives an estimate with |error| <= gamma_K * sum|x||w|; wherever that
    interval cannot decide the float32 rounding, the logit is recomputed as an
    exact rational sum and rounded directly.
    """
    x64 = np.asarray(x, np.float64)
    w64 = np.asarray(w, np.float64)
    K = x64.shape[1]
    S = x64 @ w64.T
    A = np.abs(x64) @ np.abs(w64).T
    u = 2.0 ** -53
    gamma = K * u / (1.0 - K * u)
    err = gamma * A * (1.0 + 2.0 * gamma) * 1.001
    r, ok = f32_rounding_certified(S, err)
    bad = np.argwhere(~ok)
    for t, e in bad:
        # math.fsum returns the exact sum of the (exact) float64 products,
        # correctly rounded to float64; rounding that to float32 is exact
        # unless it lands exactly on a float32 midpoint, which is settled
        # with rationals.
        prods = (x64[t] * w64[e]).tolist()
        f = math.fsum(prods)
        _, cert = f32_rounding_certified(np.array([f]), np.array([0.0]))
        if cert[0]:
            r[t, e] = np.float32(f)
        else:
            # f is exactly a float32 midpoint: the sign of the exact remainder
            # (again an exactly rounded fsum) says which way to round
            rem = math.fsum(prods + [-f])
            r[t, e] = round_fraction_to_f32(Fraction(f) + (0 if rem == 0 else Fraction(rem)))
    return r, int(len(bad))


def _sigmoid_decimal(l):
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        d = decimal.Decimal(float(l))
        return 1 / (1 + (-d).exp())


def sigmoid_exact_f32(l):
    """s = fl32(1 / (1 + exp(-l))) exactly rounded, for float32 logits l."""
    l = np.asarray(l, np.float32)
    l64 = l.astype(np.float64)
    with np.errstate(over="ignore"):
        s64 = 1.0 / (1.0 + np.exp(-l64))
    err = np.abs(s64) * 2.0 ** -44
    r, ok = f32_rounding_certified(s64, err)
    bad = np.argwhere(~ok)
    for idx in bad:
        idx = tuple(idx)
        dv = _sigmoid_decimal(l[idx])
        q = Fraction(dv)
        c = round_fraction_to_f32(q)
        # the 60-digit value is within 1e-55 (relative) of the exact sigmoid;
        # check that no float32 rounding boundary lies inside that interval
        eps = abs(q) * Fraction(1, 10 ** 55)
        cf = Fraction(float(c))
        lo = Fraction(float(np.nextafter(c, np.float32(-np.inf))))
        hi = Fraction(float(np.nextafter(c, np.float32(np.inf))))
        assert (cf + lo) / 2 < q - eps and q + eps < (cf + hi) / 2, "sigmoid rounding undecided"
        r[idx] = c
    return r, int(len(bad))


def select_experts(scores, n_group, topk_group, topk):
    """Group-limited top-k on float32 scores [T, E] -> (ids int32 [T, k], weights f32 [T, k])."""
    s = np.asarray(scores, np.float32)
    T, E = s.shape
    assert E % n_group == 0
    gsz = E // n_group
    assert gsz >= 2 and 1 <= topk_group <= n_group and 1 <= topk <= topk_group * gsz
    grp = s.reshape(T, n_group, gsz)
    top2 = -np.sort(-grp, axis=-1)[..., :2]
    gscore = (top2[..., 0] + top2[..., 1]).astype(np.float32)
    gorder = np.argsort(-gscore, axis=1, kind="stable")
    kept = np.zeros((T, n_group), bool)
    np.put_along_axis(kept, gorder[:, :topk_group], True, axis=1)
    cand = np.repeat(kept, gsz, axis=1)
    masked = np.where(cand, s.astype(np.float64), -np.inf)
    order = np.argsort(-masked, axis=1, kind="stable")
    ids = order[:, :topk].astype(np.int32)
    sel = np.take_along_axis(s, ids, axis=1)
    ssum = sel[:, 0].copy()
    for j in range(1, topk):
        ssum = (ssum + sel[:, j]).astype(np.float32)
    w = (sel / ssum[:, None]).astype(np.float32)
    return ids, w


def route(x, w_router, n_group, topk_group, topk):
    """Full router: exact FP32 logits -> exact FP32 sigmoid -> group-limited top-k.

    Returns (ids int32 [T, k], weights f32 [T, k], scores f32 [T, E], stats).
    """
    l, n_lbad = logits_exact_f32(x, w_router)
    s, n_sbad = sigmoid_exact_f32(l)
    ids, wts = select_experts(s, n_group, topk_group, topk)
    return ids, wts, s, {"logits_refined": n_lbad, "sigmoid_refined": n_sbad, "logits": l}
