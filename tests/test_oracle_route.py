"""Pins for the oracle's group-limited sigmoid router.

Rule ("Reflection releases Beam" news page, "Mixture-of-Experts details"):
sigmoid scores, groups ranked by the total of their two highest scores, the
best groups kept, the top-k experts inside them, weights renormalized to one.  Checked
against a pairwise-dominance brute force, the textbook all-groups case, exact
rationals and decimal arithmetic.
"""

import decimal
import heapq
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import route as R
from oracle.formats import round_fraction_to_f32


def _brute_select(s, n_group, topk_group, topk):
    """Selection by counting, for every group/expert, how many others beat it."""
    T, E = s.shape
    gsz = E // n_group
    ids = np.zeros((T, topk), np.int32)
    for t in range(T):
        row = [float(v) for v in s[t]]
        gs = []
        for j in range(n_group):
            vals = sorted(row[j * gsz:(j + 1) * gsz], reverse=True)
            gs.append(float(np.float32(np.float32(vals[0]) + np.float32(vals[1]))))
        kept = [j for j in range(n_group)
                if sum(1 for i in range(n_group) if gs[i] > gs[j] or (gs[i] == gs[j] and i < j)) < topk_group]
        cand = [e for e in range(E) if e // gsz in kept]
        rank = {e: sum(1 for f in cand if row[f] > row[e] or (row[f] == row[e] and f < e)) for e in cand}
        chosen = sorted([e for e in cand if rank[e] < topk], key=lambda e: rank[e])
        ids[t] = chosen
    return ids


@pytest.mark.parametrize("E,G,kg,k", [(16, 4, 2, 2), (16, 4, 2, 4), (32, 8, 4, 8), (12, 3, 1, 3), (8, 2, 2, 8)])
def test_selection_matches_bruteforce_with_ties(E, G, kg, k):
    rng = np.random.default_rng(E * 100 + k)
    T = 200
    # coarse values -> frequent exact ties among experts and among groups
    s = (rng.integers(0, 6, size=(T, E)) / 8.0 + 0.125).astype(np.float32)
    ids, w = R.select_experts(s, G, kg, k)
    assert np.array_equal(ids, _brute_select(s, G, kg, k))
    s2 = rng.random((T, E)).astype(np.float32)
    ids2, _ = R.select_experts(s2, G, kg, k)
    assert np.array_equal(ids2, _brute_select(s2, G, kg, k))


def test_all_groups_kept_is_plain_topk():
    rng = np.random.default_rng(3)
    s = rng.random((100, 64)).astype(np.float32)
    s[:, 5] = s[:, 9]  # ties
    ids, _ = R.select_experts(s, 8, 8, 8)
    for t in range(100):
        ref = heapq.nlargest(8, range(64), key=lambda e: (s[t, e], -e))
        assert list(ids[t]) == ref


def test_group_score_is_sum_of_top_two():
    # group 0 holds the single best expert but a weak runner-up; group 1 has two good ones
    s = np.full((1, 8), 0.1, np.float32)
    s[0, 0] = 0.95
    s[0, 4] = 0.6
    s[0, 5] = 0.6
    ids, _ = R.select_experts(s, 2, 1, 2)
    assert sorted(ids[0]) == [4, 5]
    # sum of two (not of all): group 0 has four moderate experts summing higher
    s = np.array([[0.3, 0.3, 0.3, 0.3, 0.5, 0.2, 0.0, 0.0]], np.float32)
    ids, _ = R.select_experts(s, 2, 1, 1)
    assert list(ids[0]) == [4]


def test_group_tie_goes_to_lower_index():
    s = np.array([[0.5, 0.25, 0.0, 0.0, 0.25, 0.5, 0.0, 0.0]], np.float32)
    ids, _ = R.select_experts(s, 2, 1, 2)
    assert list(ids[0]) == [0, 1]
    s = np.array([[0.5, 0.5, 0.5, 0.5]], np.float32)
    ids, _ = R.select_experts(s, 1, 1, 3)
    assert list(ids[0]) == [0, 1, 2]


def test_normalized_weights():
    rng = np.random.default_rng(5)
    s = rng.random((500, 256)).astype(np.float32)
    ids, w = R.select_experts(s, 8, 4, 8)
    sel = np.take_along_axis(s, ids, 1).astype(np.float64)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) < 8 * 2 ** -23)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=3e-7)
    assert np.all(np.diff(np.take_along_axis(s, ids, 1), axis=1) <= 0)


def test_logits_exact_on_random_and_cancellation():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, 96)).astype(np.float32)
    w = (rng.standard_normal((5, 96)) * 0.05).astype(np.float32)
    l, _ = R.logits_exact_f32(x, w)
    for t in range(8):
        for e in range(5):
            ex = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[t], w[e]))
            assert l[t, e] == round_fraction_to_f32(ex)
    # cancellation that float64 cannot resolve: exact value 2^-40
    x = np.array([[2.0 ** 30, 1.0, -2.0 ** 30]], np.float32)
    w = np.array([[1.0, 2.0 ** -40, 1.0]], np.float32)
    l, nbad = R.logits_exact_f32(x, w)
    assert l[0, 0] == np.float32(2.0 ** -40) and nbad == 1
    # exact midpoint between two float32 values, resolved to even
    x = np.array([[1.0, 2.0 ** -24]], np.float32)
    w = np.array([[1.0, 1.0]], np.float32)
    l, _ = R.logits_exact_f32(x, w)
    assert l[0, 0] == np.float32(1.0)
    x = np.array([[1.0, 2.0 ** -24, 2.0 ** -60]], np.float32)
    w = np.array([[1.0, 1.0, 1.0]], np.float32)
    l, _ = R.logits_exact_f32(x, w)
    assert l[0, 0] == np.nextafter(np.float32(1.0), np.float32(2.0))


def test_sigmoid_exact_against_decimal():
    rng = np.random.default_rng(7)
    l = np.concatenate([rng.standard_normal(3000) * 4, rng.uniform(-110, 30, 3000),
                        [0.0, -0.0, 16.0, 17.0, 17.4, 88.0, -87.0, -103.0, -104.0, -200.0]]).astype(np.float32)
    s, _ = R.sigmoid_exact_f32(l)
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        for li, si in zip(l[::7], s[::7]):
            d = 1 / (1 + (-decimal.Decimal(float(li))).exp())
            q = Fraction(d)
            c = np.float32(si)
            lo = np.nextafter(c, np.float32(-np.inf))
            hi = np.nextafter(c, np.float32(np.inf))
            assert abs(Fraction(float(c)) - q) <= min(abs(Fraction(float(lo)) - q), abs(Fraction(float(hi)) - q))
    assert s[np.where(l == 0)[0][0]] == 0.5
    assert s[np.where(l == np.float32(17.4))[0][0]] == 1.0
    assert s[np.where(l == np.float32(-200.0))[0][0]] == 0.0


def test_route_end_to_end_tiny_matches_bruteforce():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    wr = (rng.standard_normal((16, 256)) * 0.05).astype(np.float32)
    ids, w, s, st = R.route(x, wr, 4, 2, 2)
    assert np.array_equal(ids, _brute_select(s, 4, 2, 2))
    assert ids.dtype == np.int32 and w.dtype == np.float32
