"""Pins for the oracle's router (CPU only).

Ground truth used here is independent of the oracle's own code path:
  * brute force: the selected set is the K-subset of allowed experts with the largest
    key sum, the lexicographically smallest one among equal sums (lower index wins a
    tie); group limit likewise over M-subsets of groups, with each group's score taken
    as the best pair sum inside the group. Subset sums are correctly rounded (fsum), so
    subsets holding the same key values compare equal whatever the summation order;
  * scipy.special.softmax / expit as library routines for the weights;
  * a pure-Python triple loop for the router product on tiny shapes.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special as sps
from hypothesis import given, settings, strategies as st

import oracle
from oracle import route


def brute_select(key, K, n_groups=1, topk_groups=1):
    E = key.shape[0]
    gsz = E // n_groups
    allowed = list(range(E))
    if n_groups > 1 and topk_groups < n_groups:
        def gscore(g):
            members = range(g * gsz, (g + 1) * gsz)
            if gsz == 1:
                return key[g * gsz]
            return max(key[i] + key[j] for i, j in itertools.combinations(members, 2))
        scores = [gscore(g) for g in range(n_groups)]
        best = None
        for gs in itertools.combinations(range(n_groups), topk_groups):
            s = math.fsum(scores[g] for g in gs)
            if best is None or s > best[0]:
                best = (s, gs)
        allowed = [e for g in best[1] for e in range(g * gsz, (g + 1) * gsz)]
    best = None
    for S in itertools.combinations(sorted(allowed), K):
        s = math.fsum(key[e] for e in S)
        if best is None or s > best[0]:
            best = (s, S)
    return np.array(best[1])


@st.composite
def small_case(draw):
    n_groups = draw(st.sampled_from([1, 2, 4]))
    gsz = draw(st.integers(1, 4))
    E = n_groups * gsz
    topk_groups = draw(st.integers(1, n_groups))
    K = draw(st.integers(1, min(4, topk_groups * gsz)))
    T = draw(st.integers(1, 6))
    # small integer logits force exact ties often
    L = draw(st.lists(st.integers(-3, 3), min_size=T * E, max_size=T * E))
    return np.array(L, float).reshape(T, E), K, n_groups, topk_groups


@settings(max_examples=300, deadline=None)
@given(small_case())
def test_topk_matches_brute_force_softmax(case):
    L, K, G, M = case
    rr = route(K=K, score="softmax", n_groups=G, topk_groups=M, logits=L)
    for t in range(L.shape[0]):
        np.testing.assert_array_equal(rr.ids[t], brute_select(L[t], K, G, M))


@settings(max_examples=200, deadline=None)
@given(small_case(), st.lists(st.integers(-2, 2), min_size=16, max_size=16))
def test_topk_matches_brute_force_sigmoid_bias(case, braw):
    L, K, G, M = case
    E = L.shape[1]
    bias = np.array(braw[:E], float) * 0.25
    rr = route(K=K, score="sigmoid", n_groups=G, topk_groups=M, logits=L, bias=bias)
    key = sps.expit(L) + bias[None, :]
    # the oracle's keys are the library sigmoid plus bias (to rounding) ...
    np.testing.assert_allclose(rr.keys, key, rtol=0, atol=1e-15)
    # ... and its selection is the brute-force one on those same keys (exact ties, such
    # as sigmoid(2) + sigmoid(-2) against 1/2 + 1/2, hinge on the last bit of each key)
    for t in range(L.shape[0]):
        np.testing.assert_array_equal(rr.ids[t], brute_select(rr.keys[t], K, G, M))


def test_tie_goes_to_lower_index():
    L = np.zeros((1, 6))
    rr = route(K=3, score="softmax", logits=L)
    np.testing.assert_array_equal(rr.ids[0], [0, 1, 2])
    rr = route(K=2, score="softmax", n_groups=3, topk_groups=1, logits=L)
    np.testing.assert_array_equal(rr.ids[0], [0, 1])


def test_group_score_is_top2_sum_not_max():
    # group 0: keys (5, 0) -> top-2 sum 5, max 5; group 1: keys (4, 4) -> sum 8, max 4.
    L = np.array([[5.0, 0.0, 4.0, 4.0]])
    rr = route(K=1, score="softmax", n_groups=2, topk_groups=1, logits=L)
    np.testing.assert_array_equal(rr.ids[0], [2])   # group 1 wins, its best expert is 2


def test_softmax_weights_library():
    rng = np.random.default_rng(0)
    L = rng.normal(size=(20, 10))
    rr = route(K=3, score="softmax", logits=L)
    for t in range(20):
        sel = rr.ids[t]
        np.testing.assert_allclose(rr.weights[t], sps.softmax(L[t, sel]), rtol=1e-13)
    np.testing.assert_allclose(rr.weights.sum(1), 1.0, rtol=1e-13)
    nr = route(K=3, score="softmax", renorm=False, logits=L)
    for t in range(20):
        np.testing.assert_allclose(nr.weights[t], sps.softmax(L[t])[nr.ids[t]], rtol=1e-13)


def test_softmax_bias_enters_logits():
    rng = np.random.default_rng(1)
    L = rng.normal(size=(10, 8))
    b = rng.normal(size=8)
    rr = route(K=2, score="softmax", logits=L, bias=b)
    for t in range(10):
        sel = rr.ids[t]
        np.testing.assert_array_equal(sel, brute_select(L[t] + b, 2))
        np.testing.assert_allclose(rr.weights[t], sps.softmax((L[t] + b)[sel]), rtol=1e-13)


def test_sigmoid_weights_exclude_bias():
    rng = np.random.default_rng(2)
    L = rng.normal(size=(10, 16))
    b = rng.normal(size=16)
    rr = route(K=4, score="sigmoid", n_groups=4, topk_groups=2, logits=L, bias=b)
    for t in range(10):
        s = sps.expit(L[t, rr.ids[t]])
        np.testing.assert_allclose(rr.weights[t], s / s.sum(), rtol=1e-13)
    nr = route(K=4, score="sigmoid", renorm=False, n_groups=4, topk_groups=2, logits=L, bias=b)
    np.testing.assert_allclose(nr.weights, sps.expit(np.take_along_axis(L, nr.ids.astype(int), 1)),
                               rtol=1e-13)


def test_k_equals_e_selects_all():
    L = np.random.default_rng(3).normal(size=(4, 5))
    rr = route(K=5, score="softmax", logits=L)
    assert (rr.ids == np.arange(5)).all()
    np.testing.assert_allclose(rr.weights, sps.softmax(L, axis=1), rtol=1e-13)


def test_ids_ascending_and_distinct():
    L = np.random.default_rng(4).normal(size=(50, 64))
    rr = route(K=6, score="softmax", logits=L)
    assert (np.diff(rr.ids, axis=1) > 0).all()


def test_router_logits_triple_loop():
    rng = np.random.default_rng(5)
    x = rng.normal(size=(3, 4))
    W = rng.normal(size=(5, 4))          # [E, h]
    L = oracle.router_logits(x, W)
    for t in range(3):
        for e in range(5):
            s = 0.0
            for i in range(4):
                s += x[t, i] * W[e, i]
            assert abs(L[t, e] - s) < 1e-12


def test_gaps():
    L = np.array([[3.0, 1.0, 2.0, 2.5]])
    rr = route(K=2, score="softmax", logits=L)
    assert rr.kth_gap[0] == pytest.approx(0.5)
    rr = route(K=1, score="softmax", n_groups=2, topk_groups=1, logits=L)
    # group scores: (3 + 1) = 4 and (2 + 2.5) = 4.5
    assert rr.group_gap[0] == pytest.approx(0.5)
    np.testing.assert_array_equal(rr.ids[0], [3])


def test_planted_tie_break_mistake_is_caught(monkeypatch):
    """A plausible oracle bug (ties to the higher index) must fail the brute-force pin."""
    import sys
    R = sys.modules["oracle.route"]

    def bad_order(vals):
        idx = np.arange(vals.shape[0])
        return np.lexsort((-idx, -vals))
    monkeypatch.setattr(R, "_order_desc", bad_order)
    L = np.zeros((1, 4))
    rr = R.route(K=2, score="softmax", logits=L)
    assert not np.array_equal(rr.ids[0], brute_select(L[0], 2))
