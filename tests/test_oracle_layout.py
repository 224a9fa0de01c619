"""Pins of oracle/layout.py: closed forms, special cases, consistency with the pair
counts of dispatch, and an exactly known busiest-chip distribution."""
from fractions import Fraction

import numpy as np

import oracle
from oracle import layout as LY


def _uniform_ids(T, E, K, seed):
    keys = np.random.default_rng(seed).random((T, E))
    return oracle.route(K=K, logits=keys).ids


def test_mean_token_fanout_matches_closed_form():
    # uniform routing at the pages' EP=64 example shape: a token reaches about 7.67 chips
    T, E, N, K = 4096, 256, 64, 8
    ids = _uniform_ids(T, E, K, 1)
    st = LY.layout_stats(ids, np.ones_like(ids, bool), E, N)
    f = np.repeat(np.arange(K + 1), st.fanout_hist)
    exp = float(LY.expected_token_fanout(E, N, K))
    # the same expectation as a product of per-draw miss probabilities
    miss = 1.0
    for i in range(K):
        miss *= (E - E // N - i) / (E - i)
    assert abs(exp - N * (1 - miss)) < 1e-12 and 7.6 < exp < 7.7
    assert abs(f.mean() - exp) < 4 * f.std() / np.sqrt(T)
    assert st.fanout_hist.sum() == T and f.max() <= K


def test_one_chip_and_one_expert_per_chip():
    T, E, K = 64, 16, 3
    ids = _uniform_ids(T, E, K, 2)
    kept = np.ones_like(ids, bool)
    one = LY.layout_stats(ids, kept, E, 1)
    assert one.tokens_to.tolist() == [[T]] and one.fanout_hist[1] == T
    assert one.recv_pairs.tolist() == [T * K]
    per = LY.layout_stats(ids, kept, E, E)           # every expert its own chip
    assert per.fanout_hist[K] == T                    # K distinct experts, K chips
    assert (per.recv_pairs == np.bincount(ids.reshape(-1), minlength=E)).all()
    assert per.tokens_to.sum() == T * K


def test_consistent_with_dispatch_pair_counts():
    # capacity drops included: tokens_to <= n_ij <= K tokens_to, column sums = loads
    T, E, N, K, h = 256, 32, 8, 4, 16
    keys = np.random.default_rng(3).random((T, E))
    keys[:, :4] += 0.8                                # hot experts, so the cap bites
    ids = oracle.route(K=K, logits=keys).ids
    d = oracle.dispatch(ids, E=E, n_ep=N, ep_rank=0, capacity_factor=1.0, pad=False, h=h,
                        dtype_size=2)
    assert d.n_dropped > 0
    st = LY.layout_stats(ids, d.kept, E, N)
    n = d.send_bytes // (h * 2)
    assert (st.tokens_to <= n).all() and (n <= K * st.tokens_to).all()
    assert (st.recv_pairs == n.sum(axis=0)).all()
    assert st.recv_pairs.sum() == T * K - d.n_dropped
    assert st.tokens_to.sum() == (np.arange(K + 1) * st.fanout_hist).sum()
    assert ((st.tokens_to > 0) == (n > 0)).all()


def test_node_limited_routing_bounds_node_fanout():
    # 16 chips of 4 experts in 4 nodes; one routing group per node, top-2 nodes
    T, E, N, K, G, M = 512, 64, 16, 6, 4, 2
    keys = np.random.default_rng(4).random((T, E))
    lim = oracle.route(K=K, logits=keys, n_groups=G, topk_groups=M).ids
    free = oracle.route(K=K, logits=keys).ids
    ones = np.ones((T, K), bool)
    assert LY.node_fanout(lim, ones, E, N, N // G).max() <= M
    assert LY.node_fanout(free, ones, E, N, N // G).max() > M


def test_busiest_chip_small_exact_cases():
    rng = np.random.default_rng(5)
    # T=2 tokens, one expert each, 2 chips of 1 expert: max load 2 or 1, mean 3/2
    loads = LY.busiest_chip_loads(rng.random((4000, 2, 2)), K=1, E=2, P=2)
    assert set(np.unique(loads)) <= {1, 2}
    assert abs(loads.mean() - 1.5) < 4 * 0.5 / np.sqrt(4000)
    # T=3, 3 chips: P(all distinct) = 6/27, P(all same) = 3/27, else max 2
    loads = LY.busiest_chip_loads(rng.random((6000, 3, 3)), K=1, E=3, P=3)
    exact = Fraction(6 * 1 + 18 * 2 + 3 * 3, 27)
    var = Fraction(6 * 1 + 18 * 4 + 3 * 9, 27) - exact * exact
    assert abs(loads.mean() - float(exact)) < 4 * np.sqrt(float(var) / 6000)
    # one chip holds everything
    loads = LY.busiest_chip_loads(rng.random((5, 10, 8)), K=3, E=8, P=1)
    assert (loads == 30).all()
    m, q = LY.busiest_chip_estimate([1, 2, 2, 3])
    assert m == 2.0 and 2.9 < q <= 3.0
