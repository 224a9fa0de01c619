"""Pins for the oracle's dispatch (CPU only): capacity, drops, layout and send matrix.

Independent ground truth: the pair rank recomputed from a cumulative one-hot count
(vectorised, no walk), a queue simulation of expert buffers filling in token order,
integer invariants, and the pages' worked layout examples (tests/golden).
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import dispatch, capacity
from oracle.dispatch import permute

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def random_ids(rng, T, E, K):
    return np.stack([np.sort(rng.choice(E, K, replace=False)) for _ in range(T)]).astype(np.int32)


def test_capacity_values():
    assert capacity(1.25, 64, 2, 8) == 20          # tiny fp32 workload
    assert capacity(1.0, 8192, 6, 64) == 768       # skew workload, cf 1.0
    assert capacity(0.0, 10, 1, 1) is None
    assert capacity(1.5, 3, 1, 2) == 3             # ceil(2.25)
    assert capacity(2.0, 3, 1, 2) == 3             # exact 3, no rounding up


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 40), st.sampled_from([(4, 1), (4, 2), (8, 3), (6, 6)]),
       st.sampled_from([0.0, 0.5, 1.0, 1.25]), st.sampled_from([1, 2]), st.integers(0, 10**6))
def test_drops_match_cumulative_rank(T, EK, cf, n_ep, seed):
    E, K = EK
    rng = np.random.default_rng(seed)
    ids = random_ids(rng, T, E, K)
    d = dispatch(ids, E=E, n_ep=n_ep, ep_rank=n_ep - 1, capacity_factor=cf, h=4, dtype_size=2)
    onehot = np.zeros((T, E), np.int64)
    for t in range(T):
        onehot[t, ids[t]] = 1
    prior = np.cumsum(onehot, axis=0) - onehot          # earlier tokens per expert
    rank = np.take_along_axis(prior, ids.astype(np.int64), axis=1)
    cap = d.cap
    kept = np.ones_like(rank, bool) if cap is None else rank < cap
    np.testing.assert_array_equal(d.kept, kept)
    np.testing.assert_array_equal(d.counts, onehot.sum(0))
    assert d.n_dropped == T * K - kept.sum()
    if cap is not None:
        assert (np.minimum(d.counts, cap) == np.bincount(ids[kept], minlength=E)).all()


def test_drops_queue_simulation():
    rng = np.random.default_rng(7)
    T, E, K, cf = 50, 5, 2, 0.8
    ids = random_ids(rng, T, E, K)
    d = dispatch(ids, E=E, capacity_factor=cf)
    cap = d.cap
    buffers = {e: [] for e in range(E)}
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            if len(buffers[e]) < cap:
                buffers[e].append((t, k))
    kept = np.zeros((T, K), bool)
    for e, lst in buffers.items():
        for t, k in lst:
            kept[t, k] = True
    np.testing.assert_array_equal(d.kept, kept)
    # local rows: expert blocks in order, tokens in order inside a block
    order = [src for e in range(E) for (t, k) in buffers[e] for src in [t * K + k]]
    np.testing.assert_array_equal(d.row_src[:d.rows], order)


@pytest.mark.parametrize("pad", [False, True])
def test_layout_invariants(pad):
    rng = np.random.default_rng(11)
    T, E, K, N = 96, 16, 4, 4
    ids = random_ids(rng, T, E, K)
    for r in range(N):
        d = dispatch(ids, E=E, n_ep=N, ep_rank=r, capacity_factor=1.0, pad=pad, h=8, dtype_size=2)
        El = E // N
        e0 = r * El
        # dest_row and row_src are inverse maps on the kept local pairs
        for t in range(T):
            for k in range(K):
                dr = d.dest_row[t, k]
                local = e0 <= ids[t, k] < e0 + El
                assert (dr >= 0) == (d.kept[t, k] and local)
                if dr >= 0:
                    assert d.row_src[dr] == t * K + k
        live = d.row_src[d.row_src >= 0]
        assert len(live) == len(set(live.tolist()))
        assert ((d.dest_row >= 0).sum()) == len(live)
        # sorted by (expert, token) within the live rows
        keyv = [(int(ids[s // K, s % K]), s // K) for s in live]
        assert keyv == sorted(keyv)
        if pad:
            np.testing.assert_array_equal(d.offsets, np.arange(El + 1) * d.cap)
            for el in range(El):
                blk = d.row_src[d.offsets[el]:d.offsets[el + 1]]
                n = min(int(d.counts[e0 + el]), d.cap)
                assert (blk[:n] >= 0).all() and (blk[n:] == -1).all()
        else:
            assert d.offsets[-1] == len(live) == d.rows
            assert (d.row_src[d.rows:] == -1).all()


def test_permute_copies_rows_and_zero_pads():
    rng = np.random.default_rng(3)
    ids = random_ids(rng, 10, 4, 2)
    x = rng.normal(size=(10, 5))
    d = dispatch(ids, E=4, capacity_factor=0.75, pad=True)
    xp = permute(x, d, 2)
    for r, s in enumerate(d.row_src):
        if s >= 0:
            np.testing.assert_array_equal(xp[r], x[s // 2])
        else:
            assert (xp[r] == 0).all()


def test_send_matrix_totals_match_volume_formulas():
    """Sum of C = M_total and mean row sum = M_per_chip when nothing is dropped
    (eq. par-ep-comm-total / par-ep-comm-per-chip), at the DeepSeek-V3 EP=64 shape."""
    rng = np.random.default_rng(0)
    B, K, E, N, h, s = 4096, 8, 256, 64, 7168, 2
    keys = rng.random((B, E))
    rr = oracle.route(K=K, score="softmax", logits=keys)
    d = dispatch(rr.ids, E=E, n_ep=N, h=h, dtype_size=s)
    assert d.send_bytes.sum() == oracle.volumes.m_total(B, K, h, s)
    assert d.send_bytes.sum(1).mean() == oracle.volumes.m_per_chip(B, K, h, s, N) == 7_340_032
    # column sums = bytes each chip receives = pairs on its 4 experts * h * s
    np.testing.assert_array_equal(d.send_bytes.sum(0),
                                  d.counts.reshape(N, E // N).sum(1) * h * s)


def test_send_matrix_with_drops():
    rng = np.random.default_rng(5)
    T, E, K, N = 64, 8, 2, 4
    ids = random_ids(rng, T, E, K)
    d = dispatch(ids, E=E, n_ep=N, capacity_factor=0.5, h=16, dtype_size=4)
    assert d.n_dropped > 0
    assert d.send_bytes.sum() == (T * K - d.n_dropped) * 16 * 4
    # brute force per pair
    n = np.zeros((N, N), np.int64)
    for t in range(T):
        for k in range(K):
            if d.kept[t, k]:
                n[t // (T // N), ids[t, k] // (E // N)] += 1
    np.testing.assert_array_equal(d.send_bytes, n * 64)


def test_pair_expectation_uniform_routing():
    """E[C_ij] = m_pair under uniform routing (eq. par-ep-comm-pair), for one fixed
    off-diagonal pair, averaged over seeds (an expectation, so a sampling tolerance)."""
    B, K, E, N, h, s = 256, 4, 64, 8, 16, 2
    vals = []
    for seed in range(200):
        keys = np.random.default_rng(seed).random((B, E))
        rr = oracle.route(K=K, score="softmax", logits=keys)
        d = dispatch(rr.ids, E=E, n_ep=N, h=h, dtype_size=s)
        vals.append(d.send_bytes[2, 5])
    mp = float(oracle.volumes.m_pair(B, K, h, s, N))
    # n_25 ~ Binomial(B/N * K, 1/N) approximately -> std of the mean of 200 draws
    std = np.sqrt(B / N * K * (1 / N) * (1 - 1 / N)) * h * s / np.sqrt(200)
    assert abs(np.mean(vals) - mp) < 4 * std


def test_tbl_ep_01_experts_per_chip():
    g = json.load(open(os.path.join(GOLD, "ep_layout_examples.json")))["tbl_ep_01"]
    for n, per in g["experts_per_chip"].items():
        ids = np.arange(g["E"], dtype=np.int32).reshape(-1, 1)   # one token per expert
        d = dispatch(ids, E=g["E"], n_ep=int(n), h=1, dtype_size=1)
        assert len(d.offsets) - 1 == per
        # every chip receives exactly its `per` experts' tokens
        assert (d.send_bytes.sum(0) == per).all()


def test_two_gpu_example_chip_map():
    g = json.load(open(os.path.join(GOLD, "ep_layout_examples.json")))["two_gpu_example"]
    for e in range(g["E"]):
        ids = np.array([[e], [e]], np.int32)
        d = dispatch(ids, E=g["E"], n_ep=g["N_EP"], h=1, dtype_size=1)
        j = np.nonzero(d.send_bytes.sum(0))[0]
        assert list(j) == [g["chip_of_expert"][e]]


def test_dispatch_matrix_example():
    g = json.load(open(os.path.join(GOLD, "ep_layout_examples.json")))["dispatch_matrix_example"]
    B, K, E, N = g["B"], g["K"], g["E"], g["N_EP"]
    assert B // N == g["tokens_per_chip"] and E // N == g["experts_per_chip"]
    keys = np.random.default_rng(0).random((B, E))
    rr = oracle.route(K=K, score="softmax", logits=keys)
    d = dispatch(rr.ids, E=E, n_ep=N, h=7168, dtype_size=2)
    # a token reaches at most K chips
    for t in range(B):
        assert len(set((rr.ids[t] // (E // N)).tolist())) <= g["max_target_chips_per_token"]
    lo, hi = g["target_chips_per_chip_range"]
    tpc = oracle.volumes.targets_per_chip(d.send_bytes)
    assert lo <= tpc.mean() <= hi
    assert lo <= oracle.volumes.expected_target_chips(E, N, K, B) <= hi
    assert (tpc >= lo).mean() > 0.9 and (tpc <= hi).mean() > 0.9


def test_planted_drop_order_mistake_is_caught(monkeypatch):
    """Dropping by k-slot priority instead of token order must fail the rank pin."""
    rng = np.random.default_rng(9)
    ids = random_ids(rng, 30, 4, 2)
    d = dispatch(ids, E=4, capacity_factor=0.5)
    # k-slot-major walk (a GShard-like priority) gives a different kept set
    seen = [0] * 4
    kept = np.zeros((30, 2), bool)
    for k in range(2):
        for t in range(30):
            e = ids[t, k]
            kept[t, k] = seen[e] < d.cap
            seen[e] += 1
    assert not np.array_equal(kept, d.kept)
