"""Pins for the oracle's replica map and replicated dispatch (CPU only).

Ground truth independent of the oracle's code path:
  * brute force over every split of the redundant budget: the greedy replica counts attain
    the least possible maximum load per replica;
  * an independent implementation of the packing rule (a heap keyed on (load, rank));
  * plain dispatch, which the replicated dispatch must equal when every logical expert has
    one replica at its own physical id;
  * a sequential per-replica counter walk for the kept flags and per-replica ranks;
  * closed facts: round-robin dealing gives floor / ceil shares, send totals equal the kept
    pairs times the row size, balancedness on skewed routing.
"""
import heapq
import itertools
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import replicas as RP


def compositions(n, k):
    """All ways to write n as an ordered sum of k non-negative integers."""
    for cut in itertools.combinations(range(n + k - 1), k - 1):
        parts, prev = [], -1
        for c in cut + (n + k - 1,):
            parts.append(c - prev - 1)
            prev = c
        yield parts


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(0, 40), min_size=1, max_size=5), st.integers(0, 4))
def test_replica_counts_minimise_max_load_per_replica(load, R):
    r = RP.replica_counts(load, R)
    assert r.sum() == len(load) + R and (r >= 1).all()
    got = max(Fraction(l, int(c)) for l, c in zip(load, r))
    best = min(max(Fraction(l, 1 + x) for l, x in zip(load, extra))
               for extra in compositions(R, len(load)))
    assert got == best


def test_replica_counts_ties_go_to_lower_id():
    assert list(RP.replica_counts([5, 5, 5], 1)) == [2, 1, 1]
    assert list(RP.replica_counts([4, 8], 1)) == [1, 2]
    assert list(RP.replica_counts([4, 8], 2)) == [2, 2]    # 4/1 = 8/2: the lower id


def heap_packing(load, counts, n_ep):
    """The packing rule written again with a heap of (rank load, rank) over open ranks."""
    E = len(load)
    P = int(sum(counts))
    per = P // n_ep
    reps = sorted(((RP.replica_pairs(load[e], int(counts[e]), q), e, q)
                   for e in range(E) for q in range(counts[e])),
                  key=lambda x: (-x[0], x[1], x[2]))
    heap = [(0, j) for j in range(n_ep)]
    fill = [0] * n_ep
    where = {}
    for w, e, q in reps:
        ld, j = heapq.heappop(heap)
        where[(e, q)] = j * per + fill[j]
        fill[j] += 1
        if fill[j] < per:
            heapq.heappush(heap, (ld + w, j))
    return where


@settings(max_examples=150, deadline=None)
@given(st.lists(st.integers(0, 60), min_size=2, max_size=12), st.integers(0, 6),
       st.sampled_from([1, 2, 3, 4]))
def test_packing_follows_the_rule(load, R, n_ep):
    E = len(load)
    if (E + R) % n_ep:
        R += n_ep - (E + R) % n_ep
    rp = RP.plan(load, R, n_ep)
    P = E + R
    assert rp.P == P
    # every physical id holds one replica; every expert its r_e replicas, in replica order
    assert sorted(rp.rep_list.tolist()) == list(range(P))
    for e in range(E):
        reps = rp.rep_list[rp.rep_start[e]:rp.rep_start[e + 1]]
        assert len(reps) == rp.counts[e]
        for q, p in enumerate(reps):
            assert rp.phys_expert[p] == e and rp.phys_replica[p] == q
    where = heap_packing(load, rp.counts, n_ep)
    for (e, q), p in where.items():
        assert rp.rep_list[rp.rep_start[e] + q] == p


def test_packing_worked_example():
    # loads 9, 3, 2, 2 with 4 redundant slots on 2 ranks: replicas 9 -> 4 (per replica
    # 9/4), 3 -> 2, the others one each: pair shares (3, 2, 2, 2), (2, 1), 2, 2; packed by
    # share onto the less loaded rank: rank 0 gets {e0q0=3, e0q3=2, e2=2, e1q1=1} = 8,
    # rank 1 gets {e0q1=2, e0q2=2, e1q0=2, e3=2} = 8
    rp = RP.plan([9, 3, 2, 2], 4, 2)
    assert list(rp.counts) == [4, 2, 1, 1]
    assert list(rp.phys_expert) == [0, 0, 2, 1, 0, 0, 1, 3]
    assert list(rp.phys_replica) == [0, 3, 0, 1, 1, 2, 0, 0]


def test_plan_needs_a_multiple_of_ranks():
    with pytest.raises(ValueError):
        RP.plan([1, 2, 3], 0, 2)


def _ids(T, E, K, seed, skew=0.0):
    rng = np.random.default_rng(seed)
    logits = rng.normal(size=(T, E)) - skew * np.log(np.arange(1, E + 1))[None, :]
    return oracle.route(K=K, score="softmax", logits=logits).ids


@pytest.mark.parametrize("cf", [0.0, 1.0, 0.5])
def test_identity_map_equals_plain_dispatch(cf):
    ids = _ids(64, 16, 3, 0, skew=1.0)
    for n_ep, rank in [(1, 0), (4, 2)]:
        rp = RP.identity_plan(16, n_ep)
        assert list(rp.phys_expert) == list(range(16))
        got = RP.dispatch_replicated(ids, rp, E=16, n_ep=n_ep, ep_rank=rank, capacity_factor=cf,
                                     h=32, dtype_size=2)
        ref = oracle.dispatch(ids, E=16, n_ep=n_ep, ep_rank=rank, capacity_factor=cf, h=32,
                              dtype_size=2)
        np.testing.assert_array_equal(got.counts, ref.counts)
        np.testing.assert_array_equal(got.offsets, ref.offsets)
        np.testing.assert_array_equal(got.dest_row, ref.dest_row)
        np.testing.assert_array_equal(got.row_src, ref.row_src)
        np.testing.assert_array_equal(got.send_bytes, ref.send_bytes)
        assert got.n_dropped == ref.n_dropped


@pytest.mark.parametrize("cf", [0.0, 1.0])
def test_replicated_dispatch_against_counter_walk(cf):
    T, E, K, N = 96, 12, 3, 4
    ids = _ids(T, E, K, 1, skew=1.5)
    load = np.bincount(ids.reshape(-1), minlength=E)
    rp = RP.plan(load, 8, N)
    P = rp.P
    d = RP.dispatch_replicated(ids, rp, E=E, n_ep=N, ep_rank=1, capacity_factor=cf, h=8)
    cap = RP.capacity_physical(cf, T, K, P)
    # sequential walk: a counter per logical expert picks the replica, a counter per
    # physical expert gives the rank within it
    lcnt, pcnt = [0] * E, [0] * P
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            p = int(rp.rep_list[rp.rep_start[e] + lcnt[e] % rp.counts[e]])
            lcnt[e] += 1
            assert d.phys_of_pair[t, k] == p
            assert d.kept[t, k] == (cap is None or pcnt[p] < cap)
            pcnt[p] += 1
    np.testing.assert_array_equal(d.phys_counts, pcnt)
    # round robin: shares of one expert differ by at most one, larger ones first
    for e in range(E):
        sh = [d.phys_counts[p] for p in rp.rep_list[rp.rep_start[e]:rp.rep_start[e + 1]]]
        assert sum(sh) == load[e] and max(sh) - min(sh) <= 1 and sh == sorted(sh, reverse=True)
    # layout: dest_row / row_src inverse, rows ordered by (physical expert, token)
    Pl = P // N
    rows = [(r, s) for r, s in enumerate(d.row_src[:d.rows])]
    assert all(s >= 0 for _, s in rows)
    for r, s in rows:
        assert d.dest_row[s // K, s % K] == r
    keys = [(int(d.phys_of_pair[s // K, s % K]), s // K) for _, s in rows]
    assert keys == sorted(keys)
    assert all(Pl * 1 <= p < Pl * 2 for p, _ in keys)
    # send matrix: every kept pair once; rank loads are its column sums
    assert d.send_bytes.sum() == d.kept.sum() * 8 * 2
    np.testing.assert_array_equal(d.send_bytes.sum(0) // 16, d.rank_loads)
    assert d.n_dropped == T * K - d.kept.sum()
    if cf <= 0:
        assert d.n_dropped == 0


def test_replicas_raise_balancedness_on_skewed_routing():
    # Zipf-like skew over 64 experts at top-6 on 8 ranks: 16 redundant slots placed by the
    # per-rank loads lift mean/max well above the contiguous unreplicated layout's
    T, E, K, N = 2048, 64, 6, 8
    ids = _ids(T, E, K, 2, skew=1.2)
    load = np.bincount(ids.reshape(-1), minlength=E)
    plain = RP.rank_loads_unreplicated(ids, np.ones_like(ids, bool), E, N)
    b0 = oracle.volumes.balancedness(plain)
    rp = RP.plan(load, 16, N)
    d = RP.dispatch_replicated(ids, rp, E=E, n_ep=N, h=8)
    b1 = oracle.volumes.balancedness(d.rank_loads)
    assert d.rank_loads.sum() == plain.sum() == T * K
    assert b1 > b0 and b1 > 0.9, (b0, b1)
