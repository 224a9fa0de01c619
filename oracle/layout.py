"""Layout statistics of a routing over N_EP virtual ranks, and a Monte Carlo estimate of
the busiest rank's load. TEST INFRASTRUCTURE ONLY (see the package docstring).

Definitions followed:
  * One token reaches at most K target chips, while one chip's tokens together reach
    many chips, approaching the whole EP group as the batch grows ([EP-overview]
    "Dispatch 通信矩阵": per-token fan-out versus per-chip fan-out).
  * Node-limited routing lets each token reach at most M nodes ([EP-overview]
    "Dispatch 通信矩阵", DeepSeek-V3 node-limited routing): it is group-limited routing
    ([EP-overview] glossary "Expert group") with one group per node, so a token's
    experts span at most M nodes.
  * The load of the busiest chip under random top-K choices is estimated by sampling
    many random selections and recording the busiest chip's load, its expectation and
    an upper quantile bounding the worst case ([EP-overview] "如何在不跑模型时估算 EP
    负载？", the Monte Carlo paragraph).

Readings where the pages are silent:
  * tokens_to[i][j] counts distinct tokens of source chip i with at least one kept
    expert on chip j (a token's row crosses to a chip once, however many of its experts
    live there); the pair count n_ij of the send matrix counts every kept pair.
  * A token's fan-out is its number of distinct target chips among kept pairs (0 when
    every pair was dropped).
  * Chips hold contiguous blocks of E/N experts and tokens contiguous blocks of T/N, as
    for the send matrix.
  * "Load" of a chip is the number of kept (token, expert) pairs it receives.

Pins (tests/test_oracle_layout.py): the mean fan-out of uniformly random K-subsets
against its closed form N (1 - C(E - E/N, K) / C(E, K)); N = 1 and N = E special
cases; consistency with the pair counts of dispatch; an exact small busiest-chip
distribution (T = 2, K = 1, E = P = 2: expected maximum 3/2) and P = 1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

from .route import route


@dataclass
class LayoutStats:
    tokens_to: np.ndarray    # [N, N] int64: distinct tokens of chip i with a kept pair on j
    recv_pairs: np.ndarray   # [N] int64: kept pairs whose expert lives on chip j
    fanout_hist: np.ndarray  # [K + 1] int64: tokens by number of distinct target chips


def layout_stats(ids, kept, E, n_ep):
    """Per-token target chips of the kept pairs, walked token by token."""
    ids = np.asarray(ids)
    kept = np.asarray(kept, bool)
    T, K = ids.shape
    N = n_ep
    El = E // N
    tokens_to = np.zeros((N, N), np.int64)
    recv = np.zeros(N, np.int64)
    hist = np.zeros(K + 1, np.int64)
    tpr = T // N if T % N == 0 else None
    for t in range(T):
        chips = set()
        for k in range(K):
            if kept[t, k]:
                j = int(ids[t, k]) // El
                recv[j] += 1
                chips.add(j)
        if tpr is not None:
            i = t // tpr
            for j in chips:
                tokens_to[i, j] += 1
        hist[len(chips)] += 1
    return LayoutStats(tokens_to, recv, hist)


def node_fanout(ids, kept, E, n_ep, ranks_per_node):
    """Distinct nodes reached by each token's kept pairs (node = chip // ranks_per_node)."""
    ids = np.asarray(ids)
    El = E // n_ep
    out = np.zeros(ids.shape[0], np.int64)
    for t in range(ids.shape[0]):
        out[t] = len({int(e) // El // ranks_per_node
                      for e, k in zip(ids[t], kept[t]) if k})
    return out


def expected_token_fanout(E, N, K):
    """Expected distinct chips reached by one uniformly random K-subset of E experts on
    N chips of E/N each: N (1 - C(E - E/N, K) / C(E, K)) (a chip is missed when all K
    experts avoid its E/N)."""
    El = E // N
    return N * (1 - Fraction(math.comb(E - El, K), math.comb(E, K)))


def busiest_chip_loads(keys_trials, K, E, P):
    """One Monte Carlo sample per trial: keys [T, E] (iid scores per token and expert),
    each token takes its top-K keys (ties to the lower index), chips hold E/P experts;
    returns the busiest chip's load (kept pairs, no capacity) of every trial."""
    out = []
    for keys in keys_trials:
        rr = route(K=K, score="softmax", renorm=True, logits=np.asarray(keys, np.float64))
        load = np.bincount(rr.ids.reshape(-1) // (E // P), minlength=P)
        out.append(int(load.max()))
    return np.asarray(out, np.int64)


def busiest_chip_estimate(loads, q=0.99):
    """Mean of the sampled busiest-chip loads and their q-quantile (the worst-case bound
    the estimate reports)."""
    loads = np.asarray(loads, np.float64)
    return float(loads.mean()), float(np.quantile(loads, q))
