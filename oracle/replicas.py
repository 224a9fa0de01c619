"""Redundant experts: a logical -> physical replica map and dispatch over it, in plain Python
with exact integer / rational arithmetic. TEST INFRASTRUCTURE ONLY (see the package
docstring).

Definitions followed ([EP-overview] glossary, tbl-ep-overview-glossary):
  * A logical expert is the unit the model's weights define (256 per DeepSeek-V3 layer); a
    physical expert (replica) is an instance a placement algorithm such as EPLB makes of a
    logical expert and puts on a GPU; the number of physical experts must be a multiple of
    the number of GPUs.
  * Redundant experts are replicas budgeted beyond the logical count (256 logical + 32
    redundant = 288 physical), used to copy hot experts and flatten the load.
  * Balancedness = mean / max of the per-GPU MoE time (LMSYS definition).
  * Replicating hot experts is the third design route against skew ([EP-wiki] 设计空间与
    取舍, route 3), motivated by hot-expert skew such as Kimi-K2's ([EP-wiki] 关键观察 1).

Readings where the pages are silent (the EPLB algorithm itself is on a page not given):
  * Budget: R redundant slots, P = E + R physical experts, P a multiple of n_ep; rank j
    holds physical ids [j P/n_ep, (j+1) P/n_ep).
  * Replica counts: every logical expert starts with one replica; each redundant slot goes
    to the expert with the largest load per replica load_e / r_e (exact rational
    comparison), ties to the lower expert id. Loads are a routing's per-expert pair counts.
  * Token -> replica: the pairs of logical expert e are dealt to its r_e replicas round
    robin in token order: the pair ranked rho among e's pairs (0 = earliest token) goes to
    replica rho mod r_e, where it ranks floor(rho / r_e). Replica q of e therefore receives
    floor(load_e / r_e) + [q < load_e mod r_e] pairs.
  * Packing: replicas sorted by those pair counts (descending; ties: lower expert id, then
    lower replica index) go one by one to the rank with the least load so far among ranks
    with a free slot (ties to the lower rank); a rank's slots fill in placement order.
  * Capacity with replicas is per physical expert: cap_p = ceil(cf T K / P); a pair is kept
    iff its rank within its replica is below cap_p. No padding.
  * A rank's load is the kept pairs its physical experts receive; balancedness is mean /
    max over ranks (pairs standing in for MoE time).

Pins (tests/test_oracle_replicas.py): replica counts against brute force over all budget
splits (the greedy attains the least maximum load per replica); the packing against an
independent heap-based implementation of the same rule and its invariants; dispatch with
R = 0 equal to plain dispatch; the rank formula against a sequential per-replica counter
walk; per-replica counts within one of load/r; send totals; balancedness on skewed routing.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction

import numpy as np


@dataclass
class ReplicaPlan:
    P: int                   # physical experts
    n_ep: int
    counts: np.ndarray       # [E] replicas per logical expert (r_e >= 1)
    rep_start: np.ndarray    # [E + 1] replicas of e are rep_list[rep_start[e]:rep_start[e+1]]
    rep_list: np.ndarray     # [P] physical id of replica q of e, in replica order
    phys_expert: np.ndarray  # [P] logical expert held by each physical id
    phys_replica: np.ndarray  # [P] its replica index q


def replica_counts(load, R):
    """r_e: one replica each, then R more, each to the largest load_e / r_e (ties: lower e)."""
    load = [int(v) for v in load]
    r = [1] * len(load)
    for _ in range(R):
        best = 0
        for e in range(1, len(load)):
            # load_e / r_e > load_best / r_best, exactly
            if load[e] * r[best] > load[best] * r[e]:
                best = e
        r[best] += 1
    return np.asarray(r, np.int32)


def replica_pairs(load_e, r_e, q):
    """Pairs replica q of an expert with load_e pairs over r_e replicas receives."""
    return load_e // r_e + (1 if q < load_e % r_e else 0)


def plan(load, R, n_ep):
    """The replica map for per-expert loads, R redundant slots and n_ep ranks."""
    load = [int(v) for v in load]
    E = len(load)
    P = E + R
    if P % n_ep != 0:
        raise ValueError("physical experts must be a multiple of the ranks")
    per = P // n_ep
    r = replica_counts(load, R)
    reps = [(replica_pairs(load[e], int(r[e]), q), e, q) for e in range(E) for q in range(r[e])]
    reps.sort(key=lambda x: (-x[0], x[1], x[2]))
    rank_load = [0] * n_ep
    rank_fill = [0] * n_ep
    phys_expert = np.full(P, -1, np.int32)
    phys_replica = np.full(P, -1, np.int32)
    rep_phys = {}
    for w, e, q in reps:
        best = None
        for j in range(n_ep):
            if rank_fill[j] < per and (best is None or rank_load[j] < rank_load[best]):
                best = j
        p = best * per + rank_fill[best]
        rank_fill[best] += 1
        rank_load[best] += w
        phys_expert[p] = e
        phys_replica[p] = q
        rep_phys[(e, q)] = p
    rep_start = np.zeros(E + 1, np.int32)
    for e in range(E):
        rep_start[e + 1] = rep_start[e] + r[e]
    rep_list = np.empty(P, np.int32)
    for e in range(E):
        for q in range(r[e]):
            rep_list[rep_start[e] + q] = rep_phys[(e, q)]
    return ReplicaPlan(P=P, n_ep=n_ep, counts=r, rep_start=rep_start, rep_list=rep_list,
                       phys_expert=phys_expert, phys_replica=phys_replica)


@dataclass
class ReplicatedDispatch:
    counts: np.ndarray       # [E] pairs per logical expert (before capacity)
    phys_counts: np.ndarray  # [P] pairs per physical expert (before capacity)
    offsets: np.ndarray      # [P/n_ep + 1] first row of each local physical expert
    dest_row: np.ndarray     # [T, K] row in this rank's buffer or -1
    row_src: np.ndarray      # [R_max] t*K+k of the row or -1
    kept: np.ndarray         # [T, K] bool
    phys_of_pair: np.ndarray  # [T, K] physical expert of each pair
    n_dropped: int
    send_bytes: np.ndarray   # [N, N] int64 (None when T % N != 0)
    rank_loads: np.ndarray   # [N] kept pairs received per rank
    rows: int
    cap: int | None


def capacity_physical(capacity_factor, T, K, P):
    """ceil(cf T K / P) exactly; None when cf <= 0."""
    if capacity_factor is None or capacity_factor <= 0:
        return None
    return math.ceil(Fraction(capacity_factor) * T * K / P)


def dispatch_replicated(ids, rp: ReplicaPlan, *, E, n_ep=1, ep_rank=0, capacity_factor=0.0,
                        h=0, dtype_size=2):
    """Dispatch over the replica map: each pair walked in token order (k order within a
    token) goes to replica (its rank among its logical expert's pairs) mod r_e."""
    ids = np.asarray(ids)
    T, K = ids.shape
    P = rp.P
    Pl = P // n_ep
    p0 = ep_rank * Pl
    cap = capacity_physical(capacity_factor, T, K, P)
    seen = [0] * E
    phys_seen = [0] * P
    phys = np.zeros((T, K), np.int64)
    prank = np.zeros((T, K), np.int64)
    kept = np.zeros((T, K), bool)
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            rho = seen[e]
            seen[e] += 1
            r_e = int(rp.counts[e])
            p = int(rp.rep_list[rp.rep_start[e] + rho % r_e])
            phys[t, k] = p
            prank[t, k] = rho // r_e
            phys_seen[p] += 1
            kept[t, k] = cap is None or prank[t, k] < cap
    counts = np.asarray(seen, np.int32)
    phys_counts = np.asarray(phys_seen, np.int32)
    offsets = np.zeros(Pl + 1, np.int32)
    for pl in range(Pl):
        n = int(phys_counts[p0 + pl])
        offsets[pl + 1] = offsets[pl] + (n if cap is None else min(n, cap))
    rows = int(offsets[Pl])
    Rmax = T * min(K, Pl) if cap is None else min(T * min(K, Pl), Pl * cap)
    dest_row = np.full((T, K), -1, np.int32)
    row_src = np.full(Rmax, -1, np.int32)
    for t in range(T):
        for k in range(K):
            p = int(phys[t, k])
            if kept[t, k] and p0 <= p < p0 + Pl:
                rr = int(offsets[p - p0] + prank[t, k])
                dest_row[t, k] = rr
                row_src[rr] = t * K + k
    rank_loads = np.zeros(n_ep, np.int64)
    for t in range(T):
        for k in range(K):
            if kept[t, k]:
                rank_loads[int(phys[t, k]) // Pl] += 1
    send = None
    if T % n_ep == 0:
        tpc = T // n_ep
        n_pairs = np.zeros((n_ep, n_ep), np.int64)
        for t in range(T):
            for k in range(K):
                if kept[t, k]:
                    n_pairs[t // tpc, int(phys[t, k]) // Pl] += 1
        send = n_pairs * h * dtype_size
    return ReplicatedDispatch(counts=counts, phys_counts=phys_counts, offsets=offsets,
                              dest_row=dest_row, row_src=row_src, kept=kept,
                              phys_of_pair=phys.astype(np.int32),
                              n_dropped=int(T * K - kept.sum()), send_bytes=send,
                              rank_loads=rank_loads, rows=rows, cap=cap)


def identity_plan(E, n_ep):
    """No redundant experts: physical expert e is logical expert e."""
    return plan([0] * E, 0, n_ep) if E % n_ep == 0 else None


def rank_loads_unreplicated(ids, kept, E, n_ep):
    """Kept pairs per rank with experts in contiguous blocks of E/n_ep (no replicas)."""
    ids = np.asarray(ids)
    out = np.zeros(n_ep, np.int64)
    El = E // n_ep
    for e, k in zip(ids.reshape(-1), np.asarray(kept).reshape(-1)):
        if k:
            out[int(e) // El] += 1
    return out
