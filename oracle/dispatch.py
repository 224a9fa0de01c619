"""Dispatch: per-expert counts, capacity drops, expert-contiguous layout, send matrix.

Definitions followed:
  * Capacity is a per-expert upper bound on the tokens it takes in one micro-batch
    ([EP-concept] "技術原理", key parameters; [EP-notes] "MoE 结构回顾").
  * Tokens over capacity skip that expert's computation ([EP-notes] "MoE 结构回顾");
    a full buffer either drops or pads ([EP-notes] "负载均衡"; [EP-serving] "技術洞察":
    padding keeps each expert GEMM a predictable shape).
  * Dispatch regroups tokens by destination expert / GPU ([EP-wiki] opening summary
    and "核心思想"; [EP-overview] "Dispatch 和 Combine 各做什么？").
  * Experts live on chips in contiguous blocks, chip = expert // (E / N_EP)
    ([EP-overview] "Dispatch 通信矩阵" example and tbl-ep-01); an EP group is a run of
    contiguous chip ids ([EP-overview] glossary "EP 组").
  * Send matrix C[i][j] = n_ij * h * dtype_size, n_ij the tokens chip i routes to chip j
    ([EP-overview] eq. par-ep-dispatch-matrix); chip i holds B/N_EP tokens
    ([EP-overview] "Dispatch 通信矩阵" example: 512 tokens over 64 chips, 8 each).

Readings where the pages are silent:
  * cap = ceil(cf * T * K / E), exact rational arithmetic; cf <= 0 means no limit.
  * drop priority is token order: the pair (t, e) is kept iff fewer than cap earlier
    tokens chose e; dropped pairs are not renormalised.
  * token t sits on source chip t // (T / N_EP) (contiguous blocks); n_ij counts kept
    (token, expert) pairs, the diagonal included.
  * local rows are ordered by (expert, token); padded mode gives each local expert a
    block of exactly cap rows, unused rows have row_src = -1 and zero contents.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction

import numpy as np


def capacity(capacity_factor, T, K, E):
    """ceil(cf * T * K / E) computed exactly; None when cf <= 0 (no limit)."""
    if capacity_factor is None or capacity_factor <= 0:
        return None
    q = Fraction(capacity_factor) * T * K / E
    return math.ceil(q)


def max_rows(T, K, E, n_ep, cap, pad):
    """Upper bound on the rows of this rank's expert buffer."""
    El = E // n_ep
    if cap is None:
        return T * min(K, El)
    if pad:
        return El * cap
    return min(T * min(K, El), El * cap)


@dataclass
class DispatchResult:
    counts: np.ndarray       # [E] int32, pairs per expert before capacity
    offsets: np.ndarray      # [E_l + 1] int32, first row of each local expert
    dest_row: np.ndarray     # [T, K] int32, row in the local buffer or -1
    row_src: np.ndarray      # [R_max] int32, t*K+k of the row or -1
    kept: np.ndarray         # [T, K] bool, pair survives capacity
    n_dropped: int
    send_bytes: np.ndarray   # [N, N] int64 (or None when T % N != 0)
    n_pairs: np.ndarray      # [N, N] int64 pair counts
    rows: int                # offsets[E_l]
    cap: int | None


def dispatch(ids, *, E, n_ep=1, ep_rank=0, capacity_factor=0.0, pad=False, h=0,
             dtype_size=2) -> DispatchResult:
    ids = np.asarray(ids)
    T, K = ids.shape
    El = E // n_ep
    e0 = ep_rank * El
    cap = capacity(capacity_factor, T, K, E)
    if pad and cap is None:
        raise ValueError("padding needs a capacity")

    # Walk the pairs in token order, k order within a token, counting per expert.
    seen = [0] * E
    rank = np.zeros((T, K), np.int64)
    kept = np.zeros((T, K), bool)
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            rank[t, k] = seen[e]
            seen[e] += 1
            kept[t, k] = cap is None or rank[t, k] < cap
    counts = np.array(seen, np.int32)
    n_dropped = int(T * K - kept.sum())

    # Offsets of the local experts' row blocks.
    offsets = np.zeros(El + 1, np.int32)
    for el in range(El):
        n_el = int(counts[e0 + el]) if cap is None else min(int(counts[e0 + el]), cap)
        offsets[el + 1] = offsets[el] + (cap if pad else n_el)
    rows = int(offsets[El])

    R_max = max_rows(T, K, E, n_ep, cap, pad)
    dest_row = np.full((T, K), -1, np.int32)
    row_src = np.full(R_max, -1, np.int32)
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            if kept[t, k] and e0 <= e < e0 + El:
                r = int(offsets[e - e0] + rank[t, k])
                dest_row[t, k] = r
                row_src[r] = t * K + k

    # Send matrix over the N_EP virtual chips.
    send = None
    n_pairs = None
    if T % n_ep == 0:
        tpc = T // n_ep
        n_pairs = np.zeros((n_ep, n_ep), np.int64)
        for t in range(T):
            for k in range(K):
                if kept[t, k]:
                    n_pairs[t // tpc, int(ids[t, k]) // El] += 1
        send = n_pairs * h * dtype_size
    return DispatchResult(counts=counts, offsets=offsets, dest_row=dest_row, row_src=row_src,
                          kept=kept, n_dropped=n_dropped, send_bytes=send, n_pairs=n_pairs,
                          rows=rows, cap=cap)


def permute(x, d: DispatchResult, K):
    """xp[r] = x[row_src[r] // K]; rows with row_src = -1 are zero."""
    x = np.asarray(x)
    xp = np.zeros((d.row_src.shape[0],) + x.shape[1:], x.dtype)
    for r, src in enumerate(d.row_src):
        if src >= 0:
            xp[r] = x[src // K]
    return xp
