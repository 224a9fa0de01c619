"""Closed forms for EP traffic and load that the layout must satisfy.

  M_total    = B K h s            [EP-overview] eq. par-ep-comm-total
  M_per_chip = B K / N h s        [EP-overview] eq. par-ep-comm-per-chip
  m_pair     = B K h s / N^2      [EP-overview] eq. par-ep-comm-pair (uniform routing)
  E_active   = E/P (1 - exp(-T K / E))   [EP-overview] eq. par-ep-active-experts
               (the balls-into-bins estimate); the exact expectation for uniformly
               random K-subsets is E/P (1 - (1 - K/E)^T), since one token misses a given
               expert with probability 1 - K/E.
  zero pairs: with uniform routing a source chip's B/N tokens all miss destination
               chip j's E/N experts with probability [C(E - E/N, K) / C(E, K)]^(B/N)
               ([EP-overview] section on why EP AllToAll differs: about 36% of chip
               pairs carry nothing at EP=64, 512 tokens).
  balancedness = mean(load) / max(load)   [EP-overview] glossary "Balancedness".
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def m_total(B, K, h, s):
    return B * K * h * s


def m_per_chip(B, K, h, s, N):
    return Fraction(B * K, N) * h * s


def m_pair(B, K, h, s, N):
    return Fraction(B * K * h * s, N * N)


def e_active_poisson(E, P, T, K):
    return E / P * (1.0 - math.exp(-T * K / E))


def e_active_exact(E, P, T, K):
    return E / P * (1.0 - (1.0 - K / E) ** T)


def zero_pair_probability(E, N, K, B):
    """Probability that one (source, destination) chip pair carries no pair."""
    miss = Fraction(math.comb(E - E // N, K), math.comb(E, K))
    return float(miss) ** (B // N)


def expected_target_chips(E, N, K, B):
    return N * (1.0 - zero_pair_probability(E, N, K, B))


def zero_pair_fraction(send):
    """Fraction of (i, j) chip pairs, diagonal included, whose send count is zero."""
    send = np.asarray(send)
    return float((send == 0).sum()) / send.size


def targets_per_chip(send, include_self=True):
    send = np.asarray(send).copy()
    if not include_self:
        np.fill_diagonal(send, 0)
    return (send != 0).sum(axis=1)


def balancedness(load):
    load = np.asarray(load, dtype=np.float64)
    return float(load.mean() / load.max()) if load.max() > 0 else 1.0


def peak_to_mean(load):
    load = np.asarray(load, dtype=np.float64)
    return float(load.max() / load.mean()) if load.mean() > 0 else 0.0
