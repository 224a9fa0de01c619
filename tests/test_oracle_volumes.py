"""Pins for the traffic and load statistics: the pages' printed values (tbl-ep-02, the
36% zero-pair figure) and closed forms checked by exhaustive counting or simulation."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import volumes as V
from synth import CONFIGS, make_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")
UNIT = {"MB": 1e6, "KB": 1e3, "MiB": 2**20, "KiB": 2**10}


def test_tbl_ep_02_cells():
    g = json.load(open(os.path.join(GOLD, "tbl_ep_02.json")))
    for row in g["rows"]:
        B, K, h, N = row["B"], row["K"], row["h"], row["N_EP"]
        per_chip = V.m_per_chip(B, K, h, 2, N)
        pair = V.m_pair(B, K, h, 2, N)
        assert per_chip == B * K * h * 2 / N
        # printed to 2-3 significant figures in the row's own units
        assert round(float(per_chip) / UNIT[row["per_chip_unit"]], 1 if per_chip > 1e6 else 2) \
            == pytest.approx(row["per_chip_value"])
        printed_pair = row["pair_value"] * UNIT[row["pair_unit"]]
        if row["pair_consistent"]:
            assert abs(float(pair) - printed_pair) / printed_pair < 0.01
        else:
            # the garbled cell: formula 114688 B, printed 117 KB
            assert pair == 114_688
            assert abs(float(pair) - printed_pair) / printed_pair > 0.015
    assert V.m_per_chip(4096, 8, 7168, 2, 64) == 7_340_032
    assert V.m_per_chip(4096, 8, 7168, 2, 8) == 58_720_256
    assert V.m_per_chip(2048, 1, 768, 2, 16) == 196_608


def test_zero_pair_closed_form_by_enumeration():
    """The miss probability C(E-E/N, K)/C(E, K), checked by enumerating all K-subsets."""
    E, N, K = 8, 4, 2
    subsets = list(itertools.combinations(range(E), K))
    miss = sum(1 for S in subsets if not any(e // (E // N) == 1 for e in S)) / len(subsets)
    assert V.zero_pair_probability(E, N, K, N) == pytest.approx(miss)
    assert V.zero_pair_probability(E, N, K, 3 * N) == pytest.approx(miss ** 3)


def test_zero_pair_fraction_matches_pages():
    """About 36% of chip pairs carry no traffic at EP=64, 512 tokens, top-8 of 256."""
    g = json.load(open(os.path.join(GOLD, "ep_layout_examples.json")))["zero_pairs"]
    cf = V.zero_pair_probability(256, 64, 8, 512)
    assert round(cf, 2) == g["printed_fraction"]
    cfg = CONFIGS["layout_ep64"]
    out = oracle.forward(cfg, make_inputs(cfg))
    z0 = V.zero_pair_fraction(out["dispatch"].send_bytes)
    assert abs(z0 - g["printed_fraction"]) < 0.02
    fr = []
    for seed in range(30):
        c = cfg.with_(seed=seed + 1)
        fr.append(V.zero_pair_fraction(oracle.forward(c, make_inputs(c))["dispatch"].send_bytes))
    # per-seed std is about 0.006 (4096 weakly dependent pairs); 30 seeds
    assert abs(np.mean(fr) - cf) < 0.004


def test_active_experts_uniform():
    """Exact expectation E/P (1-(1-K/E)^T) by simulation; the balls-into-bins form of
    eq. par-ep-active-experts is close to it (both near 162 at T=32, K=8, E=256)."""
    T, K, E = 32, 8, 256
    act = []
    for seed in range(300):
        keys = np.random.default_rng(seed).random((T, E))
        rr = oracle.route(K=K, score="softmax", logits=keys)
        act.append(len(np.unique(rr.ids)))
    exact = V.e_active_exact(E, 1, T, K)
    pois = V.e_active_poisson(E, 1, T, K)
    assert exact == pytest.approx(163.3, abs=0.05)
    assert pois == pytest.approx(161.8, abs=0.05)
    sd = np.std(act) / math.sqrt(len(act))
    assert abs(np.mean(act) - exact) < 4 * sd
    # per-chip form: P chips share the experts evenly
    assert V.e_active_exact(E, 8, T, K) == pytest.approx(exact / 8)


def test_balancedness():
    assert V.balancedness([1, 1, 1, 1]) == 1.0
    assert V.balancedness([4, 0, 0, 0]) == 0.25
    assert V.peak_to_mean([4, 0, 0, 0]) == 4.0
