"""GPU parity of moe_layout_stats (token fan-out, distinct tokens per rank pair, per-rank
loads) against the oracle's layout statistics, bit-exact, and of the Monte Carlo
busiest-rank estimate trial by trial."""
import numpy as np
import pytest
import torch

import oracle
import expert_routing_amd as moe
from oracle import layout as LY
from synth import CONFIGS
from gpu_cases import gpu_inputs, np_, run_stages

pytestmark = pytest.mark.gpu

BASE = CONFIGS["mixtral_prefill"]
CASES = {
    "layout_ep64": CONFIGS["layout_ep64"],
    # capacity drops spread over 4 ranks
    "skew_cap_ep4": CONFIGS["skew_cap1"].with_(T=1024, h=128, E=64, K=6, inter=64, n_ep=4),
    "groups_ep8": CONFIGS["dsv3_ep8"].with_(T=512, h=256, E=64, K=6, inter=64, shared_inter=64),
    "tiny_f32_ep2": CONFIGS["tiny_f32"].with_(n_ep=2),
}


def _stats(p, ids, E, N, K):
    i64 = dict(dtype=torch.int64, device="cuda")
    out = dict(tokens_to=torch.full((N, N), -7, **i64), recv=torch.full((N,), -7, **i64),
               hist=torch.full((K + 1,), -7, **i64), busiest=torch.full((1,), -7, **i64))
    ws = torch.empty(moe.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    moe.moe_layout_stats(p, ids, out["tokens_to"], out["recv"], out["hist"], out["busiest"], ws)
    torch.cuda.synchronize()
    return {k: np_(v) for k, v in out.items()}


@pytest.mark.parametrize("name", list(CASES))
def test_layout_stats_match_oracle(name):
    cfg = CASES[name]
    print(f"[case] layout stats {name}", flush=True)
    inp = gpu_inputs(cfg)
    p, b = run_stages(cfg, inp)
    ids = np_(b["topk_ids"]).astype(np.int64)
    d = oracle.dispatch(ids, E=cfg.E, n_ep=cfg.n_ep, ep_rank=cfg.ep_rank,
                        capacity_factor=cfg.capacity_factor, pad=cfg.pad, h=cfg.h,
                        dtype_size=cfg.act_bytes)
    ref = LY.layout_stats(ids, d.kept, cfg.E, cfg.n_ep)
    got = _stats(p, b["topk_ids"], cfg.E, cfg.n_ep, cfg.K)
    np.testing.assert_array_equal(got["tokens_to"], ref.tokens_to)
    np.testing.assert_array_equal(got["recv"], ref.recv_pairs)
    np.testing.assert_array_equal(got["hist"], ref.fanout_hist)
    assert got["busiest"][0] == ref.recv_pairs.max()
    # the same layout as dispatch's pair counts
    n = np_(b["send_bytes"]).astype(np.int64) // (cfg.h * cfg.act_bytes)
    assert (got["tokens_to"] <= n).all() and (got["recv"] == n.sum(axis=0)).all()
    f = np.repeat(np.arange(cfg.K + 1), got["hist"])
    print(f"[layout] {name}: mean token fan-out {f.mean():.3f} ranks, busiest rank "
          f"{got['busiest'][0]} pairs (mean {got['recv'].mean():.1f})", flush=True)


def test_busiest_rank_monte_carlo_matches_oracle():
    # uniform random top-8 of 256 experts over 64 ranks, 512 tokens (the pages' example)
    T, E, K, P, trials = 512, 256, 8, 64, 6
    keys = np.random.default_rng(7).random((trials, T, E)).astype(np.float32)
    ref = LY.busiest_chip_loads(keys, K, E, P)
    p = moe.Problem(T=T, h=64, E=E, K=K, n_ep=P, inter=0)
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    got = []
    for tr in range(trials):
        moe.moe_select(p, torch.from_numpy(keys[tr]).cuda(), None, ids, w)
        got.append(_stats(p, ids, E, P, K)["busiest"][0])
    np.testing.assert_array_equal(np.asarray(got), ref)
    mean, q99 = LY.busiest_chip_estimate(ref)
    print(f"[layout] busiest of 64 ranks: mean {mean:.1f} pairs, 99% bound {q99:.1f} "
          f"(a rank's mean load {T * K / P:.0f})", flush=True)
