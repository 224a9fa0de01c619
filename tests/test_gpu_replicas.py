"""GPU parity of the replica map: moe_dispatch_replicated bit-exact against the oracle's
replicated dispatch (run on the GPU's own routing), and moe_forward_replicated's output
against the fp64 oracle built from that dispatch."""
import numpy as np
import pytest
import torch

import expert_routing_amd as moe
import oracle
from oracle import replicas as RP
from synth import CONFIGS
from gpu_cases import TOL, cpu_inputs, gpu_inputs, np_, rel_errors, run_stages

pytestmark = pytest.mark.gpu

CASES = {
    # Zipf skew over 64 experts, 8 ranks, 16 redundant, with and without capacity
    "skew_ep8": (CONFIGS["skew_nodrop"].with_(T=1024, h=128, E=64, K=6, inter=64, n_ep=8,
                                              ep_rank=3), 16),
    "skew_ep8_cap": (CONFIGS["skew_cap1"].with_(T=1024, h=128, E=64, K=6, inter=64, n_ep=8,
                                                ep_rank=0), 16),
    # the pages' 256 logical + 32 redundant = 288 physical, group-limited sigmoid routing
    "dsv3_288": (CONFIGS["dsv3_ep8"].with_(T=512, h=256, inter=64, shared_inter=64, n_ep=8,
                                           ep_rank=5), 32),
    # one rank: replicas split hot experts into several groups of the grouped GEMM
    "mixtral_1rank": (CONFIGS["mixtral_prefill"].with_(T=600, h=256, inter=128), 8),
}


def _plan(cfg, ids, R):
    load = np.bincount(ids.reshape(-1), minlength=cfg.E)
    return moe.replica_plan(cfg.E, R, cfg.n_ep, load), load


@pytest.mark.parametrize("name", list(CASES))
def test_dispatch_replicated_exact(name):
    cfg, R = CASES[name]
    print(f"[case] replicated dispatch {name}", flush=True)
    inp = gpu_inputs(cfg)
    p, b = run_stages(cfg, inp)                      # routing on the GPU
    ids = np_(b["topk_ids"]).astype(np.int64)
    plan, _ = _plan(cfg, ids, R)
    rp = RP.plan(np.bincount(ids.reshape(-1), minlength=cfg.E), R, cfg.n_ep)
    rmap = moe.DeviceReplicaMap(plan)
    P = rmap.P
    rb = moe.alloc_buffers_replicated(p, P)
    moe.moe_dispatch_replicated(p, rmap, b["topk_ids"], rb["counts"], rb["phys_counts"],
                                rb["offsets"], rb["dest_row"], rb["row_src"], rb["send_bytes"],
                                rb["n_dropped"], rb["ws"])
    torch.cuda.synchronize()
    ref = RP.dispatch_replicated(ids, rp, E=cfg.E, n_ep=cfg.n_ep, ep_rank=cfg.ep_rank,
                                 capacity_factor=cfg.capacity_factor, h=cfg.h,
                                 dtype_size=cfg.act_bytes)
    np.testing.assert_array_equal(np_(rb["counts"]), ref.counts)
    np.testing.assert_array_equal(np_(rb["phys_counts"]), ref.phys_counts)
    np.testing.assert_array_equal(np_(rb["offsets"]), ref.offsets)
    np.testing.assert_array_equal(np_(rb["dest_row"]), ref.dest_row)
    np.testing.assert_array_equal(np_(rb["row_src"])[:len(ref.row_src)], ref.row_src)
    np.testing.assert_array_equal(np_(rb["send_bytes"]), ref.send_bytes)
    assert int(np_(rb["n_dropped"])[0]) == ref.n_dropped
    base = oracle.dispatch(ids, E=cfg.E, n_ep=cfg.n_ep, capacity_factor=cfg.capacity_factor,
                           h=cfg.h, dtype_size=cfg.act_bytes)
    b0 = oracle.volumes.balancedness(base.n_pairs.sum(0))
    b1 = oracle.volumes.balancedness(ref.rank_loads)
    print(f"[replicas] {name}: P={P}, rank balancedness {b0:.3f} -> {b1:.3f}", flush=True)


@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("name", list(CASES))
def test_forward_replicated(name, gather):
    cfg, R = CASES[name]
    print(f"[case] replicated forward {name} gather={gather}", flush=True)
    El = cfg.E_local
    # every logical expert's weights (each physical expert runs its logical one's)
    full = cfg.with_(n_ep=1, ep_rank=0)
    inp = gpu_inputs(cfg)
    w_all = gpu_inputs(full)
    p = moe.problem_from_config(cfg)
    b0 = moe.alloc_buffers(p, "cuda")
    moe.moe_route(p, inp["x"], inp["w_router"], inp["bias"], b0["topk_ids"], b0["topk_w"], b0["ws"])
    torch.cuda.synchronize()
    ids = np_(b0["topk_ids"]).astype(np.int64)
    plan, load = _plan(cfg, ids, R)
    rmap = moe.DeviceReplicaMap(plan)
    rb = moe.alloc_buffers_replicated(p, rmap.P)
    t = dict(rb)
    t.update(x=inp["x"], w_router=inp["w_router"], bias=inp["bias"], w13=w_all["w13"],
             w2=w_all["w2"], w13_sh=inp["w13_sh"], w2_sh=inp["w2_sh"])
    if gather:
        t["xp"] = None
    moe.moe_forward_replicated(p, rmap, t, rb["ws"])
    torch.cuda.synchronize()
    assert torch.equal(rb["topk_ids"], b0["topk_ids"])
    # reference: the oracle's replicated dispatch of these ids, fp64 FFN of each kept local
    # pair with its logical expert's weights, the oracle's routing weights
    rp = RP.plan(load, R, cfg.n_ep)
    d = RP.dispatch_replicated(ids, rp, E=cfg.E, n_ep=cfg.n_ep, ep_rank=cfg.ep_rank,
                               capacity_factor=cfg.capacity_factor, h=cfg.h,
                               dtype_size=cfg.act_bytes)
    c = cpu_inputs(inp)
    rr = oracle.route(K=cfg.K, score=cfg.score, renorm=cfg.renorm, n_groups=cfg.n_groups,
                      topk_groups=cfg.topk_groups, bias=c["bias"], x=c["x"],
                      w_router=c["w_router"])
    flipped = (rr.ids != ids).any(axis=1)
    x64 = c["x"].double().numpy()
    w13 = w_all["w13"].cpu().double().numpy()
    w2 = w_all["w2"].cpu().double().numpy()
    y_ref = np.zeros((cfg.T, cfg.h))
    Pl = rmap.P // cfg.n_ep
    for t_ in range(cfg.T):
        for k in range(cfg.K):
            pid = int(d.phys_of_pair[t_, k])
            if d.kept[t_, k] and cfg.ep_rank * Pl <= pid < (cfg.ep_rank + 1) * Pl:
                e = int(ids[t_, k])
                y_ref[t_] += rr.weights[t_, k] * oracle.swiglu_ffn(x64[t_:t_ + 1], w13[e], w2[e])[0]
    if cfg.n_shared:
        tpr = cfg.T // cfg.n_ep
        t0 = cfg.ep_rank * tpr
        y_ref[t0:t0 + tpr] += oracle.shared_ffn(x64, c["w13_sh"], c["w2_sh"], t0, t0 + tpr)
    ok = ~flipped
    mx, mean, zexact = rel_errors(np_(rb["y"])[ok], y_ref[ok])
    print(f"[parity] replicated {name}: y max_rel {mx:.3e} mean_rel {mean:.3e} "
          f"({int(flipped.sum())} flipped)", flush=True)
    tmax, tmean = TOL[cfg.dtype]
    assert mx <= tmax and mean <= tmean and zexact
