"""One MoE layer forward in fp64: route -> dispatch -> expert FFN -> combine
([EP-overview] section "MoE 路由机制是什么？top-K 怎么用？": router, dispatch, expert
compute, combine; [EP-wiki] "核心思想" forward flow), on one rank's share:

  * all T tokens are routed (they stand in for every virtual rank's router);
  * dispatch keeps this rank's local experts [r E/N, (r+1) E/N);
  * the shared expert runs on this rank's token block [r T/N, (r+1) T/N);
  * combine gives, for every token, the sum over this rank's experts (the rows that
    would be sent back), plus the shared expert's output on the local block.
"""
from __future__ import annotations

import numpy as np

from .combine import combine
from .dispatch import dispatch, permute
from .ffn import expert_ffn, shared_ffn
from .route import _f64, route


def forward(cfg, inp, experts=None):
    """Every intermediate result of the layer for workload `cfg` and inputs `inp`
    (as made by synth.make_inputs, on any device)."""
    T = inp["T"]
    if cfg.keys == "uniform":
        rr = route(K=cfg.K, score=cfg.score, renorm=cfg.renorm, n_groups=cfg.n_groups,
                   topk_groups=cfg.topk_groups, bias=inp["bias"], logits=inp["keys"])
    else:
        rr = route(K=cfg.K, score=cfg.score, renorm=cfg.renorm, n_groups=cfg.n_groups,
                   topk_groups=cfg.topk_groups, bias=inp["bias"], x=inp["x"],
                   w_router=inp["w_router"])
    d = dispatch(rr.ids, E=cfg.E, n_ep=cfg.n_ep, ep_rank=cfg.ep_rank,
                 capacity_factor=cfg.capacity_factor, pad=cfg.pad, h=cfg.h,
                 dtype_size=cfg.act_bytes)
    out = {"route": rr, "dispatch": d}
    if cfg.inter == 0 or inp.get("w13") is None:
        return out
    x = _f64(inp["x"])
    xp = permute(x, d, cfg.K)
    yp = expert_ffn(xp, d.offsets, inp["w13"], inp["w2"], experts=experts)
    ysh, t0 = None, 0
    if cfg.n_shared:
        tpr = T // cfg.n_ep
        t0 = cfg.ep_rank * tpr
        ysh = shared_ffn(x, inp["w13_sh"], inp["w2_sh"], t0, t0 + tpr)
    y = combine(yp, d.dest_row, rr.weights, ysh, t0)
    out.update(xp=xp, yp=yp, ysh=ysh, y=y)
    return out
