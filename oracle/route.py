"""Router: scores, group limit, top-K selection and combine weights, in fp64.

Definitions followed:
  * The router computes, for every token, a score per expert and picks the top-K
    experts ([EP-overview] glossary entry "Router" and section "MoE 路由机制是什么？
    top-K 怎么用？"; [EP-concept] section "技術原理", step 1).
  * Group-limited routing: a token may only use experts inside its top-M expert
    groups ([EP-overview] glossary entry "Expert group").
  * The per-expert bias of aux-loss-free balancing only corrects the load, so it
    enters the selection key and not the weights ([EP-notes] section "负载均衡").
  * The combine weights are the routing weights of the selected experts
    ([EP-concept] section "技術原理", step 4).

Readings where the pages are silent (each is listed in the design notes):
  * softmax scoring: key = logit (= x W_r + bias); weights = softmax over all E,
    renormalised over the selected K (equal to a softmax over the selected logits).
  * sigmoid scoring: s = 1/(1+exp(-logit)), key = s + bias, weights = s / sum(s) over
    the selected K (bias excluded).
  * groups are contiguous blocks of E/G experts; a group's score is the sum of its
    two largest keys (its single key when E/G = 1); ties go to the lower group index.
  * ties between keys go to the lower expert index; ids are emitted in ascending
    expert-id order, weights aligned with them.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor (any device, any float dtype)
        a = a.detach().to("cpu")
        import torch
        a = a.to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


@dataclass
class RouteResult:
    ids: np.ndarray        # [T, K] int32, ascending expert ids per token
    weights: np.ndarray    # [T, K] float64, aligned with ids
    logits: np.ndarray     # [T, E] float64
    keys: np.ndarray       # [T, E] float64 selection keys (before group masking)
    kth_gap: np.ndarray    # [T] key gap between the K-th and (K+1)-th allowed expert
    group_gap: np.ndarray  # [T] score gap between the M-th and (M+1)-th group (inf if off)


def router_logits(x, w_router, bias=None, score="softmax"):
    """L = x W_r^T in fp64 (W_r stored [E, h], one row per expert); softmax scoring adds
    the bias into the logit itself."""
    L = _f64(x) @ _f64(w_router).T
    if score == "softmax" and bias is not None:
        L = L + _f64(bias)[None, :]
    return L


def _order_desc(vals):
    """Indices sorted by decreasing value, ties by increasing index."""
    idx = np.arange(vals.shape[0])
    return np.lexsort((idx, -vals))


def route(*, K, score="softmax", renorm=True, n_groups=1, topk_groups=1, bias=None,
          x=None, w_router=None, logits=None) -> RouteResult:
    """Route T tokens: either from (x, w_router) or from given logits [T, E]."""
    if logits is None:
        L = router_logits(x, w_router, bias, score)
    else:
        L = _f64(logits)
        if score == "softmax" and bias is not None:
            L = L + _f64(bias)[None, :]
    T, E = L.shape
    b = _f64(bias) if bias is not None else np.zeros(E)
    if score == "softmax":
        keys = L.copy()
        m = L.max(axis=1, keepdims=True)
        p = np.exp(L - m)
        p = p / p.sum(axis=1, keepdims=True)          # full softmax over E
        raw = p
    elif score == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-L))
        keys = s + b[None, :]
        raw = s
    else:
        raise ValueError(score)

    group_limited = n_groups > 1 and topk_groups < n_groups
    gsz = E // n_groups
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float64)
    kgap = np.full(T, np.inf)
    ggap = np.full(T, np.inf)
    for t in range(T):
        key = keys[t]
        allowed = np.ones(E, bool)
        if group_limited:
            gscore = np.empty(n_groups)
            for g in range(n_groups):
                top = np.sort(key[g * gsz:(g + 1) * gsz])[::-1]
                gscore[g] = top[:2].sum()
            gorder = _order_desc(gscore)
            ggap[t] = gscore[gorder[topk_groups - 1]] - gscore[gorder[topk_groups]]
            allowed[:] = False
            for g in gorder[:topk_groups]:
                allowed[g * gsz:(g + 1) * gsz] = True
        cand = np.nonzero(allowed)[0]
        order = cand[_order_desc(key[cand])]
        sel = order[:K]
        if len(order) > K:
            kgap[t] = key[order[K - 1]] - key[order[K]]
        sel = np.sort(sel)
        ids[t] = sel
        r = raw[t, sel]
        w[t] = r / r.sum() if renorm else r
    return RouteResult(ids=ids, weights=w, logits=L, keys=keys, kth_gap=kgap, group_gap=ggap)
