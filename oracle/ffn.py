"""Expert FFN in fp64: each expert is an independent feed-forward network applied to the
rows dispatched to it ([EP-concept] "技術原理", step 3; [EP-notes] "MoE 结构回顾"), and a
shared expert sees every local token ([EP-overview] glossary "Expert": DeepSeek-V3 has
256 routed experts plus one shared expert per layer).

Reading: the FFN is SwiGLU, the form the workloads name:
  a = xp W_g^T,  b = xp W_u^T,  H = silu(a) * b = a / (1 + exp(-a)) * b,  y = H W_d^T,
with w13 = [W_g; W_u] stored [2I, h] (gate rows first) and w2 = W_d stored [h, I].
No intermediate rounding.
"""
from __future__ import annotations

import numpy as np

from .route import _f64


def swiglu_ffn(xrows, w13, w2):
    """One expert on its rows: fp64 throughout."""
    xrows = _f64(xrows)
    w13 = _f64(w13)
    w2 = _f64(w2)
    inter = w13.shape[0] // 2
    a = xrows @ w13[:inter].T
    b = xrows @ w13[inter:].T
    H = a / (1.0 + np.exp(-a)) * b
    return H @ w2.T


def expert_ffn(xp, offsets, w13, w2, experts=None):
    """yp[rows of local expert e] = FFN_e(xp rows); rows past offsets[-1] stay zero.

    `w13[e]` / `w2[e]` may be any indexable yielding one expert's weights (so large
    weight sets can be fetched one expert at a time). `experts` restricts the local
    experts evaluated (rows of the others are left zero)."""
    xp = _f64(xp)
    yp = np.zeros((xp.shape[0], w2[0].shape[0]) if xp.ndim == 2 else xp.shape, np.float64)
    El = len(offsets) - 1
    for el in range(El) if experts is None else experts:
        lo, hi = int(offsets[el]), int(offsets[el + 1])
        if hi > lo:
            yp[lo:hi] = swiglu_ffn(xp[lo:hi], w13[el], w2[el])
    return yp


def shared_ffn(x, w13_sh, w2_sh, t0, t1):
    """Shared expert on the local token block x[t0:t1]."""
    return swiglu_ffn(_f64(x)[t0:t1], w13_sh, w2_sh)
