"""Combine: results return to token order and are summed with the routing weights
([EP-concept] "技術原理", step 4; [EP-overview] glossary "Combine" and "Dispatch 和
Combine 各做什么？").

  y[t] = sum over k = 0..K-1 of [dest_row[t,k] >= 0] * w[t,k] * yp[dest_row[t,k]]
         + [t0 <= t < t1] * ysh[t - t0]
in fp64, k ascending. Dropped or remote pairs add nothing (no renormalisation).
"""
from __future__ import annotations

import numpy as np

from .route import _f64


def combine(yp, dest_row, weights, ysh=None, t0=0):
    yp = _f64(yp)
    w = _f64(weights)
    dest_row = np.asarray(dest_row)
    T, K = dest_row.shape
    y = np.zeros((T, yp.shape[1]), np.float64)
    for t in range(T):
        for k in range(K):
            r = int(dest_row[t, k])
            if r >= 0:
                y[t] += w[t, k] * yp[r]
    if ysh is not None:
        ysh = _f64(ysh)
        y[t0:t0 + ysh.shape[0]] += ysh
    return y
