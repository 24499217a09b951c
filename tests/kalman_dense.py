"""Textbook dense-covariance Kalman filter for a matrix-valued memory (test helper).

Model: the memory S (d_k x d_v) drifts as S <- D S with D = diag(a) plus
process noise of covariance diag(xi) on every column, and each token observes
v^T = k^T S + noise of variance r (page "给记忆装一个信任度探测器：Kalman Delta
Networks ...", section "把记忆问题重新想成一个滤波问题": hidden drifting key->value
map, each token a noisy observation; page "Kalman Delta Networks: Uncertainty-
aware Associative Memory", section "How It Works").  All d_v columns share one
d_k x d_k covariance P because they share the observation vector k.

Predict: S <- D S, P <- D P D + diag(xi).
Update:  s = k^T P k + r, g = P k / s, S <- S + g (v - S^T k)^T,
         P <- P - g (P k)^T.
"""
from __future__ import annotations

import numpy as np


def dense_kalman(S0, P0, a, xi, k, v, r, q=None):
    S = np.array(S0, np.float64)
    P = np.array(P0, np.float64)
    outs = []
    for t in range(k.shape[0]):
        D = np.diag(a[t])
        S = D @ S
        P = D @ P @ D + np.diag(xi[t])
        Pk = P @ k[t]
        s = float(k[t] @ Pk + r[t])
        g = Pk / s
        S = S + np.outer(g, v[t] - S.T @ k[t])
        P = P - np.outer(g, Pk)
        if q is not None:
            outs.append(S.T @ q[t])
    return S, P, (np.array(outs) if q is not None else None)
