"""Chunk-parallel form of the recurrence, fp64 numpy (test helper).

An independent formulation used to pin the oracle: within a chunk of C tokens
the delta dependence is resolved by a causal triangular solve on provisional
errors, with interaction matrices that carry the cumulative decay (page
"معماری KDA: حذف تداخل حافظه با قانون دلتا در توالی‌های بلند", section "حل
مشکل وابستگی علی"; that section states the chunked output equals the serial
recurrence exactly).  Derivation, per chunk starting from state S0:

    S_t = G_t S0 + sum_{s<=t} diag(gamma_t / gamma_s) w_s e_s^T
    (I + A_kk) E = V - K~ S0,     A_kk[t,s] = sum_i k_ti w_si D_tsi  (s < t)
    O = Q~ S0 + A_qk E,           A_qk[t,s] = sum_i q_ti w_si D_tsi  (s <= t)
    S_C = diag(gamma_C) S0 + W~^T E

with D_tsi = prod_{s<r<=t} a_ri, gamma_t = prod_{r<=t} a_r, K~ = gamma (.) K,
Q~ = gamma (.) Q, W~_s = D_{C,s} (.) w_s.  The diagonal-KDN write vectors come
from the per-channel variance recursion, the isotropic-KDN ones from the
per-head scalar recursion; neither depends on S.
"""
from __future__ import annotations

import numpy as np


def chunk_form(variant, q, k, v, alpha=None, beta=None, xi=None, r=None,
               S0=None, p0=None, mu=1.0, C=8):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    Sout = np.zeros((B, H, dk, dv))
    pout = (np.zeros((B, H, dk)) if variant == "diag_kdn" else
            np.zeros((B, H)) if variant == "iso_kdn" else None)
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], np.float64)
            p = (np.array(p0[b, h], np.float64) if variant in ("diag_kdn", "iso_kdn")
                 else None)
            for c0 in range(0, T, C):
                L = min(C, T - c0)
                sl = slice(c0, c0 + L)
                K, Q, V = k[b, sl, h], q[b, sl, h], v[b, sl, h]
                if variant == "deltanet":
                    a = np.ones((L, dk))
                elif variant == "gated_deltanet":
                    a = np.repeat(np.asarray(alpha[b, sl, h], np.float64)[:, None],
                                  dk, axis=1)
                else:
                    a = np.asarray(alpha[b, sl, h], np.float64)
                W = np.zeros((L, dk))
                if variant == "diag_kdn":
                    for t in range(L):
                        pm = a[t] ** 2 * p + xi[b, c0 + t, h]
                        rt = float(r[b, c0 + t, h])
                        s = rt + np.sum(pm * K[t] ** 2)
                        W[t] = pm * K[t] / s if s != 0 else 0.0
                        den = rt + mu * pm * K[t] ** 2
                        p = np.where(den != 0, pm * rt / np.where(den != 0, den, 1), pm)
                elif variant == "iso_kdn":
                    for t in range(L):
                        pm = np.mean(a[t] ** 2) * p + np.mean(xi[b, c0 + t, h])
                        rt = float(r[b, c0 + t, h])
                        kk = float(K[t] @ K[t])
                        s = rt + pm * kk
                        W[t] = pm * K[t] / s if s != 0 else 0.0
                        den = rt + mu / dk * pm * kk
                        p = pm * rt / den if den != 0 else pm
                else:
                    W = np.asarray(beta[b, sl, h], np.float64)[:, None] * K
                # pairwise decay D[t, s] = prod_{s < r <= t} a_r  (s <= t)
                D = np.zeros((L, L, dk))
                for s_ in range(L):
                    run = np.ones(dk)
                    D[s_, s_] = run
                    for t in range(s_ + 1, L):
                        run = run * a[t]
                        D[t, s_] = run
                gam = np.cumprod(a, axis=0)
                Akk = np.einsum("ti,si,tsi->ts", K, W, D) * np.tril(np.ones((L, L)), -1)
                Aqk = np.einsum("ti,si,tsi->ts", Q, W, D) * np.tril(np.ones((L, L)), 0)
                Kt, Qt = gam * K, gam * Q
                E = np.linalg.solve(np.eye(L) + Akk, V - Kt @ S)
                o[b, sl, h] = Qt @ S + Aqk @ E
                Wt = D[L - 1] * W
                S = gam[L - 1][:, None] * S + Wt.T @ E
            Sout[b, h] = S
            if p is not None:
                pout[b, h] = p
    return o, Sout, pout
