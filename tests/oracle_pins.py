"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` takes a recurrence callable with the signature of
``oracle.recurrence`` and raises AssertionError if the oracle breaks the fact
it checks.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutations.py`` runs them on oracle builds with planted mistakes
and requires every mistake to be caught.

Pages cited:
  [TAB] "Внимание в LLM · часть 11 -- Память с поправкой"
  [KDA] "معماری KDA: حذف تداخل حافظه با قانون دلتا در توالی‌های بلند"
  [KDN] "给记忆装一个信任度探测器：Kalman Delta Networks 如何让AI知道自己"记得准不准""
  [AFS] "Kalman Delta Networks: Uncertainty-aware Associative Memory"
"""
from __future__ import annotations

import json
import os

import numpy as np

from chunk_form import chunk_form
from kalman_dense import dense_kalman

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _orthonormal(n, d, seed):
    a = _rng(seed).standard_normal((d, n))
    qm, _ = np.linalg.qr(a)
    return qm.T


def _random_inputs(variant, B, T, H, dk, dv, seed, s0=True, kdn_p0=None):
    g = _rng(seed)
    inp = dict(q=g.standard_normal((B, T, H, dk)),
               k=_unit(g.standard_normal((B, T, H, dk))),
               v=g.standard_normal((B, T, H, dv)))
    if variant == "gated_deltanet":
        inp["alpha"] = g.uniform(0.3, 1.0, (B, T, H))
    elif variant in ("kda", "diag_kdn", "iso_kdn"):
        inp["alpha"] = g.uniform(0.3, 1.0, (B, T, H, dk))
    if variant not in ("diag_kdn", "iso_kdn"):
        inp["beta"] = g.uniform(0.05, 1.0, (B, T, H))
    else:
        pshape = (B, H, dk) if variant == "diag_kdn" else (B, H)
        inp["xi"] = g.uniform(0.0, 0.2, (B, T, H, dk))
        inp["r"] = g.uniform(0.2, 2.0, (B, T, H))
        inp["p0"] = (g.uniform(0.3, 2.0, pshape) if kdn_p0 is None
                     else np.full(pshape, kdn_p0))
    if s0:
        inp["S0"] = 0.5 * g.standard_normal((B, H, dk, dv))
    return inp


# ---------------------------------------------------------------------------
# Delta rule: exact replacement ([KDA] "تکامل قانون دلتا": beta = 1 makes the
# memory return exactly v for that key; [TAB] read / compare / correct).
# ---------------------------------------------------------------------------
def pin_recall_orthonormal(rec):
    """beta = 1, orthonormal keys: every written key reads back its value;
    with q_t = k_t the output at t is v_t."""
    dk = dv = 16
    T = 12
    keys = _orthonormal(T, dk, seed=1)
    g = _rng(2)
    vals = g.standard_normal((T, dv))
    S0 = g.standard_normal((1, 1, dk, dv))
    k = keys[None, :, None, :]
    v = vals[None, :, None, :]
    o, S, _ = rec("deltanet", k, k, v, beta=np.ones((1, T, 1)), S0=S0)
    np.testing.assert_allclose(o[0, :, 0], vals, atol=1e-12)
    np.testing.assert_allclose(keys @ S[0, 0], vals, atol=1e-12)


def pin_recall_latest_value(rec):
    """A key written twice returns the latest value, not the mix (golden
    fixture: the Riga -> Prague example of [TAB])."""
    with open(os.path.join(GOLDEN, "delta_rule_overwrite.json")) as f:
        fx = json.load(f)
    key = np.array(fx["key"], np.float64)
    v_old = np.array(fx["value_old"], np.float64)
    v_new = np.array(fx["value_new"], np.float64)
    others = np.array(fx["other_keys"], np.float64)
    other_vals = np.array(fx["other_values"], np.float64)
    ks = np.concatenate([[key], others, [key]])
    vs = np.concatenate([[v_old], other_vals, [v_new]])
    T, d = ks.shape
    qs = np.repeat(key[None], T, axis=0)
    o, S, _ = rec("deltanet", qs[None, :, None], ks[None, :, None],
                  vs[None, :, None], beta=np.ones((1, T, 1)))
    np.testing.assert_allclose(o[0, -1, 0], fx["expected_delta_read"], atol=1e-12)
    np.testing.assert_allclose(o[0, 0, 0], fx["value_old"], atol=1e-12)


# ---------------------------------------------------------------------------
# Reductions between variants ([KDA] "از فراموشی کلی به فراموشی جزئی").
# ---------------------------------------------------------------------------
def pin_gdn_alpha_one_is_deltanet(rec):
    B, T, H, d = 2, 20, 3, 8
    inp = _random_inputs("deltanet", B, T, H, d, d, seed=3)
    o1, S1, _ = rec("deltanet", **inp)
    o2, S2, _ = rec("gated_deltanet", alpha=np.ones((B, T, H)), **inp)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def pin_kda_equal_entries_is_gdn(rec):
    B, T, H, d = 2, 20, 3, 8
    inp = _random_inputs("gated_deltanet", B, T, H, d, d, seed=4)
    o1, S1, _ = rec("gated_deltanet", **inp)
    inp2 = dict(inp)
    inp2["alpha"] = np.repeat(inp["alpha"][..., None], d, axis=-1)
    o2, S2, _ = rec("kda", **inp2)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S1, S2, rtol=0, atol=1e-13)


def pin_scalar_decay_closed_form(rec):
    """beta = 0: nothing is written, so S_T = (prod alpha) S0 and
    o_t = (prod_{r<=t} alpha_r) S0^T q_t (scalar and per-channel decay)."""
    B, T, H, d = 1, 9, 2, 6
    inp = _random_inputs("kda", B, T, H, d, d, seed=5)
    inp["beta"] = np.zeros((B, T, H))
    o, S, _ = rec("kda", **inp)
    gam = np.cumprod(inp["alpha"], axis=1)           # [B,T,H,d]
    for h in range(H):
        for t in range(T):
            ref = (gam[0, t, h][:, None] * inp["S0"][0, h]).T @ inp["q"][0, t, h]
            np.testing.assert_allclose(o[0, t, h], ref, atol=1e-12)
        np.testing.assert_allclose(S[0, h], gam[0, -1, h][:, None] * inp["S0"][0, h],
                                   atol=1e-12)


def pin_alpha_zero_erases(rec):
    """alpha = 0 on every channel at token t: the memory before t is erased, so
    after t the state is exactly w_t v_t^T (KDA: one channel can be fully
    cleared while another is kept)."""
    B, T, H, d = 1, 4, 1, 5
    inp = _random_inputs("kda", B, T, H, d, d, seed=6)
    inp["alpha"][0, 3, 0, :] = 0.0
    o, S, _ = rec("kda", **inp)
    w = inp["beta"][0, 3, 0] * inp["k"][0, 3, 0]
    np.testing.assert_allclose(S[0, 0], np.outer(w, inp["v"][0, 3, 0]), atol=1e-12)
    # Only channel 2 cleared: rows other than 2 keep their decayed history.
    inp2 = _random_inputs("kda", B, 1, H, d, d, seed=7)
    inp2["alpha"][0, 0, 0, :] = 1.0
    inp2["alpha"][0, 0, 0, 2] = 0.0
    inp2["beta"][:] = 0.0
    _, S2, _ = rec("kda", **inp2)
    np.testing.assert_array_equal(S2[0, 0, 2], np.zeros(d))
    np.testing.assert_allclose(np.delete(S2[0, 0], 2, axis=0),
                               np.delete(inp2["S0"][0, 0], 2, axis=0), atol=0)


# ---------------------------------------------------------------------------
# Chunked == serial ([KDA] "حل مشکل وابستگی علی").
# ---------------------------------------------------------------------------
def pin_chunk_form(rec):
    for variant in ("deltanet", "gated_deltanet", "kda", "diag_kdn", "iso_kdn"):
        for T, C in ((24, 8), (21, 8), (5, 8)):
            inp = _random_inputs(variant, 2, T, 2, 8, 6, seed=10 + T)
            mu = 3.0 if variant in ("diag_kdn", "iso_kdn") else 1.0
            o1, S1, p1 = rec(variant, mu=mu, **inp)
            o2, S2, p2 = chunk_form(variant, mu=mu, C=C, **inp)
            np.testing.assert_allclose(o1, o2, atol=1e-11, rtol=1e-11)
            np.testing.assert_allclose(S1, S2, atol=1e-11, rtol=1e-11)
            if p1 is not None:
                np.testing.assert_allclose(p1, p2, atol=1e-13, rtol=1e-12)


# ---------------------------------------------------------------------------
# Diagonal KDN against the textbook Kalman filter ([KDN] filtering and
# diagonal sections; [AFS] "Approximation 1").
# ---------------------------------------------------------------------------
def _kdn_case(T, d, seed, onehot):
    g = _rng(seed)
    if onehot:
        idx = g.integers(0, d, T)
        k = np.eye(d)[idx]
    else:
        k = _unit(g.standard_normal((T, d)))
    return dict(k=k, q=g.standard_normal((T, d)), v=g.standard_normal((T, d)),
                a=g.uniform(0.5, 1.0, (T, d)), xi=g.uniform(0.0, 0.3, (T, d)),
                r=g.uniform(0.2, 1.5, T), S0=g.standard_normal((d, d)),
                p0=g.uniform(0.2, 2.0, d))


def _kdn_rec(rec, c, mu=1.0, T=None):
    T = c["k"].shape[0] if T is None else T
    sl = slice(0, T)
    o, S, p = rec("diag_kdn", c["q"][None, sl, None], c["k"][None, sl, None],
                  c["v"][None, sl, None], alpha=c["a"][None, sl, None],
                  xi=c["xi"][None, sl, None], r=c["r"][None, sl, None],
                  S0=c["S0"][None, None], p0=c["p0"][None, None], mu=mu)
    return o[0, :, 0], S[0, 0], p[0, 0]


def pin_kdn_onehot_is_dense_kalman(rec):
    """One-hot keys keep the exact posterior covariance diagonal, so diagonal
    KDN with mu = 1 is the exact Kalman filter: same memory, outputs and
    variances."""
    c = _kdn_case(T=30, d=6, seed=20, onehot=True)
    o, S, p = _kdn_rec(rec, c)
    S_ref, P_ref, o_ref = dense_kalman(c["S0"], np.diag(c["p0"]), c["a"], c["xi"],
                                       c["k"], c["v"], c["r"], q=c["q"])
    np.testing.assert_allclose(S, S_ref, atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(p, np.diag(P_ref), atol=1e-13, rtol=1e-12)
    np.testing.assert_allclose(P_ref, np.diag(np.diag(P_ref)), atol=1e-15)


def pin_kdn_mean_exact_one_step(rec):
    """From a diagonal prior, one diagonal-KDN step moves the memory exactly as
    the dense Kalman filter does, for any key (the projection only touches the
    covariance; the mean is exact)."""
    for seed in range(21, 26):
        c = _kdn_case(T=1, d=7, seed=seed, onehot=False)
        o, S, _ = _kdn_rec(rec, c, mu=2.5)
        S_ref, _, o_ref = dense_kalman(c["S0"], np.diag(c["p0"]), c["a"], c["xi"],
                                       c["k"], c["v"], c["r"], q=c["q"])
        np.testing.assert_allclose(S, S_ref, atol=1e-12, rtol=1e-12)
        np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=1e-12)


def pin_kdn_mean_field_precision(rec):
    """With any key, the projected precision of channel i is the diagonal of
    the exact posterior precision scaled as stated: 1/p+ = 1/p- + mu k_i^2/r."""
    for mu in (1.0, 4.0):
        c = _kdn_case(T=1, d=7, seed=27, onehot=False)
        _, _, p = _kdn_rec(rec, c, mu=mu)
        pm = c["a"][0] ** 2 * c["p0"] + c["xi"][0]
        Lam = np.diag(1.0 / pm) + np.outer(c["k"][0], c["k"][0]) / c["r"][0]
        prec = 1.0 / pm + mu * (np.diag(Lam) - 1.0 / pm)
        np.testing.assert_allclose(p, 1.0 / prec, rtol=1e-13)


def pin_kdn_closed_form(rec):
    """alpha = 1, xi = 0, one key e_i observed n times with noise r_j: the
    Gaussian-conjugate posterior gives p_n = 1/(1/p0 + mu sum 1/r_j) and, from
    S0 = 0 with mu = 1, row i of S equals sum(v_j/r_j) / (1/p0 + sum 1/r_j)."""
    d, n, i = 5, 7, 2
    g = _rng(30)
    rs = g.uniform(0.1, 3.0, n)
    vs = g.standard_normal((n, d))
    k = np.zeros((n, d))
    k[:, i] = 1.0
    p0 = np.full(d, 1.7)
    for mu in (1.0, 3.0):
        o, S, p = rec("diag_kdn", np.zeros((1, n, 1, d)), k[None, :, None],
                      vs[None, :, None], alpha=np.ones((1, n, 1, d)),
                      xi=np.zeros((1, n, 1, d)), r=rs[None, :, None],
                      p0=p0[None, None], mu=mu)
        np.testing.assert_allclose(p[0, 0, i], 1.0 / (1.0 / p0[i] + mu * np.sum(1.0 / rs)),
                                   rtol=1e-13)
        np.testing.assert_allclose(np.delete(p[0, 0], i), np.delete(p0, i), rtol=1e-15)
        if mu == 1.0:
            ref = (vs / rs[:, None]).sum(0) / (1.0 / p0[i] + np.sum(1.0 / rs))
            np.testing.assert_allclose(S[0, 0, i], ref, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(np.delete(S[0, 0], i, axis=0), 0.0, atol=0)


def pin_kdn_isotropic_is_delta(rec):
    """p0 = c 1, alpha = 1, xi = 0, |k| = 1: the first KDN write equals a
    DeltaNet write with beta = c/(c + r), for any mu ([AFS] "Why It Matters":
    the delta rule uses a token-wise isotropic stand-in for the covariance)."""
    g = _rng(31)
    d, c, r = 9, 0.8, 0.6
    k = _unit(g.standard_normal(d))
    q = g.standard_normal(d)
    v = g.standard_normal(d)
    S0 = g.standard_normal((d, d))
    ref = rec("deltanet", q[None, None, None], k[None, None, None], v[None, None, None],
              beta=np.full((1, 1, 1), c / (c + r)), S0=S0[None, None])
    for mu in (1.0, 7.0):
        got = rec("diag_kdn", q[None, None, None], k[None, None, None],
                  v[None, None, None], alpha=np.ones((1, 1, 1, d)),
                  xi=np.zeros((1, 1, 1, d)), r=np.full((1, 1, 1), r),
                  S0=S0[None, None], p0=np.full((1, 1, d), c), mu=mu)
        np.testing.assert_allclose(got[0], ref[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(got[1], ref[1], rtol=1e-13, atol=1e-14)


def pin_kdn_mobius(rec):
    """The per-channel variance recursion is a Moebius map: the product of the
    2x2 matrices [[a^2, xi], [c a^2, 1 + c xi]] (c = mu k^2 / r) applied to
    (p0, 1) gives the sequential result ([KDN] "各向同性近似" last paragraph:
    composition as 2x2 matrix products, associative scan)."""
    T, d = 40, 6
    c_ = _kdn_case(T=T, d=d, seed=32, onehot=False)
    for mu in (1.0, 6.0):
        _, _, p = _kdn_rec(rec, c_, mu=mu)
        for i in range(d):
            M = np.eye(2)
            for t in range(T):
                a2 = c_["a"][t, i] ** 2
                xi = c_["xi"][t, i]
                cc = mu * c_["k"][t, i] ** 2 / c_["r"][t]
                Mt = np.array([[a2, xi], [cc * a2, 1.0 + cc * xi]])
                M = Mt @ M
                M /= np.abs(M).max()
            num, den = M @ np.array([c_["p0"][i], 1.0])
            np.testing.assert_allclose(p[i], num / den, rtol=1e-12)


def pin_kdn_mu_effects(rec):
    """mu does not change the current write, and shrinks later writes along
    the same direction ([KDN] "对角近似" information scaling)."""
    g = _rng(33)
    d = 8
    k = _unit(g.standard_normal(d))
    c = _kdn_case(T=1, d=d, seed=34, onehot=False)
    outs = [_kdn_rec(rec, c, mu=mu) for mu in (0.5, 1.0, 8.0)]
    for o_, S_, _ in outs[1:]:
        np.testing.assert_array_equal(o_, outs[0][0])
        np.testing.assert_array_equal(S_, outs[0][1])
    # Repeated key, v1 = 0, v2 = e_0, q = k, S0 = 0: o_2[0] = k^T g_2.
    gains = []
    for mu in (0.5, 1.0, 2.0, float(d), 100.0):
        kk = np.stack([k, k])[None, :, None]
        v = np.zeros((1, 2, 1, d))
        v[0, 1, 0, 0] = 1.0
        o, _, p = rec("diag_kdn", kk, kk, v, alpha=np.ones((1, 2, 1, d)),
                      xi=np.zeros((1, 2, 1, d)), r=np.full((1, 2, 1), 0.7),
                      p0=np.full((1, 1, d), 1.0), mu=mu)
        gains.append(o[0, 1, 0, 0])
    assert all(g2 < g1 for g1, g2 in zip(gains, gains[1:])), gains
    assert all(0.0 < x < 1.0 for x in gains), gains


def pin_kdn_gain_range_and_monotone_variance(rec):
    """0 <= k^T g < 1 for r > 0; with alpha = 1 and xi = 0 the variance never
    grows; zero variance and zero process noise give zero write."""
    g = _rng(35)
    d = 6
    for trial in range(20):
        k = _unit(g.standard_normal(d))
        p0 = g.uniform(0.0, 5.0, d)
        v = np.zeros(d)
        v[0] = 1.0
        o, _, _ = rec("diag_kdn", k[None, None, None], k[None, None, None],
                      v[None, None, None], alpha=g.uniform(0, 1, (1, 1, 1, d)),
                      xi=g.uniform(0, 1, (1, 1, 1, d)),
                      r=np.full((1, 1, 1), g.uniform(0.01, 3)), p0=p0[None, None])
        assert 0.0 <= o[0, 0, 0, 0] < 1.0
    c = _kdn_case(T=25, d=d, seed=36, onehot=False)
    c["a"][:] = 1.0
    c["xi"][:] = 0.0
    prev = c["p0"]
    for T in range(1, 26):
        _, _, p = _kdn_rec(rec, c, T=T)
        assert np.all(p <= prev * (1 + 1e-15))
        prev = p
    # zero variance: no write, decay only, p stays 0
    c = _kdn_case(T=10, d=d, seed=37, onehot=False)
    c["xi"][:] = 0.0
    c["p0"][:] = 0.0
    o, S, p = _kdn_rec(rec, c)
    gam = np.cumprod(c["a"], axis=0)
    np.testing.assert_array_equal(p, np.zeros(d))
    np.testing.assert_allclose(S, gam[-1][:, None] * c["S0"], rtol=1e-14, atol=0)
    for t in range(10):
        np.testing.assert_allclose(o[t], (gam[t][:, None] * c["S0"]).T @ c["q"][t],
                                   rtol=1e-12, atol=1e-14)


def pin_kdn_degenerate_noise(rec):
    """r = 0 with a one-hot key: the observed channel's variance drops to 0
    and the write is an exact replacement; r = 0 with k = 0: no write and the
    variance only follows the predict step."""
    d = 4
    k = np.zeros((1, 1, 1, d))
    k[..., 1] = 1.0
    v = np.arange(1.0, d + 1)[None, None, None]
    S0 = np.ones((1, 1, d, d))
    o, S, p = rec("diag_kdn", k, k, v, alpha=np.full((1, 1, 1, d), 0.5),
                  xi=np.full((1, 1, 1, d), 0.1), r=np.zeros((1, 1, 1)), S0=S0,
                  p0=np.ones((1, 1, d)))
    np.testing.assert_allclose(S[0, 0, 1], v[0, 0, 0], atol=1e-15)
    assert p[0, 0, 1] == 0.0
    np.testing.assert_allclose(np.delete(p[0, 0], 1), 0.25 + 0.1, rtol=1e-15)
    o, S, p = rec("diag_kdn", np.zeros((1, 1, 1, d)), np.zeros((1, 1, 1, d)), v,
                  alpha=np.full((1, 1, 1, d), 0.5), xi=np.zeros((1, 1, 1, d)),
                  r=np.zeros((1, 1, 1)), S0=S0, p0=np.zeros((1, 1, d)))
    np.testing.assert_allclose(S[0, 0], 0.5 * S0[0, 0], rtol=0)
    np.testing.assert_array_equal(p[0, 0], np.zeros(d))


# ---------------------------------------------------------------------------
# Isotropic KDN: one variance per head ([KDN] "各向同性近似"; [AFS]
# "Approximation 2: Isotropic KDN").  The reference below is the dense Kalman
# filter of the filtering section, with its covariance brought back to a
# multiple of the identity after the predict (mean of the covariance
# diagonal) and after the update (mean of the precision diagonal, its
# increment scaled by mu as in the diagonal variant).  It works on d x d
# matrices, inverses and traces, not on the oracle's scalar arithmetic.
# ---------------------------------------------------------------------------
def _iso_case(T, d, seed, key_norms=False):
    c = _kdn_case(T=T, d=d, seed=seed, onehot=False)
    g = _rng(seed + 1000)
    if key_norms:
        c["k"] = c["k"] * g.uniform(0.3, 2.0, (T, 1))
    c["p0"] = np.array(g.uniform(0.2, 2.0))
    return c


def _iso_rec(rec, c, mu=1.0, T=None):
    T = c["k"].shape[0] if T is None else T
    sl = slice(0, T)
    o, S, p = rec("iso_kdn", c["q"][None, sl, None], c["k"][None, sl, None],
                  c["v"][None, sl, None], alpha=c["a"][None, sl, None],
                  xi=c["xi"][None, sl, None], r=c["r"][None, sl, None],
                  S0=c["S0"][None, None], p0=np.reshape(c["p0"], (1, 1)), mu=mu)
    return o[0, :, 0], S[0, 0], p[0, 0]


def _projected_kalman(c, mu):
    """Dense Kalman filter with isotropic projections; returns the memory, the
    outputs, the final variance and the per-token predicted variances."""
    S = np.array(c["S0"], np.float64)
    d = S.shape[0]
    eye = np.eye(d)
    P = float(c["p0"]) * eye
    outs, pms = [], []
    for t in range(c["k"].shape[0]):
        D = np.diag(c["a"][t])
        k = c["k"][t]
        S = D @ S
        Pm = D @ P @ D + np.diag(c["xi"][t])
        Pm = np.trace(Pm) / d * eye
        pms.append(Pm[0, 0])
        g = Pm @ k / (k @ Pm @ k + c["r"][t])
        S = S + np.outer(g, c["v"][t] - S.T @ k)
        prior = np.linalg.inv(Pm)
        post = prior + np.outer(k, k) / c["r"][t]
        lam = np.trace(prior) / d + mu * (np.trace(post) - np.trace(prior)) / d
        P = eye / lam
        outs.append(S.T @ c["q"][t])
    return S, np.array(outs), P[0, 0], np.array(pms)


def pin_iso_kdn_is_projected_dense_kalman(rec):
    for mu in (1.0, 2.5):
        c = _iso_case(T=20, d=6, seed=60, key_norms=True)
        o, S, p = _iso_rec(rec, c, mu=mu)
        S_ref, o_ref, p_ref, _ = _projected_kalman(c, mu)
        np.testing.assert_allclose(S, S_ref, atol=1e-11, rtol=1e-11)
        np.testing.assert_allclose(o, o_ref, atol=1e-11, rtol=1e-11)
        np.testing.assert_allclose(p, p_ref, rtol=1e-12)


def pin_iso_kdn_is_kda_with_derived_beta(rec):
    """The isotropic variant keeps the delta-rule form: it is KDA with the
    write strength p-/(r + p- |k|^2) taken from the uncertainty recursion."""
    c = _iso_case(T=18, d=5, seed=61, key_norms=True)
    o, S, _ = _iso_rec(rec, c, mu=1.7)
    _, _, _, pms = _projected_kalman(c, 1.7)
    kk = np.sum(c["k"] ** 2, axis=1)
    beta = pms / (c["r"] + pms * kk)
    o2, S2, _ = rec("kda", c["q"][None, :, None], c["k"][None, :, None],
                    c["v"][None, :, None], alpha=c["a"][None, :, None],
                    beta=beta[None, :, None], S0=c["S0"][None, None])
    np.testing.assert_allclose(o, o2[0, :, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, S2[0, 0], rtol=1e-12, atol=1e-13)


def pin_iso_kdn_first_step_matches_diag(rec):
    """From p0 = c 1, with one decay and one process noise for every channel,
    the first isotropic step writes exactly what the diagonal one writes, and
    its precision is the mean of the diagonal variant's channel precisions."""
    d = 7
    for mu in (1.0, 5.0):
        c = _iso_case(T=1, d=d, seed=62, key_norms=True)
        c["a"][:] = 0.8
        c["xi"][:] = 0.15
        o, S, p = _iso_rec(rec, c, mu=mu)
        cd = dict(c)
        cd["p0"] = np.full(d, float(c["p0"]))
        od, Sd, pd = _kdn_rec(rec, cd, mu=mu)
        np.testing.assert_allclose(o, od, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(S, Sd, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(1.0 / p, np.mean(1.0 / pd), rtol=1e-13)


def pin_iso_kdn_single_channel_is_diag(rec):
    """With d_k = 1 the two approximations coincide for every token."""
    c = _kdn_case(T=15, d=1, seed=63, onehot=False)
    c["k"] = _rng(64).uniform(-2.0, 2.0, (15, 1))
    for mu in (1.0, 3.0):
        o, S, p = _kdn_rec(rec, c, mu=mu)
        ci = dict(c)
        ci["p0"] = np.array(c["p0"][0])
        oi, Si, pi = _iso_rec(rec, ci, mu=mu)
        np.testing.assert_allclose(oi, o, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(Si, S, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(pi, p[0], rtol=1e-13)


def pin_iso_kdn_closed_form(rec):
    """alpha = 1, xi = 0: every token adds mu |k|^2 / (d_k r) to the precision,
    so 1/p_n = 1/p0 + (mu / d_k) sum_j |k_j|^2 / r_j."""
    d, n = 6, 9
    c = _iso_case(T=n, d=d, seed=65, key_norms=True)
    c["a"][:] = 1.0
    c["xi"][:] = 0.0
    kk = np.sum(c["k"] ** 2, axis=1)
    for mu in (1.0, 4.0):
        _, _, p = _iso_rec(rec, c, mu=mu)
        ref = 1.0 / (1.0 / float(c["p0"]) + mu / d * np.sum(kk / c["r"]))
        np.testing.assert_allclose(p, ref, rtol=1e-13)


def pin_iso_kdn_mobius(rec):
    """The head variance follows the 2x2 Moebius product with mean(a^2),
    mean(xi) and c = mu |k|^2 / (d_k r) ([KDN] "各向同性近似", last paragraph)."""
    T, d = 40, 6
    c = _iso_case(T=T, d=d, seed=66, key_norms=True)
    for mu in (1.0, 6.0):
        _, _, p = _iso_rec(rec, c, mu=mu)
        M = np.eye(2)
        for t in range(T):
            a2 = np.mean(c["a"][t] ** 2)
            xi = np.mean(c["xi"][t])
            cc = mu * np.sum(c["k"][t] ** 2) / (d * c["r"][t])
            M = np.array([[a2, xi], [cc * a2, 1.0 + cc * xi]]) @ M
            M /= np.abs(M).max()
        num, den = M @ np.array([float(c["p0"]), 1.0])
        np.testing.assert_allclose(p, num / den, rtol=1e-12)


def pin_iso_kdn_gain_range_and_degenerate(rec):
    """0 <= k^T w < 1 for r > 0; alpha = 1, xi = 0 never grows the variance;
    r = 0 with k != 0 replaces the value along k exactly and drops the
    variance to 0; r = 0 with k = 0 writes nothing and only predicts."""
    g = _rng(67)
    d = 6
    for trial in range(20):
        k = _unit(g.standard_normal(d)) * g.uniform(0.2, 3.0)
        v = np.zeros(d)
        v[0] = 1.0
        o, _, _ = rec("iso_kdn", k[None, None, None], k[None, None, None],
                      v[None, None, None], alpha=g.uniform(0, 1, (1, 1, 1, d)),
                      xi=g.uniform(0, 1, (1, 1, 1, d)),
                      r=np.full((1, 1, 1), g.uniform(0.01, 3)),
                      p0=np.full((1, 1), g.uniform(0.0, 5.0)))
        assert 0.0 <= o[0, 0, 0, 0] < 1.0
    c = _iso_case(T=25, d=d, seed=68)
    c["a"][:] = 1.0
    c["xi"][:] = 0.0
    prev = float(c["p0"])
    for T in range(1, 26):
        _, _, p = _iso_rec(rec, c, T=T)
        assert p < prev
        prev = p
    k = np.array([0.0, 2.0, 0.0, -1.0])[None, None, None]
    v = np.arange(1.0, 5.0)[None, None, None]
    S0 = _rng(69).standard_normal((1, 1, 4, 4))
    o, S, p = rec("iso_kdn", k, k, v, alpha=np.full((1, 1, 1, 4), 0.5),
                  xi=np.full((1, 1, 1, 4), 0.1), r=np.zeros((1, 1, 1)), S0=S0,
                  p0=np.ones((1, 1)))
    np.testing.assert_allclose(S[0, 0].T @ k[0, 0, 0], v[0, 0, 0], rtol=1e-14)
    assert p[0, 0] == 0.0
    z = np.zeros((1, 1, 1, 4))
    o, S, p = rec("iso_kdn", z, z, v, alpha=np.full((1, 1, 1, 4), 0.5),
                  xi=np.full((1, 1, 1, 4), 0.1), r=np.zeros((1, 1, 1)), S0=S0,
                  p0=np.ones((1, 1)))
    np.testing.assert_allclose(S[0, 0], 0.5 * S0[0, 0], rtol=0)
    np.testing.assert_allclose(p[0, 0], 0.25 + 0.1, rtol=1e-15)


# ---------------------------------------------------------------------------
# Brute force: each token as a dense affine map on vec(S) ([TAB] gated state
# and delta steps; [KDA] decay before the delta write).
# ---------------------------------------------------------------------------
def pin_brute_affine(rec):
    dk = dv = 3
    T = 5
    for variant in ("deltanet", "gated_deltanet", "kda", "diag_kdn"):
        inp = _random_inputs(variant, 1, T, 1, dk, dv, seed=40)
        o, S, _ = rec(variant, mu=2.0, **inp)
        # write vectors
        ws = []
        p = inp["p0"][0, 0].copy() if variant == "diag_kdn" else None
        avec = []
        for t in range(T):
            if variant == "deltanet":
                a = np.ones(dk)
            elif variant == "gated_deltanet":
                a = np.full(dk, inp["alpha"][0, t, 0])
            else:
                a = inp["alpha"][0, t, 0]
            kt = inp["k"][0, t, 0]
            if variant == "diag_kdn":
                pm = a * a * p + inp["xi"][0, t, 0]
                rt = inp["r"][0, t, 0]
                ws.append(pm * kt / (rt + pm @ (kt * kt)))
                p = 1.0 / (1.0 / pm + 2.0 * kt * kt / rt)
            else:
                ws.append(inp["beta"][0, t, 0] * kt)
            avec.append(a)
        # vec(S) column-major over (i, j): index i + dk*j.  One step:
        #   S' = (I - w k^T) diag(a) S + w v^T  ->  A = kron(I_dv, M), b = vec(w v^T)
        A_tot = np.eye(dk * dv)
        b_tot = np.zeros(dk * dv)
        for t in range(T):
            kt, vt, qt = inp["k"][0, t, 0], inp["v"][0, t, 0], inp["q"][0, t, 0]
            M = (np.eye(dk) - np.outer(ws[t], kt)) @ np.diag(avec[t])
            A = np.kron(np.eye(dv), M)
            bvec = np.outer(ws[t], vt).reshape(-1, order="F")
            A_tot = A @ A_tot
            b_tot = A @ b_tot + bvec
            St = (A_tot @ inp["S0"][0, 0].reshape(-1, order="F") + b_tot).reshape(
                dk, dv, order="F")
            np.testing.assert_allclose(o[0, t, 0], St.T @ qt, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(S[0, 0], St, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Resume from a state: the state (S, p) is the whole memory.
# ---------------------------------------------------------------------------
def pin_continuation(rec):
    for variant in ("gated_deltanet", "diag_kdn", "iso_kdn"):
        inp = _random_inputs(variant, 2, 30, 2, 5, 4, seed=50)
        o, S, p = rec(variant, mu=1.5, **inp)
        a = {k_: (v_[:, :11] if k_ not in ("S0", "p0") else v_) for k_, v_ in inp.items()}
        o1, S1, p1 = rec(variant, mu=1.5, **a)
        b = {k_: v_[:, 11:] for k_, v_ in inp.items() if k_ not in ("S0", "p0")}
        b["S0"] = S1
        if p1 is not None:
            b["p0"] = p1
        o2, S2, p2 = rec(variant, mu=1.5, **b)
        np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=1e-13,
                                   atol=1e-14)
        np.testing.assert_allclose(S2, S, rtol=1e-13, atol=1e-14)
        if p is not None:
            np.testing.assert_allclose(p2, p, rtol=1e-14)


def pin_empty_sequence(rec):
    for variant in ("diag_kdn", "iso_kdn"):
        inp = _random_inputs(variant, 2, 0, 3, 4, 5, seed=51)
        o, S, p = rec(variant, **inp)
        assert o.shape == (2, 0, 3, 5)
        np.testing.assert_array_equal(S, inp["S0"])
        np.testing.assert_array_equal(p, inp["p0"])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


# ---------------------------------------------------------------------------
# Gradients (write-strength variants).  The pages give no gradient; the
# oracle's backward is the exact derivative of the recurrence, pinned here to
# the (pinned) forward oracle by central differences and to closed forms.
# Each ``bwd_pin_*`` takes the oracle (the module or an ``OracleLib``) and uses
# its ``recurrence``, ``backward`` and ``backward_iso``.
# ---------------------------------------------------------------------------
BWD_VARIANTS = ("deltanet", "gated_deltanet", "kda")
GRAD_NAMES = ("q", "k", "v", "alpha", "beta", "S0")


def _bwd_inputs(variant, B, T, H, dk, dv, seed):
    inp = _random_inputs(variant, B, T, H, dk, dv, seed)
    g = _rng(seed + 500)
    inp["k"] = inp["k"] * g.uniform(0.5, 1.5, inp["k"].shape[:-1] + (1,))
    return inp


def _grads(bwd, variant, inp, dO, dS):
    dq, dk, dv, da, db, dS0 = bwd(variant, inp["q"], inp["k"], inp["v"], inp.get("alpha"),
                                  inp["beta"], inp.get("S0"), dO, dS)
    return dict(q=dq, k=dk, v=dv, alpha=da, beta=db, S0=dS0)


def bwd_pin_finite_differences(lib):
    """<grad, delta> equals the central difference of L = <o, R_o> + <S_T, R_S>
    along a random delta, for every input tensor and every variant."""
    for vi, variant in enumerate(BWD_VARIANTS):
        inp = _bwd_inputs(variant, 2, 9, 2, 4, 3, seed=70 + vi)
        g = _rng(80 + vi)
        Ro = g.standard_normal(inp["v"].shape)
        RS = g.standard_normal(inp["S0"].shape)

        def loss(x):
            o, S, _ = lib.recurrence(variant, **x)
            return float(np.sum(o * Ro) + np.sum(S * RS))

        grads = _grads(lib.backward, variant, inp, Ro, RS)
        for name in GRAD_NAMES:
            if grads[name] is None:
                continue
            d = g.standard_normal(inp[name].shape)
            eps = 1e-6
            xp = dict(inp); xp[name] = inp[name] + eps * d
            xm = dict(inp); xm[name] = inp[name] - eps * d
            fd = (loss(xp) - loss(xm)) / (2 * eps)
            an = float(np.sum(grads[name] * d))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (variant, name, fd, an)


def bwd_pin_deltanet_beta_zero_closed_form(lib):
    """beta = 0: the memory stays S0, so dq_t = S0 do_t, dk = dv = 0,
    dS0 = dS_T + sum_t q_t do_t^T, and dbeta_t = k_t^T G_t (v_t - S0^T k_t)
    with G_t = dS_T + sum_{r >= t} q_r do_r^T."""
    inp = _bwd_inputs("deltanet", 1, 7, 1, 5, 4, seed=90)
    inp["beta"] = np.zeros_like(inp["beta"])
    g = _rng(91)
    dO = g.standard_normal(inp["v"].shape)
    dS = g.standard_normal(inp["S0"].shape)
    gr = _grads(lib.backward, "deltanet", inp, dO, dS)
    S0 = inp["S0"][0, 0]
    q, k, v, do = inp["q"][0, :, 0], inp["k"][0, :, 0], inp["v"][0, :, 0], dO[0, :, 0]
    np.testing.assert_allclose(gr["q"][0, :, 0], do @ S0.T, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(gr["v"], 0.0)
    np.testing.assert_allclose(gr["k"], 0.0, atol=1e-15)
    np.testing.assert_allclose(gr["S0"][0, 0], dS[0, 0] + q.T @ do, rtol=1e-13, atol=1e-13)
    for t in range(7):
        G = dS[0, 0] + q[t:].T @ do[t:]
        ref = k[t] @ G @ (v[t] - S0.T @ k[t])
        np.testing.assert_allclose(gr["beta"][0, t, 0], ref, rtol=1e-12, atol=1e-13)


def bwd_pin_no_tokens_and_linearity(lib):
    """T = 0 passes dS_T through to dS0; the gradients are linear in the
    cotangents (dO, dS_T)."""
    inp = _bwd_inputs("kda", 1, 0, 2, 4, 3, seed=92)
    dS = _rng(93).standard_normal(inp["S0"].shape)
    gr = _grads(lib.backward, "kda", inp, np.zeros(inp["v"].shape), dS)
    np.testing.assert_array_equal(gr["S0"], dS)
    inp = _bwd_inputs("gated_deltanet", 1, 6, 1, 4, 3, seed=94)
    g = _rng(95)
    o1, o2 = g.standard_normal(inp["v"].shape), g.standard_normal(inp["v"].shape)
    s1, s2 = g.standard_normal(inp["S0"].shape), g.standard_normal(inp["S0"].shape)
    a = _grads(lib.backward, "gated_deltanet", inp, o1, s1)
    b = _grads(lib.backward, "gated_deltanet", inp, o2, s2)
    c = _grads(lib.backward, "gated_deltanet", inp, o1 + 2 * o2, s1 + 2 * s2)
    for n in GRAD_NAMES:
        np.testing.assert_allclose(c[n], a[n] + 2 * b[n], rtol=1e-11, atol=1e-12)


ISO_GRAD_NAMES = ("q", "k", "v", "alpha", "xi", "r", "S0", "p0")


def bwd_pin_iso_finite_differences(lib):
    """Isotropic KDN: <grad, delta> equals the central difference of
    L = <o, R_o> + <S_T, R_S> + <p_T, R_p> for every input, including xi, r
    and p0, at mu = 1 and mu = 3, with some exact observations (r = 0)."""
    for mu in (1.0, 3.0):
        inp = _bwd_inputs("iso_kdn", 2, 9, 2, 4, 3, seed=96)
        inp["r"][0, 4, 1] = 0.0
        g = _rng(97)
        Ro = g.standard_normal(inp["v"].shape)
        RS = g.standard_normal(inp["S0"].shape)
        Rp = g.standard_normal(inp["p0"].shape)

        def loss(x):
            o, S, p = lib.recurrence("iso_kdn", mu=mu, **x)
            return float(np.sum(o * Ro) + np.sum(S * RS) + np.sum(p * Rp))

        grads = dict(zip(ISO_GRAD_NAMES, lib.backward_iso(
            inp["q"], inp["k"], inp["v"], inp["alpha"], inp["xi"], inp["r"], inp["p0"],
            inp["S0"], Ro, RS, Rp, mu=mu)))
        for name in ISO_GRAD_NAMES:
            d = g.standard_normal(inp[name].shape)
            eps = 1e-6
            xp = dict(inp); xp[name] = inp[name] + eps * d
            xm = dict(inp); xm[name] = inp[name] - eps * d
            fd = (loss(xp) - loss(xm)) / (2 * eps)
            an = float(np.sum(grads[name] * d))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (mu, name, fd, an)


def bwd_pin_diag_finite_differences(lib):
    """Diagonal KDN: <grad, delta> equals the central difference of
    L = <o, R_o> + <S_T, R_S> + <p_T, R_p> for every input (p0 and the
    cotangent R_p per channel), at mu = 1 and mu = 3, with an exact
    observation (r = 0) and a key with zero channels in the sequence."""
    for mu in (1.0, 3.0):
        inp = _bwd_inputs("diag_kdn", 2, 9, 2, 4, 3, seed=98)
        inp["r"][1, 3, 0] = 0.0
        inp["k"][0, 5, 1, :2] = 0.0
        g = _rng(99)
        Ro = g.standard_normal(inp["v"].shape)
        RS = g.standard_normal(inp["S0"].shape)
        Rp = g.standard_normal(inp["p0"].shape)

        def loss(x):
            o, S, p = lib.recurrence("diag_kdn", mu=mu, **x)
            return float(np.sum(o * Ro) + np.sum(S * RS) + np.sum(p * Rp))

        grads = dict(zip(ISO_GRAD_NAMES, lib.backward_diag(
            inp["q"], inp["k"], inp["v"], inp["alpha"], inp["xi"], inp["r"], inp["p0"],
            inp["S0"], Ro, RS, Rp, mu=mu)))
        for name in ISO_GRAD_NAMES:
            d = g.standard_normal(inp[name].shape)

            def central(eps):
                xp = dict(inp); xp[name] = inp[name] + eps * d
                xm = dict(inp); xm[name] = inp[name] - eps * d
                return (loss(xp) - loss(xm)) / (2 * eps)

            # Richardson extrapolation: the exact observation makes the loss
            # sharply curved in r, beyond what a plain central difference at
            # this step resolves
            fd = (4 * central(1e-6) - central(2e-6)) / 3
            an = float(np.sum(grads[name] * d))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (mu, name, fd, an)


BWD_PINS = [v for k, v in sorted(globals().items()) if k.startswith("bwd_pin_")]
