"""Seeded synthetic inputs for the delta-rule / KDN workloads.

This module holds input distributions only: it draws random tensors, shapes
them, normalises keys and rounds to the device dtype.  It contains none of the
recurrence's arithmetic, so the GPU tests, the benchmark and the oracle can all
take their inputs from it without sharing any of the method.

The workloads follow the shapes the pages work at: head dimension 128 and
sequence lengths inside the 2K-32K range the KDN write-up sweeps (page "给记忆装一个
信任度探测器：Kalman Delta Networks ...", section "数据说话").  Distributions:

* q, k, v ~ N(0, 1); k is L2-normalised per token (q too for the small fp32
  DeltaNet case);
* beta = sigmoid(N(0, 1)) per token and head;
* Gated DeltaNet retention alpha = exp(-softplus(N(0, 1)) * 0.1) per token/head;
* KDA / KDN retention alpha = exp(-softplus(N(-2, 1))) per channel;
* KDN process noise xi = softplus(N(-3, 1)) per channel, observation noise
  r = softplus(N(0, 1)) per token/head, initial variance p0 = 1 (per channel
  for diagonal KDN, per head for isotropic KDN).

Draw order: q, k, v, alpha, beta, xi, r (those the variant uses).  Values are
drawn in float32 and rounded to the device dtype (round-to-nearest-even);
consumers read exactly those rounded values.
"""
from __future__ import annotations

import torch
import torch.nn.functional as F

SEED_BASE = 20261203

# name -> workload definition.  ``index`` offsets the seed.
CONFIGS = {
    "deltanet_fp32": dict(index=0, variant="deltanet", B=1, H=2, T=256, dk=64,
                          dv=64, dtype="f32", chunk=64, q_norm=True),
    "gated_deltanet": dict(index=1, variant="gated_deltanet", B=4, H=16, T=4096,
                           dk=128, dv=128, dtype="bf16", chunk=64, q_norm=False),
    "kda": dict(index=2, variant="kda", B=2, H=32, T=8192, dk=128, dv=128,
                dtype="bf16", chunk=64, q_norm=False),
    "diag_kdn": dict(index=3, variant="diag_kdn", B=2, H=16, T=16384, dk=128,
                     dv=128, dtype="bf16", chunk=64, q_norm=False),
    "decode_diag_kdn": dict(index=4, variant="diag_kdn", N=256, H=32, steps=1024,
                            dk=128, dv=128, dtype="bf16", q_norm=False),
    "iso_kdn": dict(index=5, variant="iso_kdn", B=2, H=16, T=16384, dk=128,
                    dv=128, dtype="bf16", chunk=64, q_norm=False),
}

KDN_VARIANTS = ("diag_kdn", "iso_kdn")

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def seed_of(name: str) -> int:
    return SEED_BASE + CONFIGS[name]["index"]


def _normal(gen, shape, mean=0.0, device="cpu"):
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    return x + mean if mean else x


def _l2n(x):
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def gen_prefill(variant, B, T, H, dk, dv, dtype="bf16", seed=SEED_BASE,
                device="cpu", q_norm=False, random_state=False):
    """Draw one batch of prefill inputs.

    Returns a dict with q, k [B,T,H,dk], v [B,T,H,dv] in ``dtype``; ``alpha``
    ([B,T,H] for gated_deltanet, [B,T,H,dk] for kda and the KDNs) and
    ``beta`` [B,T,H] (not the KDNs), ``xi`` [B,T,H,dk] and ``r`` [B,T,H]
    (KDNs) in ``dtype``; ``S0`` [B,H,dk,dv] float32 (None unless
    ``random_state``) and ``p0`` float32, [B,H,dk] for diag_kdn and [B,H] for
    iso_kdn (ones unless ``random_state``).
    """
    tdt = TORCH_DTYPES[dtype]
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = {}
    q = _normal(gen, (B, T, H, dk), device=device)
    k = _normal(gen, (B, T, H, dk), device=device)
    v = _normal(gen, (B, T, H, dv), device=device)
    out["q"] = (_l2n(q) if q_norm else q).to(tdt)
    out["k"] = _l2n(k).to(tdt)
    out["v"] = v.to(tdt)
    if variant == "gated_deltanet":
        a = _normal(gen, (B, T, H), device=device)
        out["alpha"] = torch.exp(-F.softplus(a) * 0.1).to(tdt)
    elif variant in ("kda",) + KDN_VARIANTS:
        a = _normal(gen, (B, T, H, dk), mean=-2.0, device=device)
        out["alpha"] = torch.exp(-F.softplus(a)).to(tdt)
    if variant not in KDN_VARIANTS:
        out["beta"] = torch.sigmoid(_normal(gen, (B, T, H), device=device)).to(tdt)
    else:
        out["xi"] = F.softplus(_normal(gen, (B, T, H, dk), mean=-3.0,
                                       device=device)).to(tdt)
        out["r"] = F.softplus(_normal(gen, (B, T, H), device=device)).to(tdt)
    pshape = (B, H, dk) if variant == "diag_kdn" else (B, H)
    if random_state:
        out["S0"] = (0.5 * _normal(gen, (B, H, dk, dv), device=device)).contiguous()
        if variant in KDN_VARIANTS:
            out["p0"] = torch.rand(pshape, generator=gen, device=device,
                                   dtype=torch.float32) + 0.5
    else:
        out["S0"] = None
        if variant in KDN_VARIANTS:
            out["p0"] = torch.ones(pshape, dtype=torch.float32, device=device)
    return out


def gen_config(name, device="cpu", **overrides):
    """Inputs of a named prefill workload (sizes may be overridden)."""
    c = dict(CONFIGS[name])
    c.update(overrides)
    return gen_prefill(c["variant"], c["B"], c["T"], c["H"], c["dk"], c["dv"],
                       c["dtype"], seed=c.get("seed", seed_of(name)),
                       device=device, q_norm=c.get("q_norm", False),
                       random_state=c.get("random_state", False))


def gen_decode(N, H, steps, dk, dv, dtype="bf16", seed=SEED_BASE + 4,
               device="cpu", block=64, variant="diag_kdn"):
    """Per-step decode inputs stacked over steps: [steps, N, H, d].

    Drawn ``block`` steps at a time (same draw order as prefill within each
    block) so that the float32 temporaries stay small.
    """
    tdt = TORCH_DTYPES[dtype]
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    names = ["q", "k", "v"]
    if variant == "gated_deltanet":
        names += ["alpha"]
    elif variant in ("kda",) + KDN_VARIANTS:
        names += ["alpha"]
    names += ["beta"] if variant not in KDN_VARIANTS else ["xi", "r"]
    out = {}
    for n in names:
        if n in ("beta", "r") or (n == "alpha" and variant == "gated_deltanet"):
            shape = (steps, N, H)
        elif n == "v":
            shape = (steps, N, H, dv)
        else:
            shape = (steps, N, H, dk)
        out[n] = torch.empty(shape, dtype=tdt, device=device)
    for s0 in range(0, steps, block):
        s1 = min(steps, s0 + block)
        n_ = s1 - s0
        q = _normal(gen, (n_, N, H, dk), device=device)
        k = _normal(gen, (n_, N, H, dk), device=device)
        v = _normal(gen, (n_, N, H, dv), device=device)
        out["q"][s0:s1] = q.to(tdt)
        out["k"][s0:s1] = _l2n(k).to(tdt)
        out["v"][s0:s1] = v.to(tdt)
        del q, k, v
        if variant == "gated_deltanet":
            a = _normal(gen, (n_, N, H), device=device)
            out["alpha"][s0:s1] = torch.exp(-F.softplus(a) * 0.1).to(tdt)
        elif variant in ("kda",) + KDN_VARIANTS:
            a = _normal(gen, (n_, N, H, dk), mean=-2.0, device=device)
            out["alpha"][s0:s1] = torch.exp(-F.softplus(a)).to(tdt)
        if variant not in KDN_VARIANTS:
            out["beta"][s0:s1] = torch.sigmoid(
                _normal(gen, (n_, N, H), device=device)).to(tdt)
        else:
            out["xi"][s0:s1] = F.softplus(
                _normal(gen, (n_, N, H, dk), mean=-3.0, device=device)).to(tdt)
            out["r"][s0:s1] = F.softplus(
                _normal(gen, (n_, N, H), device=device)).to(tdt)
    out["S0"] = torch.zeros((N, H, dk, dv), dtype=torch.float32, device=device)
    if variant == "diag_kdn":
        out["p0"] = torch.ones((N, H, dk), dtype=torch.float32, device=device)
    elif variant == "iso_kdn":
        out["p0"] = torch.ones((N, H), dtype=torch.float32, device=device)
    return out


def to_f64(x):
    """Exact upcast of a (possibly bf16) tensor to a float64 numpy array."""
    if x is None:
        return None
    return x.detach().to("cpu").to(torch.float64).numpy()


def orthonormal_keys(n, d, seed=0):
    """n <= d orthonormal rows (QR of a Gaussian), float64."""
    g = torch.Generator().manual_seed(int(seed))
    a = torch.randn((d, n), generator=g, dtype=torch.float64)
    qm, _ = torch.linalg.qr(a)
    return qm.T.contiguous()


def bytes_per_elem(dtype):
    return 4 if dtype == "f32" else 2


def ceil_div(a, b):
    return -(-a // b) if b else 0


__all__ = ["CONFIGS", "SEED_BASE", "gen_prefill", "gen_config", "gen_decode",
           "seed_of", "to_f64", "orthonormal_keys", "bytes_per_elem",
           "ceil_div", "TORCH_DTYPES"]
