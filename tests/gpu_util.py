"""Helpers of the GPU parity tests: run the HIP path through the binding, run
the oracle on the same (device-rounded) inputs, and compare."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
from linear_attention_recurrent_delta_amd import kdn, synth

# max|gpu - ref| / max|ref| per output tensor
TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("q", "k", "v", "alpha", "beta", "xi", "r", "S0", "p0")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    m = float(np.abs(ref).max())
    e = float(np.abs(got - ref).max())
    if not np.isfinite(e):
        return float("inf")
    return e / m if m > 0 else e


def check(name, got, ref, tol):
    e = rel_err(got, ref)
    log(f"    {name}: rel err {e:.3e} (tol {tol:.0e})")
    assert e <= tol, f"{name}: relative error {e:.3e} > {tol:.0e}"
    return e


def to_device(inp, device="cuda"):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v)
            for k, v in inp.items()}


# Prefill schedule the GPU tests run: "auto" (two-pass, with a workspace) or
# None (single pass).  test_gpu_parity runs every case under both.
SCHEDULE = {"workspace": "auto"}


def gpu_prefill(variant, inp, mu=1.0, chunk=0, out=None):
    o, S, p = kdn.prefill(variant, inp["q"], inp["k"], inp["v"],
                          alpha=inp.get("alpha"), beta=inp.get("beta"),
                          proc_noise=inp.get("xi"), obs_noise=inp.get("r"),
                          S0=inp.get("S0"), p0=inp.get("p0"), mu=mu, chunk=chunk,
                          out=out, workspace=SCHEDULE["workspace"])
    torch.cuda.synchronize()
    return o, S, p


def np64(x):
    return None if x is None else synth.to_f64(x)


def oracle_prefill(variant, inp, mu=1.0, heads=None):
    """Oracle on all heads, or on the listed (b, h) pairs (each one is an
    independent stream, sliced out of the inputs)."""
    if heads is None:
        args = {k: np64(inp.get(k)) for k in NAMES}
        return oracle.recurrence(variant, args["q"], args["k"], args["v"],
                                 alpha=args["alpha"], beta=args["beta"],
                                 xi=args["xi"], r=args["r"], S0=args["S0"],
                                 p0=args["p0"], mu=mu)
    res = {}
    for (b, h) in heads:
        sl = {}
        for k in NAMES:
            x = inp.get(k)
            if x is None:
                sl[k] = None
            elif k in ("S0", "p0"):
                sl[k] = np64(x[b:b + 1, h:h + 1])
            else:
                sl[k] = np64(x[b:b + 1, :, h:h + 1])
        res[(b, h)] = oracle.recurrence(variant, sl["q"], sl["k"], sl["v"],
                                        alpha=sl["alpha"], beta=sl["beta"],
                                        xi=sl["xi"], r=sl["r"], S0=sl["S0"],
                                        p0=sl["p0"], mu=mu)
    return res


def compare_prefill(variant, inp, got, tol, mu=1.0, heads=None, label=""):
    o, S, p = got
    t0 = time.time()
    if heads is None:
        ro, rS, rp = oracle_prefill(variant, inp, mu=mu)
        log(f"  {label} oracle {time.time() - t0:.1f}s")
        check("o", np64(o), ro, tol)
        check("S", np64(S), rS, tol)
        if rp is not None:
            check("p", np64(p), rp, tol)
        return
    res = oracle_prefill(variant, inp, mu=mu, heads=heads)
    log(f"  {label} oracle on {len(heads)} sampled heads {time.time() - t0:.1f}s")
    for (b, h), (ro, rS, rp) in res.items():
        check(f"o[b={b},h={h}]", np64(o[b:b + 1, :, h:h + 1]), ro, tol)
        check(f"S[b={b},h={h}]", np64(S[b:b + 1, h:h + 1]), rS, tol)
        if rp is not None:
            check(f"p[b={b},h={h}]", np64(p[b:b + 1, h:h + 1]), rp, tol)


def decode_inputs_as_prefill(dinp):
    """[steps, N, H, ...] per-step inputs viewed as a [N, steps, H, ...]
    prefill batch (same values) for the oracle."""
    out = {}
    for k, v in dinp.items():
        if v is None:
            out[k] = None
        elif k in ("S0", "p0"):
            out[k] = v
        else:
            out[k] = v.transpose(0, 1)
    return out


def gpu_decode_run(variant, dinp, mu=1.0, steps=None, keep_outputs=True):
    """Run the decode entry point for every step, state resident on the GPU.
    Returns (o [steps, N, H, dv] or None, S, p)."""
    q = dinp["q"]
    steps = q.shape[0] if steps is None else steps
    S = dinp["S0"].clone()
    p = dinp["p0"].clone() if dinp.get("p0") is not None else None
    N, H, dv = q.shape[1], q.shape[2], dinp["v"].shape[-1]
    os_ = torch.empty((steps, N, H, dv), dtype=q.dtype, device=q.device) \
        if keep_outputs else None
    o = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    for t in range(steps):
        g = lambda k: (dinp[k][t] if dinp.get(k) is not None else None)
        kdn.decode(variant, g("q"), g("k"), g("v"), S, p, alpha=g("alpha"),
                   beta=g("beta"), proc_noise=g("xi"), obs_noise=g("r"), mu=mu,
                   o=os_[t] if keep_outputs else o)
    torch.cuda.synchronize()
    return os_, S, p
