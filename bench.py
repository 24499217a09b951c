"""Benchmark of the delta-rule / Kalman-delta hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--workloads all|headline]

One step is one chunkwise prefill call over the diagonal-KDN workload
(B=2, H=16, T=16384, d_k=d_v=128, bf16 inputs, fp32 state and variance,
C=64) -- the largest prefill workload -- with inputs resident in HBM.  Rank 0
prints ONE JSON line with the headline value (prefill tokens/s), the roofline
of the prefill call (HBM-bound by its algorithmic bytes; the MFMA fraction of
its algorithmic flops is reported next to it), the diagonal-KDN decode
workload beside it (256 sequences x 32 heads, 1024 steps: steps/s and its
HBM roofline), the fp64 oracle timed on the host cores on the headline
workload, and the other workloads (Gated DeltaNet, KDA and isotropic-KDN
prefill, the gradient calls of Gated DeltaNet, KDA and both KDN variants,
16-token multi-token decode) each with its own roofline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s + decode steps/s per head-state; % MFMA / % HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector
# the largest prefill workload: diagonal KDN, B2 H16 T16384, d_k = d_v = 128, bf16
HEADLINE = "diag_kdn"
KERNEL_SOURCES = ["kdn_prefill.hip", "kdn_prefill_state.hip", "kdn_prefill_chain.hip",
                  "kdn_prefill_short.hip", "kdn_variance.hip", "kdn_backward.hip", "kdn_decode.hip", "kdn_device.h",
                  "kdn_launch.h", "kdn_workspace.h"]


def kernel_hash(names=KERNEL_SOURCES):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "linear_attention_recurrent_delta_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def prefill_bytes(variant, B, T, H, dk, dv, es, has_S0):
    tok = B * T * H
    n = tok * (2 * dk + 2 * dv) * es               # q, k, v, o
    if variant == "gated_deltanet":
        n += tok * es
    elif variant in ("kda", "diag_kdn", "iso_kdn"):
        n += tok * dk * es
    if variant in ("diag_kdn", "iso_kdn"):
        n += tok * dk * es + tok * es               # xi, r
        n += 2 * B * H * (dk if variant == "diag_kdn" else 1) * 4   # p0, p_out
    else:
        n += tok * es                               # beta
    n += B * H * dk * dv * 4 * (2 if has_S0 else 1)
    return n


def prefill_flops_per_head_token(C, dk, dv):
    # A_kk, A_qk (2 C dk), T solve (C^2/3), products with T ((C-1)(dk+dv)),
    # A_qk E ((C+1) dv), K~S, Q~S, W~^T E (6 dk dv); triangles counted as half.
    return 2 * C * dk + C * C / 3 + (C - 1) * (dk + dv) + (C + 1) * dv + 6 * dk * dv


def backward_bytes(variant, B, T, H, dk, dv, es):
    """Gradient call: q, k, v, dO and the gates (beta, alpha; KDN: alpha, the
    noises and p0) read in the call dtype (p0 float32); dq, dk, dv and the
    gates' gradients written as float32; S0 = dS_out = dp_out = NULL."""
    tok = B * T * H
    kdn = variant in ("diag_kdn", "iso_kdn")
    n = tok * (2 * dk + 2 * dv) * es                        # q, k, v, dO
    n += tok * (2 * dk + dv) * 4                            # dq, dk, dv
    if not kdn:
        n += tok * es + tok * 4                             # beta, dbeta
    if variant == "gated_deltanet":
        n += tok * es + tok * 4                             # alpha, dlog_alpha
    elif variant != "deltanet":
        n += tok * dk * es + tok * dk * 4
    if kdn:
        n += tok * dk * es + tok * es + tok * dk * 4 + tok * 4   # xi, r, dxi, dr
        n += 2 * B * H * (dk if variant == "diag_kdn" else 1) * 4  # p0, dp0
    n += B * H * dk * dv * 4                                # dS0
    return n


def backward_flops_per_head_token(C, dk, dv):
    """The forward chunk pass it re-runs, then per token (multiply-adds, x2):
    the reverse state pass A_qk^T dO, W~ dS, T^T dE, Q~^T dO, K~^T dU
    (C dv + 3 dk dv) and the local gradients U, E, dE, dU, dO S^T, dU S^T,
    E dS^T, dO E^T, dU E^T and the four decay-scaled C x C x dk products
    (5 dk dv + 2.5 C dv + 2 C dk); triangles counted as half."""
    state = C * dv + 3 * dk * dv
    local = 5 * dk * dv + 2.5 * C * dv + 2 * C * dk
    return prefill_flops_per_head_token(C, dk, dv) + 2 * (state + local)


def decode_bytes(N, H, dk, dv, es):
    """Diagonal-KDN decode step: S and p read and written once; q, k, alpha,
    xi [dk], v [dv], r read; o [dv] written."""
    nh = N * H
    return (nh * dk * dv * 4 * 2 + nh * dk * 4 * 2 + nh * 4 * dk * es
            + nh * dv * es + nh * es + nh * dv * es)


def verify_bytes(N, T, H, dk, dv, es):
    """Multi-token decode of T tokens (diagonal KDN): S and p read and written
    once; per token q, k, alpha, xi [dk], v [dv], r read and o [dv] written."""
    nh = N * H
    return (nh * dk * dv * 4 * 2 + nh * dk * 4 * 2
            + T * (nh * 4 * dk * es + nh * dv * es + nh * es + nh * dv * es))


def decode_flops_per_head_token(dk, dv):
    # decay (dk dv), read S^T k (2 dk dv), write w e^T (2 dk dv), output S^T q
    # (2 dk dv); the gain's O(dk) terms are left out
    return 7 * dk * dv


def load_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they
    were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(kernel)
    if not e or e.get("kernel_hash") != kernel_hash():
        return None
    return e.get("bytes_per_launch")


def time_launches(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(steps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) / 1e3


def bench_prefill(name, steps, warmup, torch, kdn, synth, schedule="two_pass"):
    c = synth.CONFIGS[name]
    inp = synth.gen_config(name, device="cuda")
    B, T, H, dk, dv = c["B"], c["T"], c["H"], c["dk"], c["dv"]
    o = torch.empty((B, T, H, dv), dtype=inp["q"].dtype, device="cuda")
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    p = torch.empty_like(inp["p0"]) if inp.get("p0") is not None else None
    # caller-owned workspace of the two-pass schedule, allocated once
    ws = kdn.workspace(c["variant"], inp["q"], inp["v"]) if schedule == "two_pass" else None

    def step():
        kdn.prefill(c["variant"], inp["q"], inp["k"], inp["v"], alpha=inp.get("alpha"),
                    beta=inp.get("beta"), proc_noise=inp.get("xi"),
                    obs_noise=inp.get("r"), S0=inp.get("S0"), p0=inp.get("p0"),
                    out=(o, S, p), workspace=ws)

    wall, gpu = time_launches(step, steps, warmup, torch)
    es = 2 if c["dtype"] == "bf16" else 4
    C = kdn.kdn_chunk_prefill_chunk_size(1 if c["dtype"] == "bf16" else 0, dk, dv, 0)
    nbytes = prefill_bytes(c["variant"], B, T, H, dk, dv, es, inp.get("S0") is not None)
    flops = prefill_flops_per_head_token(C, dk, dv) * B * H * T
    launch_s = gpu / steps
    traffic = load_traffic(f"prefill_{name}")
    res = {
        "value": B * T * steps / wall, "unit": "tokens/s",
        "head_tokens_per_s": B * H * T * steps / wall,
        "ms_per_step": wall / steps * 1e3,
        "config": {"workload": f"{name}_prefill", "variant": c["variant"], "B": B,
                   "T": T, "H": H, "d_k": dk, "d_v": dv, "chunk": C,
                   "dtype": c["dtype"], "schedule": schedule,
                   "workspace_bytes": 0 if ws is None else ws.numel()},
        "roofline": {"bound": "hbm", "achieved": nbytes / launch_s / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nbytes / launch_s / 1e9 / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes": nbytes,
                     "kernel_ms": launch_s * 1e3},
        "mfma": {"achieved": flops / launch_s / 1e12, "peak": BF16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": flops / launch_s / 1e12 / BF16_PEAK_TFLOPS,
                 "algorithmic_flops": flops},
    }
    del inp, o, S, p, ws
    torch.cuda.empty_cache()
    return res


def bench_backward(name, steps, warmup, torch, kdn, synth):
    c = synth.CONFIGS[name]
    variant = c["variant"]
    inp = synth.gen_config(name, device="cuda")
    B, T, H, dk, dv = c["B"], c["T"], c["H"], c["dk"], c["dv"]
    g = torch.Generator(device="cuda")
    g.manual_seed(synth.seed_of(name) + 7)
    d_o = torch.randn((B, T, H, dv), generator=g, device="cuda").to(inp["q"].dtype)
    f = torch.float32
    new = lambda *shape: torch.empty(shape, dtype=f, device="cuda")
    kdn_var = variant in ("diag_kdn", "iso_kdn")
    out = dict(dq=new(B, T, H, dk), dk=new(B, T, H, dk), dv=new(B, T, H, dv),
               dlog_alpha=None if variant == "deltanet" else (
                   new(B, T, H) if variant == "gated_deltanet" else new(B, T, H, dk)),
               dbeta=None if kdn_var else new(B, T, H), dS0=new(B, H, dk, dv),
               dproc_noise=new(B, T, H, dk) if kdn_var else None,
               dobs_noise=new(B, T, H) if kdn_var else None,
               dp0=torch.empty_like(inp["p0"]) if kdn_var else None)
    dt = 1 if c["dtype"] == "bf16" else 0
    C = kdn.kdn_chunk_prefill_chunk_size(dt, dk, dv, 0)
    n = kdn.kdn_chunk_prefill_backward_workspace_size(kdn.VARIANTS[variant], dt, B, T, H,
                                                      dk, dv, 0)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")

    def step():
        kdn.prefill_backward(variant, inp["q"], inp["k"], inp["v"], d_o,
                             alpha=inp.get("alpha"), beta=inp.get("beta"),
                             proc_noise=inp.get("xi"), obs_noise=inp.get("r"),
                             p0=inp.get("p0"), out=out, workspace=ws)

    wall, gpu = time_launches(step, steps, warmup, torch)
    es = 2 if c["dtype"] == "bf16" else 4
    nbytes = backward_bytes(variant, B, T, H, dk, dv, es)
    flops = backward_flops_per_head_token(C, dk, dv) * B * H * T
    launch_s = gpu / steps
    res = {
        "value": B * T * steps / wall, "unit": "tokens/s",
        "head_tokens_per_s": B * H * T * steps / wall,
        "ms_per_step": wall / steps * 1e3,
        "config": {"workload": f"{name}_backward", "variant": variant, "B": B, "T": T,
                   "H": H, "d_k": dk, "d_v": dv, "chunk": C, "dtype": c["dtype"],
                   "gradients": "float32", "workspace_bytes": n},
        "roofline": {"bound": "hbm", "achieved": nbytes / launch_s / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nbytes / launch_s / 1e9 / HBM_PEAK_GBS,
                     "traffic": load_traffic(f"backward_{name}"), "algorithmic_bytes": nbytes,
                     "kernel_ms": launch_s * 1e3},
        "mfma": {"achieved": flops / launch_s / 1e12, "peak": BF16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": flops / launch_s / 1e12 / BF16_PEAK_TFLOPS,
                 "algorithmic_flops": flops},
    }
    del inp, d_o, out, ws
    torch.cuda.empty_cache()
    return res


def bench_decode(name, reps, torch, kdn, synth, shape=None):
    """Decode steps of the diagonal-KDN decode workload (or, with shape =
    (N, H, d, steps), of another batch of sequences and head size)."""
    c = dict(synth.CONFIGS[name])
    if shape is not None:
        c["N"], c["H"], c["dk"], c["steps"] = shape
        c["dv"] = c["dk"]
    N, H, steps, dk, dv = c["N"], c["H"], c["steps"], c["dk"], c["dv"]
    d = synth.gen_decode(N, H, steps, dk, dv, c["dtype"], seed=synth.seed_of(name),
                         device="cuda")
    S = d["S0"].clone()
    p = d["p0"].clone()
    o = torch.empty((N, H, dv), dtype=d["q"].dtype, device="cuda")
    args = [(d["q"][t], d["k"][t], d["v"][t], d["alpha"][t], d["xi"][t], d["r"][t])
            for t in range(steps)]

    def run_all():
        for (q, k, v, a, x, r) in args:
            kdn.decode("diag_kdn", q, k, v, S, p, alpha=a, proc_noise=x, obs_noise=r,
                       o=o)

    wall, gpu = time_launches(run_all, reps, 1, torch)
    nsteps = steps * reps
    es = 2 if c["dtype"] == "bf16" else 4
    nbytes = decode_bytes(N, H, dk, dv, es)
    launch_s = gpu / nsteps
    res = {
        "value": nsteps / wall, "unit": "steps/s",
        "head_state_steps_per_s": nsteps * N * H / wall,
        "ms_per_step": wall / nsteps * 1e3,
        "config": {"workload": name if shape is None else f"{name}_N{N}_H{H}_d{dk}",
                   "variant": "diag_kdn", "N": N, "H": H,
                   "steps": steps, "d_k": dk, "d_v": dv, "dtype": c["dtype"]},
        "roofline": {"bound": "hbm", "achieved": nbytes / launch_s / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nbytes / launch_s / 1e9 / HBM_PEAK_GBS,
                     "traffic": load_traffic(name) if shape is None else None,
                     "algorithmic_bytes": nbytes, "kernel_ms": launch_s * 1e3},
    }
    del d, S, p, o, args
    torch.cuda.empty_cache()
    return res


def bench_verify(T, reps, torch, kdn, synth, path="chunk"):
    """T draft tokens per sequence checked against the resident state at the
    decode workload's size (diagonal KDN): path "chunk" is one
    kdn_chunk_prefill call (the short-sequence kernel: chunk form on MFMA),
    path "token" one kdn_recurrent_decode_multi call (token by token, the
    bits of T decode steps)."""
    name = "decode_diag_kdn"
    c = synth.CONFIGS[name]
    N, H, dk, dv = c["N"], c["H"], c["dk"], c["dv"]
    inp = synth.gen_prefill("diag_kdn", N, T, H, dk, dv, c["dtype"],
                            seed=synth.seed_of(name) + 100, device="cuda",
                            random_state=True)
    o = torch.empty((N, T, H, dv), dtype=inp["q"].dtype, device="cuda")
    S = torch.empty_like(inp["S0"])
    p = torch.empty_like(inp["p0"])

    def step():
        if path == "chunk":
            kdn.prefill("diag_kdn", inp["q"], inp["k"], inp["v"], alpha=inp["alpha"],
                        proc_noise=inp["xi"], obs_noise=inp["r"], S0=inp["S0"],
                        p0=inp["p0"], out=(o, S, p), workspace=None)
        else:
            kdn.decode_multi("diag_kdn", inp["q"], inp["k"], inp["v"], alpha=inp["alpha"],
                             proc_noise=inp["xi"], obs_noise=inp["r"], S0=inp["S0"],
                             p0=inp["p0"], out=(o, S, p))

    wall, gpu = time_launches(step, reps, 3, torch)
    es = 2 if c["dtype"] == "bf16" else 4
    nbytes = verify_bytes(N, T, H, dk, dv, es)
    launch_s = gpu / reps
    workload = f"verify{T}_diag_kdn" if path == "chunk" else f"multi{T}_diag_kdn"
    res = {
        "value": N * T * reps / wall, "unit": "tokens/s",
        "head_tokens_per_s": N * H * T * reps / wall,
        "ms_per_step": wall / reps * 1e3,
        "config": {"workload": workload, "variant": "diag_kdn", "N": N, "T": T, "H": H,
                   "d_k": dk, "d_v": dv, "dtype": c["dtype"],
                   "path": "kdn_chunk_prefill (short-sequence kernel)" if path == "chunk"
                           else "kdn_recurrent_decode_multi (token by token)"},
        "roofline": {"bound": "hbm", "achieved": nbytes / launch_s / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nbytes / launch_s / 1e9 / HBM_PEAK_GBS,
                     "traffic": load_traffic(workload),
                     "algorithmic_bytes": nbytes, "kernel_ms": launch_s * 1e3},
    }
    if path == "chunk":
        flops = prefill_flops_per_head_token(16, dk, dv) * N * H * T
        res["mfma"] = {"achieved": flops / launch_s / 1e12, "peak": BF16_PEAK_TFLOPS,
                       "unit": "TFLOP/s",
                       "frac": flops / launch_s / 1e12 / BF16_PEAK_TFLOPS,
                       "algorithmic_flops": flops}
    else:
        flops = decode_flops_per_head_token(dk, dv) * N * H * T
        res["alu"] = {"achieved": flops / launch_s / 1e12, "peak": FP32_VALU_PEAK_TFLOPS,
                      "unit": "TFLOP/s",
                      "frac": flops / launch_s / 1e12 / FP32_VALU_PEAK_TFLOPS,
                      "algorithmic_flops": flops}
    del inp, o, S, p
    torch.cuda.empty_cache()
    return res


def measure_achievable(torch, copy_mib=2048, gemm_n=8192, reps=10):
    """What this machine reaches on plain work, reported beside the published
    peaks (the roofline fractions stay against the published ones): a plain
    streaming kernel out = 1.0 * in over 2 GiB of float32 (read + write bytes
    / time) and a dense bf16 GEMM through the vendor library (2 n^3 flop /
    time).  Context for the fractions, not part of the path."""
    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps
    n = copy_mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t_copy = timed(lambda: torch.mul(src, 1.0, out=dst))
    del src, dst
    a = torch.randn(gemm_n, gemm_n, device="cuda").to(torch.bfloat16).contiguous()
    b = torch.randn(gemm_n, gemm_n, device="cuda").to(torch.bfloat16).contiguous()
    c = torch.empty(gemm_n, gemm_n, dtype=torch.bfloat16, device="cuda")
    t_gemm = timed(lambda: torch.matmul(a, b, out=c))
    del a, b, c
    torch.cuda.empty_cache()
    return {"hbm_copy_GBs": 2 * n * 4 / t_copy / 1e9,
            "bf16_gemm_TFLOPs": 2 * gemm_n ** 3 / t_gemm / 1e12,
            "method": f"out = 1.0 * in over {copy_mib} MiB float32; {gemm_n}^3 bf16 "
                      f"matmul (vendor library); mean of {reps} after 3 warm-ups"}


def cpu_baseline(name, synth, budget_s=20.0):
    """The fp64 oracle, as it stands, on a bounded sample of the workload:
    whole-length (batch, head) streams, as many as fit the time budget."""
    import numpy as np
    import torch
    import oracle
    c = synth.CONFIGS[name]
    inp = synth.gen_config(name, device="cpu")
    B, T, H = c["B"], c["T"], c["H"]
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    f64 = synth.to_f64

    def sample(nheads):
        heads = [(i // H, i % H) for i in range(nheads)]
        sl = {}
        for k in ("q", "k", "v", "alpha", "beta", "xi", "r"):
            x = inp.get(k)
            if x is None:
                sl[k] = None
                continue
            parts = [f64(x[b:b + 1, :, h:h + 1]) for (b, h) in heads]
            sl[k] = np.concatenate(parts, axis=2)
        p0 = (np.ones((1, nheads, c["dk"])) if c["variant"] == "diag_kdn" else
              np.ones((1, nheads)) if c["variant"] == "iso_kdn" else None)
        return sl, p0

    sl, p0 = sample(1)
    t0 = time.perf_counter()
    oracle.recurrence(c["variant"], sl["q"], sl["k"], sl["v"], alpha=sl["alpha"],
                      beta=sl["beta"], xi=sl["xi"], r=sl["r"], p0=p0, nthreads=1)
    one = time.perf_counter() - t0
    nheads = int(max(1, min(B * H, budget_s * threads / max(one, 1e-6))))
    nheads = max(1, (nheads // threads) * threads) if nheads >= threads else nheads
    sl, p0 = sample(nheads)
    used = min(threads, nheads)
    reps, el = 0, 0.0
    # whole sample, repeated until about a quarter of the budget has elapsed
    while reps == 0 or el < budget_s / 4:
        t0 = time.perf_counter()
        oracle.recurrence(c["variant"], sl["q"], sl["k"], sl["v"], alpha=sl["alpha"],
                          beta=sl["beta"], xi=sl["xi"], r=sl["r"], p0=p0,
                          nthreads=threads)
        el += time.perf_counter() - t0
        reps += 1
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh
                          if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": reps * nheads * T / H / el, "unit": "tokens/s", "cores": used,
            "kind": "oracle", "cpu_model": model,
            "one_thread_value": T / H / one,
            "one_thread_sample": f"1 (batch, head) stream at T={T}, {one:.2f} s on 1 thread",
            "sample": f"{nheads} of {B * H} (batch, head) streams at full length "
                      f"T={T} ({nheads * T} head-tokens) x {reps} passes, fp64, "
                      f"{el:.1f} s on {used} threads; tokens/s counts all {H} heads "
                      f"of a token"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workloads", choices=["all", "headline"], default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="run one workload and print its JSON object only (for "
                         "profiling): <name>_prefill, <name>_backward, "
                         "decode_diag_kdn, verify16_diag_kdn (chunk path) or "
                         "multi16_diag_kdn (token by token)")
    ap.add_argument("--decode-sweep", action="store_true",
                    help="time diagonal-KDN decode steps over several batch sizes "
                         "and head sizes (one JSON line each) instead of the bench")
    ap.add_argument("--schedule", choices=["two_pass", "single_pass"], default="two_pass",
                    help="prefill schedule: with a workspace (two-pass) or without")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain streaming kernel (out = 1.0 * in, "
                         "float32) over this many MiB, as a reference for "
                         "hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on one GPU only; the recurrence shards "
              "over (batch, head) with no communication, so N GPUs = N "
              "independent copies of this run.", file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_recurrent_delta_amd import kdn, synth
    kdn.ensure_built()
    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if args.decode_sweep:
        # (sequences, heads, head size, steps): from a launch-bound batch to
        # four times the decode workload, and head size 64
        for shape in [(8, 32, 128, 256), (32, 32, 128, 256), (128, 32, 128, 128),
                      (256, 32, 128, 64), (1024, 32, 128, 32), (256, 32, 64, 128),
                      (1024, 32, 64, 64)]:
            r = bench_decode("decode_diag_kdn", 4, torch, kdn, synth, shape)
            r["kernel_hash"] = kernel_hash()
            print(json.dumps(r), flush=True)
        return

    if args.only:
        w = args.only
        if w.endswith("_prefill"):
            r = bench_prefill(w[:-len("_prefill")], args.steps, args.warmup, torch, kdn,
                              synth, args.schedule)
        elif w.endswith("_backward"):
            r = bench_backward(w[:-len("_backward")], args.steps, args.warmup, torch, kdn,
                               synth)
        elif w == "decode_diag_kdn":
            r = bench_decode(w, max(1, args.steps // 1024), torch, kdn, synth)
        elif w.startswith("verify") and w.endswith("_diag_kdn"):
            r = bench_verify(int(w[len("verify"):-len("_diag_kdn")]), args.steps, torch,
                             kdn, synth, "chunk")
        elif w.startswith("multi") and w.endswith("_diag_kdn"):
            r = bench_verify(int(w[len("multi"):-len("_diag_kdn")]), args.steps, torch,
                             kdn, synth, "token")
        else:
            raise SystemExit(f"bench.py: unknown workload {w!r}")
        r["kernel_hash"] = kernel_hash()
        print(json.dumps(r), flush=True)
        return

    head = bench_prefill(HEADLINE, args.steps, args.warmup, torch, kdn, synth,
                         args.schedule)
    out = {
        "metric": METRIC, "value": head["value"], "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the workloads)",
        "config": dict(head["config"], parallelism="single GPU"),
        "roofline": head["roofline"], "mfma": head["mfma"],
    }
    # decode beside prefill: the metric's second half
    out["decode"] = bench_decode("decode_diag_kdn", 2, torch, kdn, synth)
    if args.workloads == "all":
        w = {}
        for name in ("gated_deltanet", "kda", "iso_kdn"):
            w[f"{name}_prefill"] = bench_prefill(name, max(3, args.steps // 2),
                                                 args.warmup, torch, kdn, synth,
                                                 args.schedule)
        for name in ("gated_deltanet", "kda", "diag_kdn", "iso_kdn"):
            w[f"{name}_backward"] = bench_backward(name, max(3, args.steps // 2),
                                                   args.warmup, torch, kdn, synth)
        w["verify16_diag_kdn"] = bench_verify(16, 20, torch, kdn, synth, "chunk")
        w["multi16_diag_kdn"] = bench_verify(16, 20, torch, kdn, synth, "token")
        out["workloads"] = w
    ach = measure_achievable(torch)
    out["achievable"] = ach
    # the same achieved rates against what this machine reaches on plain work
    for r in [out, out["decode"]] + list(out.get("workloads", {}).values()):
        rl = r["roofline"]
        base = ach["hbm_copy_GBs"] if rl["bound"] == "hbm" else None
        rl["frac_of_measured_copy"] = rl["achieved"] / base if base else None
        if r.get("mfma"):
            r["mfma"]["frac_of_measured_gemm"] = r["mfma"]["achieved"] / ach["bf16_gemm_TFLOPs"]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(HEADLINE, synth)
    out["kernel_hash"] = kernel_hash()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
