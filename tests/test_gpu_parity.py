"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every case generates seeded inputs, runs the library on the GPU, runs the
oracle on exactly the same rounded values, and compares each output tensor
(o, S, p) by max|gpu - ref| / max|ref| against 1e-4 (float32 inputs) or 2e-2
(bfloat16 inputs, float32 state).  The full-size prefill workloads are
compared on every (batch, head) stream, in the launch configuration the
benchmark times; the full decode workload on 256 streams spread over all
sequences and heads.
"""
import numpy as np
import pytest
import torch

import gpu_util

from gpu_util import (TOL, check, compare_prefill, decode_inputs_as_prefill,
                      gpu_decode_run, gpu_prefill, log, np64, oracle_prefill,
                      to_device)
from linear_attention_recurrent_delta_amd import kdn, synth

pytestmark = pytest.mark.gpu

VARIANTS = ["deltanet", "gated_deltanet", "kda", "diag_kdn", "iso_kdn"]
KDNS = ("diag_kdn", "iso_kdn")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kdn.ensure_built()
    yield


@pytest.fixture(params=["two_pass", "single_pass"], autouse=True)
def schedule(request):
    """Every prefill case runs under both schedules of kdn_chunk_prefill."""
    gpu_util.SCHEDULE["workspace"] = "auto" if request.param == "two_pass" else None
    log(f"schedule {request.param}")
    yield request.param
    gpu_util.SCHEDULE["workspace"] = "auto"


def _inputs(variant, B, T, H, dk, dv, dtype, seed, random_state=True, device="cuda"):
    return synth.gen_prefill(variant, B, T, H, dk, dv, dtype, seed=seed,
                             device=device, random_state=random_state)


# ---------------------------------------------------------------------------
# Small cases: several chunks plus a ragged tail, every variant and dtype.
# ---------------------------------------------------------------------------
SMALL = [(v, dt, dk, dv) for v in VARIANTS for dt in ("bf16", "f32")
         for (dk, dv) in ((64, 64), (128, 128), (128, 64), (64, 128))]


@pytest.mark.parametrize("variant,dtype,dk,dv", SMALL,
                         ids=[f"{v}-{d}-k{a}v{b}" for v, d, a, b in SMALL])
def test_prefill_small(variant, dtype, dk, dv):
    log(f"prefill {variant} {dtype} dk={dk} dv={dv} B2 T200 H3")
    inp = _inputs(variant, 2, 200, 3, dk, dv, dtype, seed=11)
    got = gpu_prefill(variant, inp, mu=1.0)
    compare_prefill(variant, inp, got, TOL[dtype])


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_chunk32(variant, dtype):
    log(f"prefill chunk 32 {variant} {dtype}")
    inp = _inputs(variant, 1, 150, 4, 64, 64, dtype, seed=12)
    got = gpu_prefill(variant, inp, chunk=32)
    compare_prefill(variant, inp, got, TOL[dtype])


@pytest.mark.parametrize("T", [0, 1, 2, 15, 16, 63, 64, 65, 128, 129])
@pytest.mark.parametrize("variant,dtype", [("diag_kdn", "bf16"), ("deltanet", "f32"),
                                           ("kda", "bf16"), ("iso_kdn", "bf16"),
                                           ("iso_kdn", "f32")])
def test_prefill_lengths(variant, dtype, T):
    log(f"prefill length T={T} {variant} {dtype}")
    inp = _inputs(variant, 2, T, 2, 128, 128, dtype, seed=13 + T)
    got = gpu_prefill(variant, inp)
    compare_prefill(variant, inp, got, TOL[dtype])


@pytest.mark.parametrize("variant", KDNS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_kdn_mu(variant, dtype):
    for mu in (128.0, 0.25):
        log(f"prefill {variant} mu={mu} {dtype}")
        inp = _inputs(variant, 2, 300, 2, 128, 128, dtype, seed=14)
        got = gpu_prefill(variant, inp, mu=mu)
        compare_prefill(variant, inp, got, TOL[dtype], mu=mu)


@pytest.mark.parametrize("variant", ["gated_deltanet", "kda", "diag_kdn", "iso_kdn"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_alpha_zero(variant, dtype):
    """alpha = 0 (full erase) on some tokens: the chunks containing them take
    the exact-decay path."""
    log(f"prefill alpha=0 {variant} {dtype}")
    inp = _inputs(variant, 1, 200, 2, 64, 64, dtype, seed=15)
    a = inp["alpha"].float()
    a[:, 10] = 0.0
    a[:, 100:103] = 0.0
    if a.dim() == 4:
        a[:, 150, :, :32] = 0.0         # half the channels only
    inp["alpha"] = a.to(inp["alpha"].dtype)
    got = gpu_prefill(variant, inp)
    compare_prefill(variant, inp, got, TOL[dtype])


@pytest.mark.parametrize("variant", ["gated_deltanet", "kda", "diag_kdn", "iso_kdn"])
def test_prefill_strong_decay(variant):
    """A chunk whose cumulative decay drops below 2^-90 (tiny alpha)."""
    log(f"prefill strong decay {variant}")
    inp = _inputs(variant, 1, 192, 2, 128, 128, "bf16", seed=16)
    a = inp["alpha"].float()
    a[:, 64:128] = 0.2                   # 0.2^64 ~ 5e-45 within one chunk
    inp["alpha"] = a.to(inp["alpha"].dtype)
    got = gpu_prefill(variant, inp)
    compare_prefill(variant, inp, got, TOL["bf16"])


@pytest.mark.parametrize("variant", KDNS)
def test_prefill_kdn_degenerate_values(variant):
    log(f"prefill {variant} p0 = 0, xi = 0 (zero write); tiny r; r = 0")
    inp = _inputs(variant, 1, 130, 2, 128, 128, "bf16", seed=17)
    z = dict(inp)
    z["p0"] = torch.zeros_like(inp["p0"])
    z["xi"] = torch.zeros_like(inp["xi"])
    o, S, p = gpu_prefill(variant, z)
    assert torch.count_nonzero(p).item() == 0
    compare_prefill(variant, z, (o, S, p), TOL["bf16"])
    t = dict(inp)
    t["r"] = torch.full_like(inp["r"], 1e-6)
    compare_prefill(variant, t, gpu_prefill(variant, t), TOL["bf16"])
    # exact observations on a few tokens (r = 0, keys nonzero): the variance
    # drops to 0 there and the write replaces the value along k
    e = dict(inp)
    r = inp["r"].clone()
    r[:, 5] = 0
    r[:, 16] = 0          # first token of a 16-token segment of the prep's chain
    r[:, 47:49] = 0       # last and first tokens on either side of a segment start
    r[:, 64:67] = 0
    r[:, 129] = 0
    e["r"] = r
    compare_prefill(variant, e, gpu_prefill(variant, e), TOL["bf16"])


@pytest.mark.parametrize("variant", VARIANTS)
def test_prefill_state_in_place(variant, schedule):
    log(f"prefill S_out is S0 {variant}")
    inp = _inputs(variant, 2, 100, 2, 128, 128, "bf16", seed=18)
    ref = oracle_prefill(variant, inp)
    S = inp["S0"].clone()
    o = torch.empty((2, 100, 2, 128), dtype=torch.bfloat16, device="cuda")
    p = torch.empty_like(inp["p0"]) if variant in KDNS else None
    inp2 = dict(inp)
    inp2["S0"] = S
    gpu_prefill(variant, inp2, out=(o, S, p))
    check("o", np64(o), ref[0], TOL["bf16"])
    check("S (in place)", np64(S), ref[1], TOL["bf16"])
    if variant not in KDNS:
        return
    # p_out == p0 as well: allowed with a workspace (two-pass schedule),
    # refused by the single-pass schedule
    S = inp["S0"].clone()
    p = inp["p0"].clone()
    inp3 = dict(inp, S0=S, p0=p)
    if schedule == "single_pass":
        with pytest.raises(kdn.KdnError) as ei:
            gpu_prefill(variant, inp3, out=(o, S, p))
        assert ei.value.status == 5          # KDN_ERR_ALIAS
        return
    gpu_prefill(variant, inp3, out=(o, S, p))
    check("o (S and p in place)", np64(o), ref[0], TOL["bf16"])
    check("S (S and p in place)", np64(S), ref[1], TOL["bf16"])
    check("p (in place)", np64(p), ref[2], TOL["bf16"])


@pytest.mark.parametrize("variant", VARIANTS)
def test_prefill_continuation(variant):
    """prefill(T1) then prefill(T2) from its state equals prefill(T1 + T2)."""
    log(f"prefill continuation {variant}")
    inp = _inputs(variant, 2, 300, 2, 128, 128, "bf16", seed=19)
    o, S, p = gpu_prefill(variant, inp)
    first = {k: (v[:, :100].contiguous() if k not in ("S0", "p0") and v is not None
                 else v) for k, v in inp.items()}
    o1, S1, p1 = gpu_prefill(variant, first)
    second = {k: (v[:, 100:].contiguous() if k not in ("S0", "p0") and v is not None
                  else v) for k, v in inp.items()}
    second["S0"] = S1
    if p1 is not None:
        second["p0"] = p1
    o2, S2, p2 = gpu_prefill(variant, second)
    ref = oracle_prefill(variant, inp)
    check("o (two calls)", np.concatenate([np64(o1), np64(o2)], axis=1), ref[0],
          TOL["bf16"])
    check("S (two calls)", np64(S2), ref[1], TOL["bf16"])
    if p is not None:
        check("p (two calls)", np64(p2), ref[2], TOL["bf16"])


@pytest.mark.parametrize("variant", KDNS)
def test_prefill_deterministic(variant):
    log(f"prefill bitwise determinism {variant}")
    inp = _inputs(variant, 2, 500, 4, 128, 128, "bf16", seed=20)
    a = gpu_prefill(variant, inp)
    b = gpu_prefill(variant, inp)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------
DEC = [(v, dt, dk, dv) for v in VARIANTS for dt in ("bf16", "f32")
       for (dk, dv) in ((128, 128), (64, 64), (64, 128), (128, 64))]


@pytest.mark.parametrize("variant,dtype,dk,dv", DEC,
                         ids=[f"{v}-{d}-k{a}v{b}" for v, d, a, b in DEC])
def test_decode_small(variant, dtype, dk, dv):
    log(f"decode {variant} {dtype} dk={dk} dv={dv} N5 H3 20 steps")
    d = synth.gen_decode(5, 3, 20, dk, dv, dtype, seed=21, device="cuda",
                         variant=variant)
    g = torch.Generator(device="cuda").manual_seed(5)
    d["S0"] = 0.5 * torch.randn(d["S0"].shape, generator=g, device="cuda")
    if variant not in KDNS:
        d.pop("p0", None)
    os_, S, p = gpu_decode_run(variant, d)
    pre = decode_inputs_as_prefill(d)
    ro, rS, rp = oracle_prefill(variant, pre)
    check("o", np64(os_.transpose(0, 1)), ro, TOL[dtype])
    check("S", np64(S), rS, TOL[dtype])
    if rp is not None:
        check("p", np64(p), rp, TOL[dtype])


@pytest.mark.parametrize("variant", VARIANTS)
def test_prefill_equals_repeated_decode(variant):
    log(f"prefill vs decode {variant}")
    d = synth.gen_decode(3, 2, 70, 128, 128, "bf16", seed=22, device="cuda",
                         variant=variant)
    if variant not in KDNS:
        d.pop("p0", None)
    os_, S, p = gpu_decode_run(variant, d)
    pre = {k: (v.contiguous() if isinstance(v, torch.Tensor) else v)
           for k, v in decode_inputs_as_prefill(d).items()}
    o2, S2, p2 = gpu_prefill(variant, pre)
    check("o decode vs prefill", np64(os_.transpose(0, 1)), np64(o2), TOL["bf16"])
    check("S decode vs prefill", np64(S), np64(S2), TOL["bf16"])


# ---------------------------------------------------------------------------
# The workloads at full size.
# ---------------------------------------------------------------------------
def test_workload_deltanet_fp32_full():
    log("workload DeltaNet fp32 B1 H2 T256 d64: every output")
    inp = synth.gen_config("deltanet_fp32", device="cuda")
    got = gpu_prefill("deltanet", inp)
    compare_prefill("deltanet", inp, got, TOL["f32"])


# Oracle results of the full-size workloads, shared by the two schedules.
_FULL_REF = {}


def _full_ref(name, inp, variant):
    if name not in _FULL_REF:
        import time
        t0 = time.time()
        _FULL_REF[name] = oracle_prefill(variant, inp)
        log(f"  {name} oracle over every stream {time.time() - t0:.1f}s")
    return _FULL_REF[name]


def _check_every_stream(label, got, ref, tol):
    """Per (batch, head) stream: max|gpu - ref| / max|ref| of that stream.
    The first two axes of ``got``/``ref`` are (b, t) for o and (b, h) for S
    and p; ``head_axis`` picks the head axis."""
    worst, where = 0.0, None
    g = np.asarray(got, np.float64)
    for b in range(ref.shape[0]):
        for h in range(ref.shape[label[1]]):
            sl = (b, slice(None), h) if label[1] == 2 else (b, h)
            e = gpu_util.rel_err(g[sl], ref[sl])
            if e > worst:
                worst, where = e, (b, h)
    log(f"    {label[0]}: worst stream rel err {worst:.3e} at (b, h) = {where} "
        f"(tol {tol:.0e})")
    assert worst <= tol, f"{label[0]}: stream {where} relative error {worst:.3e} > {tol:.0e}"


@pytest.mark.parametrize("name", ["gated_deltanet", "kda", "diag_kdn", "iso_kdn"])
def test_workload_full_size_every_stream(name):
    """The workload at full size in the launch configuration the benchmark
    times; every (batch, head) stream compared with the oracle."""
    c = synth.CONFIGS[name]
    log(f"workload {name} B{c['B']} H{c['H']} T{c['T']}: every stream")
    inp = synth.gen_config(name, device="cuda")
    o, S, p = gpu_prefill(c["variant"], inp)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    if p is not None:
        assert torch.isfinite(p).all() and (p >= 0).all()
    ro, rS, rp = _full_ref(name, inp, c["variant"])
    tol = TOL[c["dtype"]]
    check("o (whole tensor)", np64(o), ro, tol)
    check("S (whole tensor)", np64(S), rS, tol)
    _check_every_stream(("o", 2), np64(o), ro, tol)
    _check_every_stream(("S", 1), np64(S), rS, tol)
    if rp is not None:
        check("p (whole tensor)", np64(p), rp, tol)
        _check_every_stream(("p", 1), np64(p), rp, tol)


def test_workload_decode_reduced_all_heads():
    log("workload decode diag_kdn reduced N16 H4 32 steps: every output")
    d = synth.gen_decode(16, 4, 32, 128, 128, "bf16", seed=synth.seed_of("decode_diag_kdn"),
                         device="cuda")
    os_, S, p = gpu_decode_run("diag_kdn", d)
    ro, rS, rp = oracle_prefill("diag_kdn", decode_inputs_as_prefill(d))
    check("o", np64(os_.transpose(0, 1)), ro, TOL["bf16"])
    check("S", np64(S), rS, TOL["bf16"])
    check("p", np64(p), rp, TOL["bf16"])


def test_workload_decode_full_size_sampled():
    """The decode workload at full size (256 sequences x 32 heads, 1024
    steps): 256 (sequence, head) streams, one per sequence with the heads
    spread over all 32, so every workgroup slot position is covered."""
    c = synth.CONFIGS["decode_diag_kdn"]
    log(f"workload decode diag_kdn N{c['N']} H{c['H']} {c['steps']} steps: 256 streams")
    d = synth.gen_decode(c["N"], c["H"], c["steps"], c["dk"], c["dv"], c["dtype"],
                         seed=synth.seed_of("decode_diag_kdn"), device="cuda")
    os_, S, p = gpu_decode_run("diag_kdn", d)
    assert torch.isfinite(S).all() and torch.isfinite(p).all()
    ns = torch.arange(c["N"], device="cuda")
    hs = (ns * 13 + 5) % c["H"]
    # [steps, 256, 1, ...]: sequence n with its head hs[n] as a one-head batch
    sub = {k: (v[:, ns, hs].unsqueeze(2) if k not in ("S0", "p0")
               else v[ns, hs].unsqueeze(1)) for k, v in d.items()}
    ro, rS, rp = oracle_prefill("diag_kdn", decode_inputs_as_prefill(sub))
    go = os_[:, ns, hs].unsqueeze(2).transpose(0, 1)
    check("o (256 streams)", np64(go), ro, TOL["bf16"])
    check("S (256 streams)", np64(S[ns, hs].unsqueeze(1)), rS, TOL["bf16"])
    check("p (256 streams)", np64(p[ns, hs].unsqueeze(1)), rp, TOL["bf16"])
    _check_every_stream(("o", 2), np64(go), ro, TOL["bf16"])
    _check_every_stream(("S", 1), np64(S[ns, hs].unsqueeze(1)), rS, TOL["bf16"])
