"""Gradients of the chunkwise prefill on the GPU (kdn_chunk_prefill_backward)
against the fp64 oracle's reverse-mode backward.

Every case draws seeded inputs and cotangents (dO, dS_out), runs the library,
runs the oracle on exactly the same rounded values, and compares each
gradient tensor (dq, dk, dv, dlog_alpha, dbeta, dS0) by
max|gpu - ref| / max|ref| against TOL (1e-4 for float32 inputs, 2e-2 for
bfloat16 inputs with float32 state, as for the forward pass).  The oracle's
decay gradient dL/dalpha is compared as alpha * dL/dalpha, the quantity the
library returns.
"""
import pytest
import torch

import oracle
from gpu_util import TOL, check, log, np64
from linear_attention_recurrent_delta_amd import kdn, synth

pytestmark = pytest.mark.gpu

VARIANTS = ["deltanet", "gated_deltanet", "kda"]
NAMES = ("q", "k", "v", "log_alpha", "beta", "S0")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kdn.ensure_built()
    yield


def _inputs(variant, B, T, H, dk, dv, dtype, seed, state=True, ds=True):
    inp = synth.gen_prefill(variant, B, T, H, dk, dv, dtype, seed=seed, device="cuda",
                            random_state=state)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 7)
    inp["dO"] = torch.randn((B, T, H, dv), generator=g, device="cuda").to(inp["q"].dtype)
    inp["dS"] = torch.randn((B, H, dk, dv), generator=g, device="cuda") if ds else None
    return inp


def _ref(variant, inp, heads=None):
    f = lambda x: None if x is None else np64(x)
    sl = lambda x, b, h, state: None if x is None else (
        x[b:b + 1, h:h + 1] if state else x[b:b + 1, :, h:h + 1])
    if heads is None:
        parts = [(inp, None)]
    else:
        parts = [({k: sl(v, b, h, k in ("S0", "dS")) for k, v in inp.items()}, (b, h))
                 for (b, h) in heads]
    out = []
    for x, key in parts:
        dq, dk, dv, da, db, dS0 = oracle.backward(
            variant, f(x["q"]), f(x["k"]), f(x["v"]), f(x.get("alpha")), f(x["beta"]),
            f(x.get("S0")), f(x["dO"]), f(x.get("dS")))
        if da is not None:
            da = da * f(x["alpha"])
        out.append((key, dict(zip(NAMES, (dq, dk, dv, da, db, dS0)))))
    return out


def _gpu(variant, inp, chunk=0):
    got = kdn.prefill_backward(variant, inp["q"], inp["k"], inp["v"], inp["dO"],
                               alpha=inp.get("alpha"), beta=inp.get("beta"),
                               S0=inp.get("S0"), dS_out=inp.get("dS"), chunk=chunk)
    torch.cuda.synchronize()
    return {n: got["d" + n] for n in NAMES}


def _compare(variant, inp, tol, chunk=0, heads=None):
    got = _gpu(variant, inp, chunk)
    for n in NAMES:
        if got[n] is not None:
            assert torch.isfinite(got[n]).all(), f"d{n} not finite"
    for key, ref in _ref(variant, inp, heads):
        for n in NAMES:
            if ref[n] is None:
                assert got[n] is None
                continue
            g = got[n]
            if key is not None:
                b, h = key
                g = g[b:b + 1, h:h + 1] if n == "S0" else g[b:b + 1, :, h:h + 1]
            check(f"d{n}" + ("" if key is None else f"[b={key[0]},h={key[1]}]"),
                  np64(g), ref[n], tol)


CASES = [(v, dt, dk, dv) for v in VARIANTS for dt in ("bf16", "f32")
         for (dk, dv) in ((128, 128), (64, 64), (128, 64), (64, 128))]


@pytest.mark.parametrize("variant,dtype,dk,dv", CASES,
                         ids=[f"{v}-{d}-k{a}v{b}" for v, d, a, b in CASES])
def test_backward_small(variant, dtype, dk, dv):
    log(f"backward {variant} {dtype} dk={dk} dv={dv} B2 T200 H2")
    inp = _inputs(variant, 2, 200, 2, dk, dv, dtype, seed=101)
    _compare(variant, inp, TOL[dtype])


@pytest.mark.parametrize("variant", VARIANTS)
def test_backward_chunk32(variant):
    log(f"backward chunk 32 {variant} bf16")
    inp = _inputs(variant, 1, 150, 3, 128, 128, "bf16", seed=102)
    _compare(variant, inp, TOL["bf16"], chunk=32)


@pytest.mark.parametrize("T", [0, 1, 2, 63, 64, 65, 129])
@pytest.mark.parametrize("variant,dtype", [("gated_deltanet", "bf16"), ("kda", "f32")])
def test_backward_lengths(variant, dtype, T):
    log(f"backward length T={T} {variant} {dtype}")
    inp = _inputs(variant, 2, T, 2, 128, 128 if dtype == "bf16" else 64, dtype, seed=103 + T)
    _compare(variant, inp, TOL[dtype])


@pytest.mark.parametrize("variant", VARIANTS)
def test_backward_without_state_cotangent(variant):
    log(f"backward S0 = NULL, dS_out = NULL {variant}")
    inp = _inputs(variant, 2, 140, 2, 128, 128, "bf16", seed=104, state=False, ds=False)
    _compare(variant, inp, TOL["bf16"])


@pytest.mark.parametrize("variant", ["gated_deltanet", "kda"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_alpha_zero(variant, dtype):
    """alpha = 0 on some tokens: those chunks take the exact elementwise path."""
    log(f"backward alpha=0 {variant} {dtype}")
    inp = _inputs(variant, 1, 200, 2, 64, 64, dtype, seed=105)
    a = inp["alpha"].float()
    a[:, 10] = 0.0
    a[:, 100:103] = 0.0
    if a.dim() == 4:
        a[:, 150, :, :32] = 0.0
    inp["alpha"] = a.to(inp["alpha"].dtype)
    _compare(variant, inp, TOL[dtype])


@pytest.mark.parametrize("variant", ["gated_deltanet", "kda"])
def test_backward_strong_decay(variant):
    """A chunk whose cumulative decay drops below 2^-90."""
    log(f"backward strong decay {variant}")
    inp = _inputs(variant, 1, 192, 2, 128, 128, "bf16", seed=106)
    a = inp["alpha"].float()
    a[:, 64:128] = 0.2
    inp["alpha"] = a.to(inp["alpha"].dtype)
    _compare(variant, inp, TOL["bf16"])


def test_backward_workload_sampled():
    """Gated DeltaNet workload (B4 H16 T4096, d = 128, bf16): every head on the
    GPU, sampled heads against the oracle at full length."""
    c = synth.CONFIGS["gated_deltanet"]
    log(f"backward workload gated_deltanet B{c['B']} H{c['H']} T{c['T']}: sampled heads")
    inp = _inputs("gated_deltanet", c["B"], c["T"], c["H"], c["dk"], c["dv"], c["dtype"],
                  seed=synth.seed_of("gated_deltanet"), state=False)
    _compare("gated_deltanet", inp, TOL["bf16"], heads=[(0, 0), (3, 15)])


# ---------------------------------------------------------------------------
# KDN: the memory part with the derived write vectors (isotropic: beta k from
# the head variance; diagonal: the gain), then the variance chain (gradients
# of xi, r, p0 and the extra alpha, k terms).
# ---------------------------------------------------------------------------
KDN_NAMES = ("q", "k", "v", "log_alpha", "proc_noise", "obs_noise", "S0", "p0")
KDNS = ["diag_kdn", "iso_kdn"]


def _kdn_inputs(variant, B, T, H, dk, dv, dtype, seed, state=True, ds=True):
    inp = _inputs(variant, B, T, H, dk, dv, dtype, seed, state=state, ds=ds)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 11)
    inp["dp"] = torch.randn(tuple(inp["p0"].shape), generator=g, device="cuda") if ds else None
    return inp


def _kdn_compare(variant, inp, tol, mu=1.0, chunk=0, heads=None):
    got = kdn.prefill_backward(variant, inp["q"], inp["k"], inp["v"], inp["dO"],
                               alpha=inp["alpha"], proc_noise=inp["xi"], obs_noise=inp["r"],
                               S0=inp.get("S0"), p0=inp["p0"], dS_out=inp.get("dS"),
                               dp_out=inp.get("dp"), mu=mu, chunk=chunk)
    torch.cuda.synchronize()
    got = {n: got["d" + n] for n in KDN_NAMES}
    for n in KDN_NAMES:
        assert torch.isfinite(got[n]).all(), f"d{n} not finite"
    f = lambda x: None if x is None else np64(x)
    ref_fn = oracle.backward_iso if variant == "iso_kdn" else oracle.backward_diag
    if heads is None:
        parts = [(inp, None)]
    else:
        sl = lambda x, b, h, st: None if x is None else (
            x[b:b + 1, h:h + 1] if st else x[b:b + 1, :, h:h + 1])
        parts = [({k: sl(v, b, h, k in ("S0", "dS", "p0", "dp")) for k, v in inp.items()},
                  (b, h)) for (b, h) in heads]
    for x, key in parts:
        ref = ref_fn(f(x["q"]), f(x["k"]), f(x["v"]), f(x["alpha"]), f(x["xi"]), f(x["r"]),
                     f(x["p0"]), f(x.get("S0")), f(x["dO"]), f(x.get("dS")), f(x.get("dp")),
                     mu=mu)
        ref = dict(zip(KDN_NAMES, ref))
        ref["log_alpha"] = ref["log_alpha"] * f(x["alpha"])
        for n in KDN_NAMES:
            g = got[n]
            if key is not None:
                b, h = key
                g = g[b:b + 1, h:h + 1] if n in ("S0", "p0") else g[b:b + 1, :, h:h + 1]
            check(f"d{n}" + ("" if key is None else f"[b={key[0]},h={key[1]}]"),
                  np64(g), ref[n], tol)


KDN_CASES = [(v, dt, dk, dv) for v in KDNS for dt in ("bf16", "f32")
             for (dk, dv) in ((128, 128), (64, 64), (128, 64), (64, 128))]


@pytest.mark.parametrize("variant,dtype,dk,dv", KDN_CASES,
                         ids=[f"{v}-{d}-k{a}v{b}" for v, d, a, b in KDN_CASES])
def test_backward_kdn_small(variant, dtype, dk, dv):
    log(f"backward {variant} {dtype} dk={dk} dv={dv} B2 T200 H2")
    _kdn_compare(variant, _kdn_inputs(variant, 2, 200, 2, dk, dv, dtype, seed=111), TOL[dtype])


@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 130])
@pytest.mark.parametrize("variant", KDNS)
def test_backward_kdn_lengths(variant, T):
    log(f"backward {variant} length T={T}")
    _kdn_compare(variant, _kdn_inputs(variant, 2, T, 2, 128, 128, "bf16", seed=112 + T),
                 TOL["bf16"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("variant", KDNS)
def test_backward_kdn_mu_and_exact_observations(variant, dtype):
    log(f"backward {variant} mu = d_k, r = 0 on some tokens {dtype}")
    inp = _kdn_inputs(variant, 1, 180, 2, 128, 128 if dtype == "bf16" else 64, dtype,
                      seed=113)
    r = inp["r"].clone()
    r[:, 7] = 0
    r[:, 64:66] = 0
    inp["r"] = r
    _kdn_compare(variant, inp, TOL[dtype], mu=128.0)


@pytest.mark.parametrize("variant", KDNS)
def test_backward_kdn_without_cotangents(variant):
    log(f"backward {variant} S0, dS_out, dp_out = NULL")
    _kdn_compare(variant, _kdn_inputs(variant, 2, 150, 2, 128, 128, "bf16", seed=114,
                                      state=False, ds=False), TOL["bf16"])


@pytest.mark.parametrize("variant", KDNS)
def test_backward_kdn_long_sampled(variant):
    """KDN at the workload's heads and head size (B2 H16, d = 128, bf16) over
    2048 tokens: every head on the GPU, sampled heads against the oracle
    (whose backward keeps every memory of a stream)."""
    log(f"backward {variant} B2 H16 T2048: sampled heads")
    inp = _kdn_inputs(variant, 2, 2048, 16, 128, 128, "bf16", seed=synth.seed_of(variant))
    _kdn_compare(variant, inp, TOL["bf16"], heads=[(0, 0), (1, 9)])


# ---------------------------------------------------------------------------
# The gradient workloads bench.py times (KDA B2 H32 T8192; diagonal and
# isotropic KDN B2 H16 T16384; d = 128, bf16, default chunk and workspace),
# with exactly its inputs and dO: every head on the GPU, two sampled heads
# against the oracle at full length.
BENCH_BWD = ("kda", "diag_kdn", "iso_kdn")


@pytest.mark.parametrize("name", BENCH_BWD)
def test_backward_bench_workload_sampled(name):
    c = synth.CONFIGS[name]
    B, T, H, dv = c["B"], c["T"], c["H"], c["dv"]
    log(f"backward workload {name} B{B} H{H} T{T}: sampled heads")
    inp = synth.gen_config(name, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(synth.seed_of(name) + 7)
    inp["dO"] = torch.randn((B, T, H, dv), generator=g, device="cuda").to(inp["q"].dtype)
    inp["dS"] = None
    heads = [(0, 0), (B - 1, H - 1)]
    if name == "kda":
        _compare(name, inp, TOL["bf16"], heads=heads)
    else:
        inp["dp"] = None
        _kdn_compare(name, inp, TOL["bf16"], heads=heads)


@pytest.mark.parametrize("variant", KDNS)
def test_backward_kdn_chunk32(variant):
    """The KDN chain kernels at a chunk of 32 (bf16, d = 128), over several
    chunks and a ragged tail."""
    log(f"backward {variant} chunk 32 B2 T200 H2")
    _kdn_compare(variant, _kdn_inputs(variant, 2, 200, 2, 128, 128, "bf16", seed=131),
                 TOL["bf16"], chunk=32)
