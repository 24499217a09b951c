"""Short bf16 prefills (T <= 16 tokens per sequence) on the GPU.

kdn_chunk_prefill sends these to the one-workgroup-per-head kernel (chunks of
16 tokens, state in MFMA accumulators), whatever the schedule asked for.  It
is checked here against the fp64 oracle like every prefill (bf16 tolerance),
over every variant and head size, the exact-decay path (alpha = 0, strong
decay), the KDN degenerate values, in-place state, and at the size of
checking 16 draft tokens of the decode workload (256 sequences x 32 heads),
where it is also compared with the token-by-token multi-token decode.
"""
import pytest
import torch

from gpu_util import TOL, check, compare_prefill, gpu_prefill, log, np64
from linear_attention_recurrent_delta_amd import kdn, synth

pytestmark = pytest.mark.gpu

VARIANTS = ["deltanet", "gated_deltanet", "kda", "diag_kdn", "iso_kdn"]
DECAYING = ["gated_deltanet", "kda", "diag_kdn", "iso_kdn"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kdn.ensure_built()
    yield


def _inputs(variant, B, T, H, dk=128, dv=128, seed=0):
    return synth.gen_prefill(variant, B, T, H, dk, dv, "bf16", seed=seed, device="cuda",
                             random_state=True)


CASES = [(v, T, dk, dv) for v in VARIANTS for T in (1, 7, 16)
         for (dk, dv) in ((128, 128), (64, 64), (128, 64), (64, 128))]


@pytest.mark.parametrize("variant,T,dk,dv", CASES,
                         ids=[f"{v}-T{t}-k{a}v{b}" for v, t, a, b in CASES])
def test_short_prefill_parity(variant, T, dk, dv):
    log(f"short prefill {variant} T={T} dk={dk} dv={dv} B3 H5")
    inp = _inputs(variant, 3, T, 5, dk, dv, seed=200 + T)
    compare_prefill(variant, inp, gpu_prefill(variant, inp), TOL["bf16"])


@pytest.mark.parametrize("variant", DECAYING)
def test_short_prefill_exact_decay(variant):
    """alpha = 0 on a token, and a decay whose product over the 16 tokens
    drops below 2^-90: the chunk's A matrices take the exact path."""
    log(f"short prefill exact decay {variant}")
    inp = _inputs(variant, 2, 16, 3, seed=210)
    a = inp["alpha"].float()
    a[0, 5] = 0.0
    a[1] = 1e-6                          # (1e-6)^16 = 1e-96
    inp["alpha"] = a.to(inp["alpha"].dtype)
    compare_prefill(variant, inp, gpu_prefill(variant, inp), TOL["bf16"])


@pytest.mark.parametrize("variant", ["diag_kdn", "iso_kdn"])
def test_short_prefill_kdn_degenerate(variant):
    log(f"short prefill {variant}: r = 0 tokens, p0 = xi = 0, mu = d_k")
    inp = _inputs(variant, 2, 12, 3, seed=220)
    e = dict(inp)
    r = inp["r"].clone()
    r[:, 3] = 0
    r[:, 11] = 0
    e["r"] = r
    compare_prefill(variant, e, gpu_prefill(variant, e), TOL["bf16"])
    z = dict(inp)
    z["p0"] = torch.zeros_like(inp["p0"])
    z["xi"] = torch.zeros_like(inp["xi"])
    o, S, p = gpu_prefill(variant, z)
    assert torch.count_nonzero(p).item() == 0
    compare_prefill(variant, z, (o, S, p), TOL["bf16"])
    compare_prefill(variant, inp, gpu_prefill(variant, inp, mu=128.0), TOL["bf16"],
                    mu=128.0)


@pytest.mark.parametrize("variant", VARIANTS)
def test_short_prefill_state_in_place(variant):
    log(f"short prefill S_out is S0, p_out is p0 {variant}")
    inp = _inputs(variant, 2, 16, 4, seed=230)
    o_ref, S_ref, p_ref = gpu_prefill(variant, inp)
    S = inp["S0"].clone()
    p = inp["p0"].clone() if inp.get("p0") is not None else None
    o = torch.empty_like(o_ref)
    inp2 = dict(inp)
    inp2["S0"], inp2["p0"] = S, p
    gpu_prefill(variant, inp2, out=(o, S, p))
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    if p is not None:
        assert torch.equal(p, p_ref)


def test_short_prefill_verify_workload():
    """16 draft tokens for each of 256 sequences x 32 heads (diagonal KDN,
    d = 128) from a resident state: sampled heads against the oracle, and every
    output against the token-by-token multi-token decode of the same tokens."""
    c = synth.CONFIGS["decode_diag_kdn"]
    N, H, T = c["N"], c["H"], 16
    log(f"short prefill verify workload N{N} H{H} T{T}")
    inp = _inputs("diag_kdn", N, T, H, c["dk"], c["dv"], seed=240)
    o, S, p = gpu_prefill("diag_kdn", inp)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    assert torch.isfinite(p).all() and (p >= 0).all()
    compare_prefill("diag_kdn", inp, (o, S, p), TOL["bf16"],
                    heads=[(0, 0), (255, 31), (97, 12)], label="verify")
    om, Sm, pm = kdn.decode_multi("diag_kdn", inp["q"], inp["k"], inp["v"],
                                  alpha=inp["alpha"], proc_noise=inp["xi"],
                                  obs_noise=inp["r"], S0=inp["S0"], p0=inp["p0"])
    torch.cuda.synchronize()
    check("o vs multi-token decode", np64(o), np64(om), TOL["bf16"])
    check("S vs multi-token decode", np64(S), np64(Sm), TOL["bf16"])
    check("p vs multi-token decode", np64(p), np64(pm), TOL["bf16"])
