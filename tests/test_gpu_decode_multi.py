"""Multi-token decode (kdn_recurrent_decode_multi) on the GPU.

Its inputs are laid out like a prefill batch ([N, T, H, .]) and its result is
the recurrence run token by token from a resident state, so the fp64 oracle
of the prefill checks it directly, per output tensor, against 1e-4 (float32)
or 2e-2 (bfloat16 inputs, float32 state).  Beyond the oracle it must give the
same bits as T single-token decode steps (the same arithmetic per token), leave
S0 / p0 untouched when the outputs go elsewhere (the rollback of a rejected
draft), update in place when they are the same buffers, and pass the state
through for T = 0.
"""
import pytest
import torch

from gpu_util import TOL, compare_prefill, log
from linear_attention_recurrent_delta_amd import kdn, synth

pytestmark = pytest.mark.gpu

VARIANTS = ["deltanet", "gated_deltanet", "kda", "diag_kdn", "iso_kdn"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kdn.ensure_built()
    yield


def _inputs(variant, N, T, H, dk, dv, dtype, seed):
    return synth.gen_prefill(variant, N, T, H, dk, dv, dtype, seed=seed, device="cuda",
                             random_state=True)


def _multi(variant, inp, mu=1.0, out=None, S0="input"):
    o, S, p = kdn.decode_multi(variant, inp["q"], inp["k"], inp["v"],
                               alpha=inp.get("alpha"), beta=inp.get("beta"),
                               proc_noise=inp.get("xi"), obs_noise=inp.get("r"),
                               S0=inp.get("S0") if S0 == "input" else S0,
                               p0=inp.get("p0"), mu=mu, out=out)
    torch.cuda.synchronize()
    return o, S, p


def _token(x, t):
    return None if x is None else x[:, t].contiguous()


CASES = [(v, dt, dk, dv) for v in VARIANTS for dt in ("bf16", "f32")
         for (dk, dv) in ((128, 128), (64, 64), (128, 64), (64, 128))]


@pytest.mark.parametrize("variant,dtype,dk,dv", CASES,
                         ids=[f"{v}-{d}-k{a}v{b}" for v, d, a, b in CASES])
def test_decode_multi_parity(variant, dtype, dk, dv):
    log(f"decode_multi {variant} {dtype} dk={dk} dv={dv} N3 T5 H2")
    inp = _inputs(variant, 3, 5, 2, dk, dv, dtype, seed=31)
    S0 = inp["S0"].clone()
    p0 = inp["p0"].clone() if inp.get("p0") is not None else None
    got = _multi(variant, inp)
    compare_prefill(variant, inp, got, TOL[dtype])
    # the resident state is untouched: rolling back a rejected draft is free
    assert torch.equal(inp["S0"], S0)
    if p0 is not None:
        assert torch.equal(inp["p0"], p0)


@pytest.mark.parametrize("T", [1, 2, 16, 33])
@pytest.mark.parametrize("variant", VARIANTS)
def test_decode_multi_lengths(variant, T):
    log(f"decode_multi {variant} bf16 T={T}")
    inp = _inputs(variant, 4, T, 3, 128, 128, "bf16", seed=40 + T)
    compare_prefill(variant, inp, _multi(variant, inp), TOL["bf16"])


@pytest.mark.parametrize("variant", VARIANTS)
def test_decode_multi_zero_tokens_passes_state(variant):
    log(f"decode_multi {variant} T=0")
    inp = _inputs(variant, 3, 0, 2, 128, 128, "bf16", seed=50)
    o, S, p = _multi(variant, inp)
    assert o.numel() == 0
    assert torch.equal(S, inp["S0"])
    if p is not None:
        assert torch.equal(p, inp["p0"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_decode_multi_equals_decode_steps_bitwise(variant, dtype):
    """Token t of a multi-token call equals the t-th single-token decode."""
    log(f"decode_multi vs {7} decode steps {variant} {dtype}")
    N, T, H = 4, 7, 3
    inp = _inputs(variant, N, T, H, 128, 128, dtype, seed=60)
    o, S, p = _multi(variant, inp)
    S1 = inp["S0"].clone()
    p1 = inp["p0"].clone() if inp.get("p0") is not None else None
    for t in range(T):
        ot = kdn.decode(variant, _token(inp["q"], t), _token(inp["k"], t),
                        _token(inp["v"], t), S1, p1, alpha=_token(inp.get("alpha"), t),
                        beta=_token(inp.get("beta"), t), proc_noise=_token(inp.get("xi"), t),
                        obs_noise=_token(inp.get("r"), t))
        torch.cuda.synchronize()
        assert torch.equal(ot, o[:, t]), f"o differs at token {t}"
    assert torch.equal(S1, S)
    if p is not None:
        assert torch.equal(p1, p)


@pytest.mark.parametrize("variant", VARIANTS)
def test_decode_multi_in_place(variant):
    log(f"decode_multi in place {variant}")
    inp = _inputs(variant, 3, 6, 2, 128, 128, "bf16", seed=70)
    o_ref, S_ref, p_ref = _multi(variant, inp)
    S = inp["S0"].clone()
    p = inp["p0"].clone() if inp.get("p0") is not None else None
    o = torch.empty_like(o_ref)
    inp2 = dict(inp)
    inp2["S0"], inp2["p0"] = S, p
    _multi(variant, inp2, out=(o, S, p))
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    if p is not None:
        assert torch.equal(p, p_ref)


@pytest.mark.parametrize("variant", ["gated_deltanet", "diag_kdn", "iso_kdn"])
def test_decode_multi_null_state_is_zero(variant):
    log(f"decode_multi S0 = NULL {variant}")
    inp = _inputs(variant, 2, 4, 2, 128, 128, "bf16", seed=80)
    a = _multi(variant, inp, S0=None)
    b = _multi(variant, inp, S0=torch.zeros_like(inp["S0"]))
    for x, y in zip(a, b):
        assert (x is None and y is None) or torch.equal(x, y)


@pytest.mark.parametrize("variant", ["diag_kdn", "iso_kdn"])
def test_decode_multi_kdn_mu(variant):
    log(f"decode_multi {variant} mu = d_k")
    inp = _inputs(variant, 3, 9, 2, 128, 128, "f32", seed=90)
    compare_prefill(variant, inp, _multi(variant, inp, mu=128.0), TOL["f32"],
                    mu=128.0)


def test_decode_multi_verify_workload_sampled():
    """Verifying 16 draft tokens at the decode workload's size (256 sequences x
    32 heads, d = 128, bf16, diagonal KDN), sampled streams against the oracle."""
    c = synth.CONFIGS["decode_diag_kdn"]
    N, H, T = c["N"], c["H"], 16
    log(f"decode_multi workload N{N} H{H} T{T}: sampled heads")
    inp = _inputs("diag_kdn", N, T, H, c["dk"], c["dv"], c["dtype"], seed=95)
    o, S, p = _multi("diag_kdn", inp)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    assert torch.isfinite(p).all() and (p >= 0).all()
    compare_prefill("diag_kdn", inp, (o, S, p), TOL["bf16"],
                    heads=[(0, 0), (255, 31), (97, 12)], label="verify")
