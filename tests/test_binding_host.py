"""Host-side checks of the Python binding's tensor validation (no GPU needed).

The C library sees only pointers and sizes, so the binding checks what a
pointer cannot carry -- shape, dtype, contiguity and that the memory is on the
GPU -- before any call into it.  Every call below must raise ValueError (or
TypeError) from those checks; none reaches the library's kernels.
"""
import pytest
import torch

from linear_attention_recurrent_delta_amd import kdn

B, T, H, DK, DV = 1, 8, 2, 64, 64


@pytest.fixture(scope="module", autouse=True)
def _lib():
    kdn.ensure_built()


def _prefill_inputs(variant="diag_kdn", dtype=torch.bfloat16):
    z = lambda *s, dt=dtype: torch.zeros(s, dtype=dt)
    inp = dict(q=z(B, T, H, DK), k=z(B, T, H, DK), v=z(B, T, H, DV))
    if variant == "gated_deltanet":
        inp.update(alpha=z(B, T, H), beta=z(B, T, H))
    elif variant == "kda":
        inp.update(alpha=z(B, T, H, DK), beta=z(B, T, H))
    else:
        inp.update(alpha=z(B, T, H, DK), proc_noise=z(B, T, H, DK), obs_noise=z(B, T, H),
                   p0=torch.ones(B, H, DK) if variant == "diag_kdn" else torch.ones(B, H))
    return inp


def _call_prefill(variant, inp):
    return kdn.prefill(variant, inp.pop("q"), inp.pop("k"), inp.pop("v"), **inp)


def test_prefill_host_tensors_rejected():
    with pytest.raises(ValueError, match="GPU memory"):
        _call_prefill("diag_kdn", _prefill_inputs())


@pytest.mark.parametrize("variant,key,bad,what", [
    ("diag_kdn", "k", torch.zeros(B, T, H, DK + 1, dtype=torch.bfloat16), "shape"),
    ("diag_kdn", "p0", torch.ones(B, H), "shape"),
    ("diag_kdn", "p0", torch.ones(B, H, DK, dtype=torch.float64), "dtype"),
    ("diag_kdn", "alpha", torch.zeros(B, T, H, DK), "dtype"),
    ("diag_kdn", "obs_noise", torch.zeros(B, T, H, 1, dtype=torch.bfloat16), "shape"),
    ("iso_kdn", "p0", torch.ones(B, H, DK), "shape"),
    ("gated_deltanet", "alpha", torch.zeros(B, T, H, DK, dtype=torch.bfloat16), "shape"),
    ("gated_deltanet", "beta", torch.zeros(B, T, H), "dtype"),
    ("kda", "S0", torch.zeros(B, H, DK, DV, dtype=torch.bfloat16), "dtype"),
    ("kda", "S0", torch.zeros(B, H, DV, DK + 64), "shape"),
    ("kda", "v", torch.zeros(B, T, H, 2 * DV, dtype=torch.bfloat16)[..., ::2], "contiguous"),
])
def test_prefill_bad_tensor(variant, key, bad, what):
    inp = _prefill_inputs(variant)
    inp[key] = bad
    with pytest.raises(ValueError, match=what):
        _call_prefill(variant, inp)


def test_prefill_bad_output():
    inp = _prefill_inputs("kda")
    o = torch.empty(B, T, H, DV, dtype=torch.float32)          # must be q's dtype
    S = torch.empty(B, H, DK, DV)
    with pytest.raises(ValueError, match="dtype"):
        kdn.prefill("kda", inp["q"], inp["k"], inp["v"], alpha=inp["alpha"],
                    beta=inp["beta"], out=(o, S, None))


def test_decode_checks():
    z = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt)
    N = 3
    args = dict(alpha=z(N, H, DK), proc_noise=z(N, H, DK), obs_noise=z(N, H))
    S, p = torch.zeros(N, H, DK, DV), torch.ones(N, H, DK)
    with pytest.raises(ValueError, match="GPU memory"):
        kdn.decode("diag_kdn", z(N, H, DK), z(N, H, DK), z(N, H, DV), S, p, **args)
    with pytest.raises(ValueError, match="shape"):
        kdn.decode("diag_kdn", z(N, H, DK), z(N, H, DK), z(N, H, DV), S, torch.ones(N, H),
                   **args)
    with pytest.raises(ValueError, match="dtype"):
        kdn.decode("diag_kdn", z(N, H, DK), z(N, H, DK), z(N, H, DV), S.double(), p, **args)


def test_decode_multi_checks():
    z = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt)
    N, TT = 2, 3
    with pytest.raises(ValueError, match="dtype"):
        kdn.decode_multi("kda", z(N, TT, H, DK), z(N, TT, H, DK), z(N, TT, H, DV),
                         alpha=z(N, TT, H, DK), beta=z(N, TT, H),
                         S0=torch.zeros(N, H, DK, DV, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="shape"):
        kdn.decode_multi("kda", z(N, TT, H, DK), z(N, TT, H, DK), z(N, TT, H, DV),
                         alpha=z(N, TT + 1, H, DK), beta=z(N, TT, H))
    with pytest.raises(ValueError, match="GPU memory"):
        kdn.decode_multi("kda", z(N, TT, H, DK), z(N, TT, H, DK), z(N, TT, H, DV),
                         alpha=z(N, TT, H, DK), beta=z(N, TT, H))


def test_backward_checks():
    inp = _prefill_inputs("gated_deltanet")
    d_o = torch.zeros(B, T, H, DV, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="dtype"):
        kdn.prefill_backward("gated_deltanet", inp["q"], inp["k"], inp["v"], d_o,
                             alpha=inp["alpha"], beta=inp["beta"],
                             dS_out=torch.zeros(B, H, DK, DV, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="shape"):
        kdn.prefill_backward("gated_deltanet", inp["q"], inp["k"], inp["v"], d_o[:, :4],
                             alpha=inp["alpha"], beta=inp["beta"])
    with pytest.raises(ValueError, match="GPU memory"):
        kdn.prefill_backward("gated_deltanet", inp["q"], inp["k"], inp["v"], d_o,
                             alpha=inp["alpha"], beta=inp["beta"])


def test_raw_entry_point_rejects_host_tensor():
    x = torch.zeros(4)
    with pytest.raises(ValueError, match="GPU memory"):
        kdn._ptr(x)
