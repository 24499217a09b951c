"""kdn_chunk_prefill_noalloc (the two-pass prefill on the library's static
scratch) against kdn_chunk_prefill with a caller-owned workspace, through the
C ABI, on two calls in a row: the full diagonal-KDN workload (B2 H16 T16384,
run in segments because its workspace exceeds the scratch), then a smaller
Gated DeltaNet call that fits in one piece.  Tolerance: the bf16 bar,
max|a - b| / max|b| <= 2e-2 per output tensor."""
import pytest
import torch

from gpu_util import TOL, check, log, np64
from linear_attention_recurrent_delta_amd import kdn, synth

pytestmark = pytest.mark.gpu


def _run(variant, inp, noalloc):
    q, v = inp["q"], inp["v"]
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    vid = kdn.VARIANTS[variant]
    o = torch.full((B, T, H, dv), float("nan"), dtype=q.dtype, device="cuda")
    S = torch.full((B, H, dk, dv), float("nan"), device="cuda")
    p = None if inp.get("p0") is None else torch.full_like(inp["p0"], float("nan"))
    args = (vid, kdn.DTYPES[q.dtype], B, T, H, dk, dv, 0, 1.0, q, inp["k"], v,
            inp.get("alpha"), inp.get("beta"), inp.get("xi"), inp.get("r"),
            inp.get("S0"), inp.get("p0"), o, S, p)
    if noalloc:
        kdn.kdn_chunk_prefill_noalloc(*args)
    else:
        ws = kdn.workspace(vid, q, v)
        kdn.kdn_chunk_prefill(*args, workspace=ws)
    torch.cuda.synchronize()
    return o, S, p


def _compare(variant, inp):
    ref = _run(variant, inp, noalloc=False)
    got = _run(variant, inp, noalloc=True)
    for name, g, r in zip(("o", "S", "p"), got, ref):
        if r is None:
            continue
        assert torch.isfinite(g.float()).all(), f"{name}: not every element written"
        check(f"{name} (no-alloc vs workspace)", np64(g), np64(r), TOL["bf16"])


def test_noalloc_matches_workspace_call_twice():
    assert torch.cuda.is_available()
    kdn.ensure_built()
    scratch = kdn.kdn_noalloc_scratch_bytes()
    c = synth.CONFIGS["diag_kdn"]
    inp = synth.gen_config("diag_kdn", device="cuda")
    need = kdn.kdn_chunk_prefill_workspace_size(3, 1, c["B"], c["T"], c["H"], c["dk"],
                                                c["dv"], 0)
    log(f"call 1: diag_kdn B{c['B']} H{c['H']} T{c['T']}, workspace {need} B "
        f"> scratch {scratch} B (segmented)")
    assert need > scratch
    _compare("diag_kdn", inp)
    del inp
    torch.cuda.empty_cache()
    inp = synth.gen_prefill("gated_deltanet", 1, 1000, 4, 128, 128, "bf16", seed=5,
                            device="cuda", random_state=True)
    log("call 2: gated_deltanet B1 H4 T1000 (fits the scratch)")
    _compare("gated_deltanet", inp)
