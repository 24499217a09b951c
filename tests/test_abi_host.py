"""Host-side checks of the C ABI (no GPU needed).

The library must load and export every symbol include/kdn.h declares, and
argument validation must reject bad calls with the documented status codes
before any HIP call.  Pointers here are fake addresses: every call below fails
validation, so nothing touches a device.
"""
import ctypes
import os
import re

import pytest

from linear_attention_recurrent_delta_amd import kdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kdn.h")

OK, ENULL, ESHAPE, EUNSUP, EALIGN, EALIAS, EHIP, EWS, ESCRATCH = range(9)
A = 1 << 32          # fake, 16-byte aligned device addresses spaced far apart
MB = 1 << 26


@pytest.fixture(scope="module")
def lib():
    return kdn.ensure_built()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kdn_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kdn_chunk_prefill", "kdn_recurrent_decode", "kdn_status_string",
              "kdn_recurrent_decode_multi", "kdn_chunk_prefill_backward",
              "kdn_chunk_prefill_backward_workspace_size",
              "kdn_chunk_prefill_chunk_size", "kdn_abi_version",
              "kdn_chunk_prefill_workspace_size", "kdn_chunk_prefill_noalloc",
              "kdn_noalloc_scratch_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_abi_version(lib):
    assert lib.kdn_abi_version() == 5


def test_status_strings(lib):
    seen = set()
    for s in range(9):
        msg = lib.kdn_status_string(s).decode()
        assert msg and msg not in seen
        seen.add(msg)
    assert lib.kdn_status_string(99).decode() == "unknown status"


def test_chunk_size_query(lib):
    f = lib.kdn_chunk_prefill_chunk_size
    assert f(1, 128, 128, 0) == 64
    assert f(0, 64, 64, 0) == 64
    assert f(0, 128, 128, 0) == 32
    assert f(0, 128, 128, 64) == -1
    assert f(1, 128, 64, 32) == 32
    assert f(1, 96, 128, 0) == -1
    assert f(1, 128, 128, 48) == -1
    assert f(2, 128, 128, 0) == -1


def _prefill_args(variant=1, dtype=1, B=2, T=100, H=4, dk=128, dv=128, chunk=0,
                  **over):
    kdn_ = variant in (3, 4)
    a = dict(q=A, k=A + MB, v=A + 2 * MB,
             alpha=None if variant == 0 else A + 3 * MB,
             beta=None if kdn_ else A + 4 * MB,
             xi=A + 5 * MB if kdn_ else None, r=A + 6 * MB if kdn_ else None,
             S0=A + 7 * MB, p0=A + 8 * MB if kdn_ else None, o=A + 9 * MB,
             S_out=A + 10 * MB, p_out=A + 11 * MB if kdn_ else None,
             ws=None, ws_bytes=0)
    a.update(over)
    return (variant, dtype, B, T, H, dk, dv, chunk, 1.0, a["q"], a["k"], a["v"],
            a["alpha"], a["beta"], a["xi"], a["r"], a["S0"], a["p0"], a["o"],
            a["S_out"], a["p_out"], a["ws"], a["ws_bytes"], None)


def _ws_size(lib, variant=1, dtype=1, B=2, T=100, H=4, dk=128, dv=128, chunk=0):
    st = ctypes.c_int(-1)
    n = lib.kdn_chunk_prefill_workspace_size(variant, dtype, B, T, H, dk, dv, chunk,
                                             ctypes.byref(st))
    return n, st.value


def test_workspace_size_query(lib):
    # bf16, d_k = 128, C = 64: K~, Q~, W~^T (3 x 16 KiB), A_qk and T (2 x 8 KiB)
    # and gamma_C (512 B) per (sequence, head, chunk) record
    rec = 3 * 64 * 128 * 2 + 2 * 64 * 64 * 2 + 128 * 4
    assert rec == 66048
    assert _ws_size(lib) == (2 * 4 * 2 * rec, OK)                # T = 100: 2 chunks
    # variance chunk maps, chunk-start variances, and the maps from each chunk
    # start to its token segments 1..3 (four segments of 16 tokens at d_k = 128)
    kdn_extra = 128 * 4 * 4 + 128 * 4 + 3 * 128 * 4 * 4
    assert kdn_extra == 8704
    assert _ws_size(lib, variant=3) == (2 * 4 * 2 * (rec + kdn_extra), OK)
    iso_extra = 4 * 4 + 64 * 4 * 4 + 4                           # map, token sums, p0
    assert iso_extra == 1044
    assert _ws_size(lib, variant=4) == (2 * 4 * 2 * (rec + iso_extra), OK)
    # float32, d_k = 128: default chunk 32, record rounded up to 256 bytes
    rec32 = 3 * 32 * 128 * 4 + 2 * 32 * 32 * 4 + 128 * 4
    assert _ws_size(lib, dtype=0) == (2 * 4 * 4 * ((rec32 + 255) // 256 * 256), OK)
    assert _ws_size(lib, T=0) == (0, OK)
    assert _ws_size(lib, B=0) == (0, OK)
    assert _ws_size(lib, dk=96) == (0, EUNSUP)
    assert _ws_size(lib, T=-1) == (0, ESHAPE)
    assert _ws_size(lib, chunk=48) == (0, EUNSUP)
    assert lib.kdn_chunk_prefill_workspace_size(1, 1, 1, 64, 1, 64, 64, 0, None) > 0


def _ws_ok(lib, **kw):
    n, st = _ws_size(lib, **kw)
    assert st == OK and n > 0
    return n


def test_workspace_validation(lib):
    n = _ws_ok(lib)
    W = A + 12 * MB
    call = lambda **o: lib.kdn_chunk_prefill(*_prefill_args(**o))
    assert call(ws=W, ws_bytes=n - 1) == EWS
    assert call(ws=W, ws_bytes=0) == EWS
    assert call(ws=W + 16, ws_bytes=n) == EALIGN
    assert call(ws=A + 9 * MB, ws_bytes=n) == EALIAS           # overlaps o
    assert call(ws=A + 10 * MB - 256, ws_bytes=n) == EALIAS    # runs into S_out
    assert call(ws=A + 2 * MB, ws_bytes=n) == EALIAS           # overlaps v
    nk = _ws_ok(lib, variant=3)
    assert lib.kdn_chunk_prefill(*_prefill_args(variant=3, ws=W, ws_bytes=nk - 1)) == EWS
    # p_out == p0 (in-place variance) passes the alias checks with a workspace:
    # the call then fails only on the workspace size, which is checked after
    for v in (3, 4):
        nv = _ws_ok(lib, variant=v)
        assert lib.kdn_chunk_prefill(*_prefill_args(variant=v, p_out=A + 8 * MB, ws=W,
                                                    ws_bytes=nv - 1)) == EWS
        # a partial overlap is still refused
        assert lib.kdn_chunk_prefill(*_prefill_args(variant=v, p_out=A + 8 * MB + 16, ws=W,
                                                    ws_bytes=nv)) == EALIAS
    # validation of the other arguments still comes first
    assert call(q=None, ws=W, ws_bytes=0) == ENULL


def _decode_args(variant=3, dtype=1, N=8, H=4, dk=128, dv=128, **over):
    kdn_ = variant in (3, 4)
    a = dict(q=A, k=A + MB, v=A + 2 * MB,
             alpha=None if variant == 0 else A + 3 * MB,
             beta=None if kdn_ else A + 4 * MB,
             xi=A + 5 * MB if kdn_ else None, r=A + 6 * MB if kdn_ else None,
             S=A + 7 * MB, p=A + 8 * MB if kdn_ else None, o=A + 9 * MB)
    a.update(over)
    return (variant, dtype, N, H, dk, dv, 1.0, a["q"], a["k"], a["v"], a["alpha"],
            a["beta"], a["xi"], a["r"], a["S"], a["p"], a["o"], None)


PREFILL_CASES = [
    ("bad variant", dict(variant=7), EUNSUP),
    ("bad dtype", dict(dtype=5), EUNSUP),
    ("negative B", dict(B=-1), ESHAPE),
    ("negative T", dict(T=-3), ESHAPE),
    ("negative H", dict(H=-2), ESHAPE),
    ("zero d_k", dict(dk=0), ESHAPE),
    ("d_k 96", dict(dk=96), EUNSUP),
    ("d_v 256", dict(dv=256), EUNSUP),
    ("chunk 48", dict(chunk=48), EUNSUP),
    ("f32 d128 chunk 64", dict(dtype=0, chunk=64), EUNSUP),
    ("state too large", dict(B=1 << 14, H=1 << 4), ESHAPE),
    ("q NULL", dict(q=None), ENULL),
    ("o NULL", dict(o=None), ENULL),
    ("S_out NULL", dict(S_out=None), ENULL),
    ("GDN without alpha", dict(alpha=None), ENULL),
    ("GDN without beta", dict(beta=None), ENULL),
    ("DeltaNet with alpha", dict(variant=0, alpha=A + 3 * MB), ENULL),
    ("GDN with proc noise", dict(xi=A + 5 * MB), ENULL),
    ("GDN with p0", dict(p0=A + 8 * MB), ENULL),
    ("KDN with beta", dict(variant=3, beta=A + 4 * MB), ENULL),
    ("KDN without obs noise", dict(variant=3, r=None), ENULL),
    ("KDN without p0", dict(variant=3, p0=None), ENULL),
    ("KDN without p_out", dict(variant=3, p_out=None), ENULL),
    ("misaligned q", dict(q=A + 8), EALIGN),
    ("misaligned S0", dict(S0=A + 7 * MB + 4), EALIGN),
    ("misaligned KDA alpha", dict(variant=2, alpha=A + 3 * MB + 2), EALIGN),
    ("odd scalar beta", dict(beta=A + 4 * MB + 1), EALIGN),
    ("o overlaps v", dict(o=A + 2 * MB + 4096), EALIAS),
    ("S_out overlaps q", dict(S_out=A + 64), EALIAS),
    ("S_out partially overlaps S0", dict(S_out=A + 7 * MB + 1024), EALIAS),
    ("o overlaps S_out", dict(o=A + 10 * MB + 16), EALIAS),
    ("KDN p_out equals p0 without workspace", dict(variant=3, p_out=A + 8 * MB), EALIAS),
    ("iso KDN p_out equals p0 without workspace", dict(variant=4, p_out=A + 8 * MB), EALIAS),
    ("iso KDN with beta", dict(variant=4, beta=A + 4 * MB), ENULL),
    ("iso KDN without proc noise", dict(variant=4, xi=None), ENULL),
    ("iso KDN without p0", dict(variant=4, p0=None), ENULL),
    ("iso KDN odd p0", dict(variant=4, p0=A + 8 * MB + 2), EALIGN),
    # p is [B, H] for isotropic KDN: 4-byte alignment suffices, and 4 bytes
    # past p0 still overlaps it ([B, H, d_k] needs 16 bytes: misaligned)
    ("iso KDN p_out 4 B past p0", dict(variant=4, p_out=A + 8 * MB + 4), EALIAS),
    ("diag KDN p_out 4 B past p0", dict(variant=3, p_out=A + 8 * MB + 4), EALIGN),
    ("iso KDN p_out overlaps S_out", dict(variant=4, p_out=A + 10 * MB + 12), EALIAS),
]


@pytest.mark.parametrize("name,over,status", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_validation(lib, name, over, status):
    assert lib.kdn_chunk_prefill(*_prefill_args(**over)) == status


DECODE_CASES = [
    ("bad variant", dict(variant=-1), EUNSUP),
    ("negative N", dict(N=-1), ESHAPE),
    ("d_k 32", dict(dk=32), EUNSUP),
    ("S NULL", dict(S=None), ENULL),
    ("KDN without p", dict(p=None), ENULL),
    ("GDN with p", dict(variant=1, p=A + 8 * MB), ENULL),
    ("KDN with beta", dict(beta=A + 4 * MB), ENULL),
    ("misaligned o", dict(o=A + 9 * MB + 2), EALIGN),
    ("misaligned S", dict(S=A + 7 * MB + 8), EALIGN),
    ("odd scalar r", dict(r=A + 6 * MB + 1), EALIGN),
    ("o overlaps S", dict(o=A + 7 * MB + 512), EALIAS),
    ("S overlaps k", dict(S=A + MB), EALIAS),
    ("p overlaps S", dict(p=A + 7 * MB + 256), EALIAS),
    ("iso KDN with beta", dict(variant=4, beta=A + 4 * MB), ENULL),
    ("iso KDN without p", dict(variant=4, p=None), ENULL),
    ("iso KDN odd p", dict(variant=4, p=A + 8 * MB + 1), EALIGN),
    ("iso KDN p overlaps o", dict(variant=4, p=A + 9 * MB + 4), EALIAS),
]


@pytest.mark.parametrize("name,over,status", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_validation(lib, name, over, status):
    assert lib.kdn_recurrent_decode(*_decode_args(**over)) == status


def _multi_args(variant=3, dtype=1, N=8, T=4, H=4, dk=128, dv=128, **over):
    kdn_ = variant in (3, 4)
    a = dict(q=A, k=A + MB, v=A + 2 * MB,
             alpha=None if variant == 0 else A + 3 * MB,
             beta=None if kdn_ else A + 4 * MB,
             xi=A + 5 * MB if kdn_ else None, r=A + 6 * MB if kdn_ else None,
             S0=A + 7 * MB, p0=A + 8 * MB if kdn_ else None, o=A + 9 * MB,
             S_out=A + 10 * MB, p_out=A + 11 * MB if kdn_ else None)
    a.update(over)
    return (variant, dtype, N, T, H, dk, dv, 1.0, a["q"], a["k"], a["v"], a["alpha"],
            a["beta"], a["xi"], a["r"], a["S0"], a["p0"], a["o"], a["S_out"],
            a["p_out"], None)


MULTI_CASES = [
    ("bad variant", dict(variant=9), EUNSUP),
    ("bad dtype", dict(dtype=3), EUNSUP),
    ("negative T", dict(T=-1), ESHAPE),
    ("negative N", dict(N=-2), ESHAPE),
    ("d_v 96", dict(dv=96), EUNSUP),
    ("state too large", dict(N=1 << 14, H=1 << 4), ESHAPE),
    ("q NULL", dict(q=None), ENULL),
    ("S_out NULL", dict(S_out=None), ENULL),
    ("KDN without p0", dict(p0=None), ENULL),
    ("KDN without p_out", dict(p_out=None), ENULL),
    ("GDN with p0", dict(variant=1, p0=A + 8 * MB, p_out=None), ENULL),
    ("KDN with beta", dict(beta=A + 4 * MB), ENULL),
    ("misaligned k", dict(k=A + MB + 4), EALIGN),
    ("misaligned S_out", dict(S_out=A + 10 * MB + 8), EALIGN),
    ("odd scalar r", dict(r=A + 6 * MB + 1), EALIGN),
    ("o overlaps q", dict(o=A + 32), EALIAS),
    ("S_out partially overlaps S0", dict(S_out=A + 7 * MB + 1024), EALIAS),
    ("S_out overlaps v", dict(S_out=A + 2 * MB), EALIAS),
    ("p_out partially overlaps p0", dict(p_out=A + 8 * MB + 16), EALIAS),
    ("p_out overlaps S0", dict(p_out=A + 7 * MB + 64), EALIAS),
    ("o overlaps p_out", dict(o=A + 11 * MB), EALIAS),
    ("iso KDN without r", dict(variant=4, r=None), ENULL),
    ("iso KDN odd p_out", dict(variant=4, p_out=A + 11 * MB + 2), EALIGN),
    ("iso KDN p_out partially overlaps p0", dict(variant=4, p_out=A + 8 * MB + 4), EALIAS),
]


@pytest.mark.parametrize("name,over,status", MULTI_CASES, ids=[c[0] for c in MULTI_CASES])
def test_decode_multi_validation(lib, name, over, status):
    assert lib.kdn_recurrent_decode_multi(*_multi_args(**over)) == status


def test_decode_multi_accepts_in_place_and_empty(lib):
    # in place (S_out == S0, p_out == p0) and empty sizes pass validation; with
    # N = 0 or H = 0 nothing is launched, so the fake pointers are never used
    assert lib.kdn_recurrent_decode_multi(
        *_multi_args(N=0, S_out=A + 7 * MB, p_out=A + 8 * MB)) == OK
    assert lib.kdn_recurrent_decode_multi(*_multi_args(H=0, T=0)) == OK
    assert lib.kdn_recurrent_decode_multi(
        *_multi_args(N=0, q=None, k=None, v=None, o=None, S0=None)) == OK


def _bwd_args(variant=1, dtype=1, B=2, T=100, H=4, dk=128, dv=128, chunk=0, **over):
    iso = variant == 4
    a = dict(q=A, k=A + MB, v=A + 2 * MB, alpha=None if variant == 0 else A + 3 * MB,
             beta=None if iso else A + 4 * MB, xi=A + 14 * MB if iso else None,
             r=A + 15 * MB if iso else None, S0=A + 5 * MB,
             p0=A + 17 * MB if iso else None, do=A + 6 * MB, dS=A + 7 * MB,
             dp=A + 18 * MB if iso else None,
             gq=A + 8 * MB, gk=A + 9 * MB, gv=A + 10 * MB,
             da=None if variant == 0 else A + 11 * MB, db=None if iso else A + 12 * MB,
             dxi=A + 19 * MB if iso else None, dr=A + 20 * MB if iso else None,
             dS0=A + 13 * MB, dp0=A + 21 * MB if iso else None,
             ws=A + 32 * MB, ws_bytes=1 << 40)
    a.update(over)
    return (variant, dtype, B, T, H, dk, dv, chunk, 1.0, a["q"], a["k"], a["v"], a["alpha"],
            a["beta"], a["xi"], a["r"], a["S0"], a["p0"], a["do"], a["dS"], a["dp"],
            a["gq"], a["gk"], a["gv"], a["da"], a["db"], a["dxi"], a["dr"], a["dS0"],
            a["dp0"], a["ws"], a["ws_bytes"], None)


BWD_CASES = [
    ("diag KDN with beta", dict(variant=3, xi=A + 14 * MB, r=A + 15 * MB,
                                p0=A + 17 * MB, da=A + 11 * MB), ENULL),
    ("diag KDN misaligned p0", dict(variant=3, beta=None, xi=A + 14 * MB, r=A + 15 * MB,
                                    p0=A + 17 * MB + 4, db=None, dxi=A + 19 * MB,
                                    dr=A + 20 * MB), EALIGN),
    ("iso KDN with beta", dict(variant=4, beta=A + 4 * MB), ENULL),
    ("iso KDN with dbeta", dict(variant=4, db=A + 12 * MB), ENULL),
    ("iso KDN without p0", dict(variant=4, p0=None), ENULL),
    ("iso KDN without dproc_noise", dict(variant=4, dxi=None), ENULL),
    ("iso KDN odd dp0", dict(variant=4, dp0=A + 21 * MB + 2), EALIGN),
    ("iso KDN dobs_noise overlaps dbeta area", dict(variant=4, dr=A + 8 * MB), EALIAS),
    ("GDN with p0", dict(p0=A + 17 * MB), ENULL),
    ("GDN with dp0", dict(dp0=A + 21 * MB), ENULL),
    ("bad dtype", dict(dtype=2), EUNSUP),
    ("negative T", dict(T=-1), ESHAPE),
    ("d_k 32", dict(dk=32), EUNSUP),
    ("d_o NULL", dict(do=None), ENULL),
    ("dq NULL", dict(gq=None), ENULL),
    ("dbeta NULL", dict(db=None), ENULL),
    ("GDN without dlog_alpha", dict(da=None), ENULL),
    ("DeltaNet with dlog_alpha", dict(variant=0, da=A + 11 * MB), ENULL),
    ("GDN without beta", dict(beta=None), ENULL),
    ("misaligned dk", dict(gk=A + 9 * MB + 8), EALIGN),
    ("misaligned dS_out", dict(dS=A + 7 * MB + 4), EALIGN),
    ("odd dbeta", dict(db=A + 12 * MB + 2), EALIGN),
    ("KDA misaligned dlog_alpha", dict(variant=2, da=A + 11 * MB + 4), EALIGN),
    ("no workspace", dict(ws=None, ws_bytes=0), EWS),
    ("small workspace", dict(ws_bytes=1000), EWS),
    ("misaligned workspace", dict(ws=A + 16 * MB + 64), EALIGN),
    ("dq overlaps q", dict(gq=A + 1024), EALIAS),
    ("dk overlaps dq", dict(gk=A + 8 * MB + 4096), EALIAS),
    ("dS0 overlaps dS_out", dict(dS0=A + 7 * MB), EALIAS),
    ("workspace overlaps dv", dict(ws=A + 10 * MB), EALIAS),
]


@pytest.mark.parametrize("name,over,status", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_validation(lib, name, over, status):
    assert lib.kdn_chunk_prefill_backward(*_bwd_args(**over)) == status


def test_backward_workspace_size(lib):
    st = ctypes.c_int(-1)
    f = lib.kdn_chunk_prefill_backward_workspace_size
    rec = 66048
    n = f(1, 1, 2, 100, 4, 128, 128, 0, ctypes.byref(st))
    assert st.value == OK and n == 2 * 4 * 2 * (rec + 2 * 128 * 128 * 2)
    n_diag = f(3, 1, 2, 100, 4, 128, 128, 0, ctypes.byref(st))
    assert st.value == OK and n_diag > n
    n_iso = f(4, 1, 2, 100, 4, 128, 128, 0, ctypes.byref(st))
    assert st.value == OK and n_iso > n
    assert f(1, 1, 2, 0, 4, 128, 128, 0, ctypes.byref(st)) == 0 and st.value == OK
    # no tokens: nothing to launch for B*H = 0, and no workspace is needed
    assert lib.kdn_chunk_prefill_backward(*_bwd_args(B=0, ws=None, ws_bytes=0)) == OK


def test_binding_raises_with_status(lib):
    with pytest.raises(kdn.KdnError) as e:
        kdn.kdn_chunk_prefill(*_prefill_args(q=None)[:-1], stream=0)
    assert e.value.status == ENULL
    with pytest.raises(kdn.KdnError) as e:
        kdn.kdn_chunk_prefill_workspace_size(1, 1, 2, 100, 4, 96, 128, 0)
    assert e.value.status == EUNSUP


def test_binding_missing_library_raises(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        kdn.load(str(tmp_path / "libkdn.so"))


def test_noalloc_validation(lib):
    """kdn_chunk_prefill_noalloc checks every argument of the full call, and
    the static scratch's limit, before any HIP call."""
    f = lib.kdn_chunk_prefill_noalloc
    assert lib.kdn_noalloc_scratch_bytes() == 64 << 20

    def call(**over):
        a = list(_prefill_args(**over))
        return f(*(a[:21] + [None]))          # no workspace arguments
    for name, over, status in PREFILL_CASES:
        if "without workspace" in name:
            continue                          # in-place p is allowed here
        assert call(**over) == status, name
    # one chunk of all heads of a sequence exceeds the 64 MiB scratch
    # (d = 64: 41,216 bytes per head and chunk; the fake tensors stay apart)
    big = dict(B=1, T=10, H=1700, dk=64, dv=64)
    assert call(**big) == ESCRATCH
    assert call(variant=3, **big) == ESCRATCH
    assert call(q=None, **big) == ENULL         # argument errors come first
