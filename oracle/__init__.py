"""fp64 CPU oracle of the gated delta-rule / Kalman (diagonal and isotropic) recurrence.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The HIP library and its
Python binding never import this package, and this package never imports them.

The arithmetic lives in ``kdn_oracle.c`` (plain C, double precision, the
token-by-token recurrence in the order the pages give it).  This module only
builds that file with gcc, loads it with ctypes and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kdn_oracle.c")
_LIB = os.path.join(_HERE, "libkdn_oracle.so")

VARIANTS = {"deltanet": 0, "gated_deltanet": 1, "kda": 2, "diag_kdn": 3, "iso_kdn": 4}

_default = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile an oracle C source into a shared library (gcc, -O3, no fast-math)."""
    global _default
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-std=c11", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", "-o", tmp, src]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    if out == _LIB:
        _default = None
    return out


class OracleLib:
    """ctypes handle on one build of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.c_void_p
        lib.kdn_oracle_recurrence.restype = ctypes.c_int
        lib.kdn_oracle_recurrence.argtypes = (
            [ctypes.c_int] + [ctypes.c_long] * 5 + [ctypes.c_double]
            + [dp] * 12 + [ctypes.c_int])
        lib.kdn_oracle_backward.restype = ctypes.c_int
        lib.kdn_oracle_backward.argtypes = (
            [ctypes.c_int] + [ctypes.c_long] * 5 + [dp] * 14 + [ctypes.c_int])
        lib.kdn_oracle_backward_iso.restype = ctypes.c_int
        lib.kdn_oracle_backward_iso.argtypes = (
            [ctypes.c_long] * 5 + [ctypes.c_double] + [dp] * 19 + [ctypes.c_int])
        lib.kdn_oracle_backward_diag.restype = ctypes.c_int
        lib.kdn_oracle_backward_diag.argtypes = (
            [ctypes.c_long] * 5 + [ctypes.c_double] + [dp] * 19)
        lib.kdn_oracle_max_threads.restype = ctypes.c_int
        lib.kdn_oracle_max_threads.argtypes = []
        self.lib = lib
        self.path = path

    def max_threads(self) -> int:
        return int(self.lib.kdn_oracle_max_threads())

    def recurrence(self, variant, q, k, v, alpha=None, beta=None, xi=None,
                   r=None, S0=None, p0=None, mu=1.0, nthreads=0):
        return _run(self.lib, variant, q, k, v, alpha, beta, xi, r, S0, p0, mu,
                    nthreads)


    def backward(self, variant, q, k, v, alpha=None, beta=None, S0=None, dO=None,
                 dS_T=None, nthreads=0):
        return _run_backward(self.lib, variant, q, k, v, alpha, beta, S0, dO, dS_T,
                             nthreads)

    def backward_diag(self, q, k, v, alpha, xi, r, p0, S0=None, dO=None, dS_T=None,
                      dp_T=None, mu=1.0):
        return _run_backward_kdn(self.lib, 3, q, k, v, alpha, xi, r, p0, S0, dO, dS_T, dp_T,
                                 mu, 0)

    def backward_iso(self, q, k, v, alpha, xi, r, p0, S0=None, dO=None, dS_T=None,
                     dp_T=None, mu=1.0, nthreads=0):
        return _run_backward_kdn(self.lib, 4, q, k, v, alpha, xi, r, p0, S0, dO, dS_T, dp_T,
                                 mu, nthreads)


def load() -> OracleLib:
    """The oracle built from kdn_oracle.c (built on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build()
        _default = OracleLib(_LIB)
    return _default


def max_threads() -> int:
    return load().max_threads()


def _f64(x, shape, name):
    if x is None:
        return None
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if tuple(a.shape) != tuple(shape):
        raise ValueError(f"oracle: {name} has shape {a.shape}, expected {shape}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def recurrence(variant, q, k, v, alpha=None, beta=None, xi=None, r=None,
               S0=None, p0=None, mu=1.0, nthreads=0):
    """Run the recurrence over [B, T, H, d] inputs.

    Returns ``(o, S, p)``: o [B,T,H,dv], final S [B,H,dk,dv], final p [B,H,dk]
    for diagonal KDN, [B,H] for isotropic KDN, else None.  Every input is converted
    to float64 first; values that were rounded to a device dtype upstream keep
    exactly that rounding.
    """
    return load().recurrence(variant, q, k, v, alpha, beta, xi, r, S0, p0, mu,
                             nthreads)


def _run(lib, variant, q, k, v, alpha, beta, xi, r, S0, p0, mu, nthreads):
    vid = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    q = np.asarray(q)
    B, T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    q = _f64(q, (B, T, H, dk), "q")
    k = _f64(k, (B, T, H, dk), "k")
    v = _f64(v, (B, T, H, dv), "v")
    if vid == 1:
        alpha = _f64(alpha, (B, T, H), "alpha")
    elif vid in (2, 3, 4):
        alpha = _f64(alpha, (B, T, H, dk), "alpha")
    else:
        alpha = None
    kdn = vid in (3, 4)
    pshape = (B, H, dk) if vid == 3 else (B, H)
    beta = _f64(beta, (B, T, H), "beta") if not kdn else None
    if kdn:
        xi = _f64(xi, (B, T, H, dk), "xi")
        r = _f64(r, (B, T, H), "r")
        p0 = _f64(p0, pshape, "p0")
    else:
        xi = r = p0 = None
    S0 = _f64(S0, (B, H, dk, dv), "S0") if S0 is not None else None

    o = np.zeros((B, T, H, dv), dtype=np.float64)
    S = np.zeros((B, H, dk, dv), dtype=np.float64)
    p = np.zeros(pshape, dtype=np.float64) if kdn else None
    rc = lib.kdn_oracle_recurrence(
        vid, B, T, H, dk, dv, float(mu), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
        _ptr(beta), _ptr(xi), _ptr(r), _ptr(S0), _ptr(p0), _ptr(o), _ptr(S),
        _ptr(p), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"kdn_oracle_recurrence failed with code {rc}")
    return o, S, p


def backward(variant, q, k, v, alpha=None, beta=None, S0=None, dO=None, dS_T=None,
             nthreads=0):
    """Gradients of a scalar loss through the recurrence (DeltaNet, Gated
    DeltaNet, KDA), given dO = dL/do [B,T,H,dv] and dS_T = dL/dS_final
    [B,H,dk,dv] (None: zero).

    Returns ``(dq, dk, dv, dalpha, dbeta, dS0)``; dalpha is dL/dalpha
    ([B,T,H] for Gated DeltaNet, [B,T,H,dk] for KDA, None for DeltaNet).
    """
    return load().backward(variant, q, k, v, alpha, beta, S0, dO, dS_T, nthreads)


def _run_backward(lib, variant, q, k, v, alpha, beta, S0, dO, dS_T, nthreads):
    vid = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    if vid not in (0, 1, 2):
        raise ValueError("oracle backward: write-strength variants only")
    q = np.asarray(q)
    B, T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    q = _f64(q, (B, T, H, dk), "q")
    k = _f64(k, (B, T, H, dk), "k")
    v = _f64(v, (B, T, H, dv), "v")
    ashape = (B, T, H) if vid == 1 else (B, T, H, dk)
    alpha = _f64(alpha, ashape, "alpha") if vid != 0 else None
    beta = _f64(beta, (B, T, H), "beta")
    S0 = _f64(S0, (B, H, dk, dv), "S0") if S0 is not None else None
    dO = _f64(dO, (B, T, H, dv), "dO")
    dS_T = _f64(dS_T, (B, H, dk, dv), "dS_T") if dS_T is not None else None
    dq = np.zeros((B, T, H, dk))
    dk_ = np.zeros((B, T, H, dk))
    dv_ = np.zeros((B, T, H, dv))
    da = np.zeros(ashape) if vid != 0 else None
    db = np.zeros((B, T, H))
    dS0 = np.zeros((B, H, dk, dv))
    rc = lib.kdn_oracle_backward(
        vid, B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _ptr(S0), _ptr(dO), _ptr(dS_T), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(da),
        _ptr(db), _ptr(dS0), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"kdn_oracle_backward failed with code {rc}")
    return dq, dk_, dv_, da, db, dS0


def backward_iso(q, k, v, alpha, xi, r, p0, S0=None, dO=None, dS_T=None, dp_T=None,
                 mu=1.0, nthreads=0):
    """Gradients through isotropic KDN, given dO [B,T,H,dv], dS_T [B,H,dk,dv]
    and dp_T [B,H] (None: zero).  Returns ``(dq, dk, dv, dalpha, dxi, dr, dS0,
    dp0)`` with dalpha = dL/dalpha [B,T,H,dk]."""
    return load().backward_iso(q, k, v, alpha, xi, r, p0, S0, dO, dS_T, dp_T, mu, nthreads)


def backward_diag(q, k, v, alpha, xi, r, p0, S0=None, dO=None, dS_T=None, dp_T=None,
                  mu=1.0):
    """Gradients through diagonal KDN, given dO [B,T,H,dv], dS_T [B,H,dk,dv]
    and dp_T [B,H,dk] (None: zero).  Returns ``(dq, dk, dv, dalpha, dxi, dr,
    dS0, dp0)`` with dalpha = dL/dalpha [B,T,H,dk] and dp0 [B,H,dk]."""
    return load().backward_diag(q, k, v, alpha, xi, r, p0, S0, dO, dS_T, dp_T, mu)


def _run_backward_kdn(lib, vid, q, k, v, alpha, xi, r, p0, S0, dO, dS_T, dp_T, mu, nthreads):
    q = np.asarray(q)
    B, T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    q = _f64(q, (B, T, H, dk), "q")
    k = _f64(k, (B, T, H, dk), "k")
    v = _f64(v, (B, T, H, dv), "v")
    alpha = _f64(alpha, (B, T, H, dk), "alpha")
    xi = _f64(xi, (B, T, H, dk), "xi")
    r = _f64(r, (B, T, H), "r")
    pshape = (B, H) if vid == 4 else (B, H, dk)
    p0 = _f64(p0, pshape, "p0")
    S0 = _f64(S0, (B, H, dk, dv), "S0") if S0 is not None else None
    dO = _f64(dO, (B, T, H, dv), "dO")
    dS_T = _f64(dS_T, (B, H, dk, dv), "dS_T") if dS_T is not None else None
    dp_T = _f64(dp_T, pshape, "dp_T") if dp_T is not None else None
    out = dict(dq=np.zeros((B, T, H, dk)), dk=np.zeros((B, T, H, dk)),
               dv=np.zeros((B, T, H, dv)), da=np.zeros((B, T, H, dk)),
               dxi=np.zeros((B, T, H, dk)), dr=np.zeros((B, T, H)),
               dS0=np.zeros((B, H, dk, dv)), dp0=np.zeros(pshape))
    args = (B, T, H, dk, dv, float(mu), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(xi),
            _ptr(r), _ptr(S0), _ptr(p0), _ptr(dO), _ptr(dS_T), _ptr(dp_T), _ptr(out["dq"]),
            _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["da"]), _ptr(out["dxi"]),
            _ptr(out["dr"]), _ptr(out["dS0"]), _ptr(out["dp0"]))
    if vid == 4:
        rc = lib.kdn_oracle_backward_iso(*args, int(nthreads))
    else:
        rc = lib.kdn_oracle_backward_diag(*args)
    if rc != 0:
        raise RuntimeError(f"kdn_oracle backward (variant {vid}) failed with code {rc}")
    return (out["dq"], out["dk"], out["dv"], out["da"], out["dxi"], out["dr"], out["dS0"],
            out["dp0"])
