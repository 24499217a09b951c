"""ctypes binding of libkdn.so (the C ABI declared in include/kdn.h).

Argument marshalling only: tensors become device pointers, the current HIP
stream is passed through, and a non-OK status raises.  Every step of the
recurrence runs in the library's gfx950 kernels; PyTorch provides device
memory and streams.  If the library is not built this module raises -- there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkdn.so")

# kdn_variant / kdn_dtype / kdn_status values of include/kdn.h
VARIANTS = {"deltanet": 0, "gated_deltanet": 1, "kda": 2, "diag_kdn": 3, "iso_kdn": 4}


def _p_shape(vid, N, H, dk):
    """Shape of the variance tensor p: [N,H,dk] (diagonal KDN), [N,H]
    (isotropic KDN), or None (no variance)."""
    return (N, H, dk) if vid == 3 else ((N, H) if vid == 4 else None)


def _new_p(vid, N, H, dk, device):
    shp = _p_shape(vid, N, H, dk)
    return None if shp is None else torch.empty(shp, dtype=torch.float32, device=device)
DTYPES = {torch.float32: 0, torch.bfloat16: 1}
STATUS = {0: "KDN_OK", 1: "KDN_ERR_NULL", 2: "KDN_ERR_SHAPE",
          3: "KDN_ERR_UNSUPPORTED", 4: "KDN_ERR_ALIGN", 5: "KDN_ERR_ALIAS",
          6: "KDN_ERR_HIP", 7: "KDN_ERR_WORKSPACE", 8: "KDN_ERR_SCRATCH"}

_lib = None


class KdnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load libkdn.so and declare its signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run `python -m linear_attention_recurrent_delta_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.kdn_chunk_prefill.restype = i
    u64 = ctypes.c_ulonglong
    lib.kdn_chunk_prefill.argtypes = [i, i, i, i, i, i, i, i, f] + [vp] * 12 + [vp, u64, vp]
    lib.kdn_chunk_prefill_noalloc.restype = i
    lib.kdn_chunk_prefill_noalloc.argtypes = [i, i, i, i, i, i, i, i, f] + [vp] * 12 + [vp]
    lib.kdn_noalloc_scratch_bytes.restype = u64
    lib.kdn_noalloc_scratch_bytes.argtypes = []
    lib.kdn_chunk_prefill_workspace_size.restype = u64
    lib.kdn_chunk_prefill_workspace_size.argtypes = [i] * 8 + [ctypes.POINTER(i)]
    lib.kdn_recurrent_decode.restype = i
    lib.kdn_recurrent_decode.argtypes = [i, i, i, i, i, i, f] + [vp] * 11
    lib.kdn_recurrent_decode_multi.restype = i
    lib.kdn_recurrent_decode_multi.argtypes = [i, i, i, i, i, i, i, f] + [vp] * 13
    lib.kdn_chunk_prefill_backward.restype = i
    lib.kdn_chunk_prefill_backward.argtypes = [i] * 8 + [f] + [vp] * 21 + [vp, u64, vp]
    lib.kdn_chunk_prefill_backward_workspace_size.restype = u64
    lib.kdn_chunk_prefill_backward_workspace_size.argtypes = [i] * 8 + [ctypes.POINTER(i)]
    lib.kdn_status_string.restype = ctypes.c_char_p
    lib.kdn_status_string.argtypes = [i]
    lib.kdn_chunk_prefill_chunk_size.restype = i
    lib.kdn_chunk_prefill_chunk_size.argtypes = [i, i, i, i]
    lib.kdn_abi_version.restype = i
    lib.kdn_abi_version.argtypes = []
    if path == LIB_PATH:
        _lib = lib
    return lib


def ensure_built():
    """Build the library if no build is present, then load it."""
    if not os.path.exists(LIB_PATH):
        from . import build
        build.build()
    return load()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError("kdn: tensor arguments must be contiguous")
    if x.device.type != "cuda":
        raise ValueError(f"kdn: tensor arguments must be in GPU memory, not on {x.device}")
    return x.data_ptr()


def _expect(args, device):
    """Check (name, tensor or None, shape, dtype) tuples before a call: the
    shape, then the dtype, then contiguity, then that every tensor lives on
    ``device`` (a GPU).  The C library checks sizes and pointers only; a host
    tensor, a tensor on another GPU or a wrongly shaped one would otherwise
    reach the kernels."""
    for name, x, shape, dtype in args:
        if x is None:
            continue
        if not isinstance(x, torch.Tensor):
            raise TypeError(f"kdn: {name} must be a tensor or None")
        if tuple(x.shape) != tuple(shape):
            raise ValueError(f"kdn: {name} has shape {tuple(x.shape)}, expected {tuple(shape)}")
        if x.dtype != dtype:
            raise ValueError(f"kdn: {name} has dtype {x.dtype}, expected {dtype}")
        if not x.is_contiguous():
            raise ValueError(f"kdn: {name} must be contiguous")
    if device.type != "cuda":
        raise ValueError(f"kdn: tensors must be in GPU memory, not on {device}")
    for name, x, _, _ in args:
        if x is not None and x.device != device:
            raise ValueError(f"kdn: {name} is on {x.device}, the other tensors on {device}")


def _gate_specs(vid, lead, dk, dt, alpha, beta, proc_noise, obs_noise):
    """Expected (name, tensor, shape, dtype) of the gates for leading dims
    ``lead`` ([B,T,H] or [N,H])."""
    lead = tuple(lead)
    a_shape = lead if vid == 1 else lead + (dk,)
    return [("alpha", alpha, a_shape, dt), ("beta", beta, lead, dt),
            ("proc_noise", proc_noise, lead + (dk,), dt), ("obs_noise", obs_noise, lead, dt)]


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(lib, st):
    if st != 0:
        raise KdnError(st, lib.kdn_status_string(st).decode())


def kdn_status_string(status: int) -> str:
    return load().kdn_status_string(int(status)).decode()


def kdn_abi_version() -> int:
    return int(load().kdn_abi_version())


def kdn_chunk_prefill_chunk_size(dtype: int, d_k: int, d_v: int, chunk: int) -> int:
    return int(load().kdn_chunk_prefill_chunk_size(int(dtype), d_k, d_v, chunk))


def kdn_chunk_prefill(variant, dtype, B, T, H, d_k, d_v, chunk, mu, q, k, v,
                      alpha, beta, proc_noise, obs_noise, S0, p0, o, S_out,
                      p_out, workspace=None, workspace_bytes=0, stream=None):
    """Raw entry point: same arguments as the C function (tensors or ints
    for pointers, None for NULL).  A tensor workspace passes its byte size
    when ``workspace_bytes`` is 0."""
    lib = load()
    if workspace is not None and not isinstance(workspace, int) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib.kdn_chunk_prefill(
        int(variant), int(dtype), int(B), int(T), int(H), int(d_k), int(d_v),
        int(chunk), float(mu), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
        _ptr(beta), _ptr(proc_noise), _ptr(obs_noise), _ptr(S0), _ptr(p0),
        _ptr(o), _ptr(S_out), _ptr(p_out), _ptr(workspace), int(workspace_bytes),
        _stream(stream))
    _check(lib, st)


def kdn_chunk_prefill_noalloc(variant, dtype, B, T, H, d_k, d_v, chunk, mu, q, k, v,
                              alpha, beta, proc_noise, obs_noise, S0, p0, o, S_out,
                              p_out, stream=None):
    """Raw entry point: same arguments as the C function (the two-pass
    prefill on the library's static scratch; allocates nothing)."""
    lib = load()
    st = lib.kdn_chunk_prefill_noalloc(
        int(variant), int(dtype), int(B), int(T), int(H), int(d_k), int(d_v),
        int(chunk), float(mu), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
        _ptr(beta), _ptr(proc_noise), _ptr(obs_noise), _ptr(S0), _ptr(p0),
        _ptr(o), _ptr(S_out), _ptr(p_out), _stream(stream))
    _check(lib, st)


def kdn_noalloc_scratch_bytes() -> int:
    return int(load().kdn_noalloc_scratch_bytes())


def kdn_chunk_prefill_workspace_size(variant, dtype, B, T, H, d_k, d_v, chunk):
    """Bytes of workspace for the two-pass schedule; raises on invalid sizes."""
    lib = load()
    st = ctypes.c_int(0)
    n = lib.kdn_chunk_prefill_workspace_size(int(variant), int(dtype), int(B), int(T),
                                             int(H), int(d_k), int(d_v), int(chunk),
                                             ctypes.byref(st))
    _check(lib, st.value)
    return int(n)


def kdn_chunk_prefill_backward(variant, dtype, B, T, H, d_k, d_v, chunk, mu, q, k, v,
                               alpha, beta, proc_noise, obs_noise, S0, p0, d_o, dS_out,
                               dp_out, dq, dk, dv, dlog_alpha, dbeta, dproc_noise,
                               dobs_noise, dS0, dp0, workspace=None, workspace_bytes=0,
                               stream=None):
    """Raw entry point: same arguments as the C function."""
    lib = load()
    if workspace is not None and not isinstance(workspace, int) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib.kdn_chunk_prefill_backward(
        int(variant), int(dtype), int(B), int(T), int(H), int(d_k), int(d_v), int(chunk),
        float(mu), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(proc_noise),
        _ptr(obs_noise), _ptr(S0), _ptr(p0), _ptr(d_o), _ptr(dS_out), _ptr(dp_out),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dlog_alpha), _ptr(dbeta), _ptr(dproc_noise),
        _ptr(dobs_noise), _ptr(dS0), _ptr(dp0), _ptr(workspace), int(workspace_bytes),
        _stream(stream))
    _check(lib, st)


def kdn_chunk_prefill_backward_workspace_size(variant, dtype, B, T, H, d_k, d_v, chunk):
    """Bytes of workspace the gradient call needs; raises on invalid sizes."""
    lib = load()
    st = ctypes.c_int(0)
    n = lib.kdn_chunk_prefill_backward_workspace_size(
        int(variant), int(dtype), int(B), int(T), int(H), int(d_k), int(d_v), int(chunk),
        ctypes.byref(st))
    _check(lib, st.value)
    return int(n)


def kdn_recurrent_decode(variant, dtype, N, H, d_k, d_v, mu, q, k, v, alpha,
                         beta, proc_noise, obs_noise, S, p, o, stream=None):
    """Raw entry point: same arguments as the C function."""
    lib = load()
    st = lib.kdn_recurrent_decode(
        int(variant), int(dtype), int(N), int(H), int(d_k), int(d_v),
        float(mu), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _ptr(proc_noise), _ptr(obs_noise), _ptr(S), _ptr(p), _ptr(o),
        _stream(stream))
    _check(lib, st)


def kdn_recurrent_decode_multi(variant, dtype, N, T, H, d_k, d_v, mu, q, k, v,
                               alpha, beta, proc_noise, obs_noise, S0, p0, o,
                               S_out, p_out, stream=None):
    """Raw entry point: same arguments as the C function."""
    lib = load()
    st = lib.kdn_recurrent_decode_multi(
        int(variant), int(dtype), int(N), int(T), int(H), int(d_k), int(d_v),
        float(mu), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _ptr(proc_noise), _ptr(obs_noise), _ptr(S0), _ptr(p0), _ptr(o),
        _ptr(S_out), _ptr(p_out), _stream(stream))
    _check(lib, st)


# ---------------------------------------------------------------------------
# Tensor-shaped conveniences (allocate outputs, infer sizes, then call the
# entry points above).
# ---------------------------------------------------------------------------
def workspace(variant, q, v, chunk=0):
    """A workspace tensor (uint8, on q's device) for the two-pass prefill of
    inputs shaped like q [B,T,H,dk] and v [B,T,H,dv]; None if none is needed."""
    vid = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    B, T, H, dk = q.shape
    n = kdn_chunk_prefill_workspace_size(vid, DTYPES[q.dtype], B, T, H, dk,
                                         v.shape[-1], chunk)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def prefill(variant, q, k, v, alpha=None, beta=None, proc_noise=None,
            obs_noise=None, S0=None, p0=None, mu=1.0, chunk=0, out=None,
            workspace="auto", stream=None):
    """Chunkwise prefill.  q, k [B,T,H,dk], v [B,T,H,dv] (float32 or bf16).
    Returns (o, S, p); p is None unless the variant is a KDN ([B,H,dk] for
    diag_kdn, [B,H] for iso_kdn).  ``out`` may pass
    preallocated (o, S_out, p_out).  ``workspace``: "auto" allocates one for
    the two-pass schedule, None selects the single-pass kernel, a uint8
    tensor from :func:`workspace` is used as given."""
    vid = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = DTYPES[q.dtype]
    if out is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
        S = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
        p = _new_p(vid, B, H, dk, q.device)
    else:
        o, S, p = out
    f32, pshape = torch.float32, _p_shape(vid, B, H, dk)
    _expect([("q", q, (B, T, H, dk), q.dtype), ("k", k, (B, T, H, dk), q.dtype),
             ("v", v, (B, T, H, dv), q.dtype)]
            + _gate_specs(vid, (B, T, H), dk, q.dtype, alpha, beta, proc_noise, obs_noise)
            + [("S0", S0, (B, H, dk, dv), f32), ("p0", p0, pshape, f32),
               ("o", o, (B, T, H, dv), q.dtype), ("S_out", S, (B, H, dk, dv), f32),
               ("p_out", p, pshape, f32)], q.device)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"kdn: workspace must be 'auto', None or a tensor, not {workspace!r}")
        workspace = globals()["workspace"](vid, q, v, chunk)
    kdn_chunk_prefill(vid, dt, B, T, H, dk, dv, chunk, mu, q, k, v, alpha, beta,
                      proc_noise, obs_noise, S0, p0, o, S, p, workspace, 0, stream)
    return o, S, p


def decode(variant, q, k, v, S, p=None, alpha=None, beta=None, proc_noise=None,
           obs_noise=None, mu=1.0, o=None, stream=None):
    """One decode step; S [N,H,dk,dv] (and p: [N,H,dk] for diag_kdn, [N,H]
    for iso_kdn) are updated in place.  Returns o [N,H,dv]."""
    vid = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    N, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    f32 = torch.float32
    _expect([("q", q, (N, H, dk), q.dtype), ("k", k, (N, H, dk), q.dtype),
             ("v", v, (N, H, dv), q.dtype)]
            + _gate_specs(vid, (N, H), dk, q.dtype, alpha, beta, proc_noise, obs_noise)
            + [("S", S, (N, H, dk, dv), f32), ("p", p, _p_shape(vid, N, H, dk), f32),
               ("o", o, (N, H, dv), q.dtype)], q.device)
    kdn_recurrent_decode(vid, DTYPES[q.dtype], N, H, dk, dv, mu, q, k, v, alpha,
                         beta, proc_noise, obs_noise, S, p, o, stream)
    return o


def decode_multi(variant, q, k, v, alpha=None, beta=None, proc_noise=None,
                 obs_noise=None, S0=None, p0=None, mu=1.0, out=None, stream=None):
    """T decode steps in one pass over the state (speculative verify).
    q, k [N,T,H,dk], v [N,T,H,dv]; S0 [N,H,dk,dv] (None: zeros) and p0
    ([N,H,dk] diag_kdn, [N,H] iso_kdn) are read, not modified, unless ``out``
    passes them as S_out / p_out (in place).  Returns (o [N,T,H,dv], S_out,
    p_out); p_out is None unless the variant is a KDN."""
    vid = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    N, T, H, dk = q.shape
    dv = v.shape[-1]
    if out is None:
        o = torch.empty((N, T, H, dv), dtype=q.dtype, device=q.device)
        S = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
        p = _new_p(vid, N, H, dk, q.device)
    else:
        o, S, p = out
    f32, pshape = torch.float32, _p_shape(vid, N, H, dk)
    _expect([("q", q, (N, T, H, dk), q.dtype), ("k", k, (N, T, H, dk), q.dtype),
             ("v", v, (N, T, H, dv), q.dtype)]
            + _gate_specs(vid, (N, T, H), dk, q.dtype, alpha, beta, proc_noise, obs_noise)
            + [("S0", S0, (N, H, dk, dv), f32), ("p0", p0, pshape, f32),
               ("o", o, (N, T, H, dv), q.dtype), ("S_out", S, (N, H, dk, dv), f32),
               ("p_out", p, pshape, f32)], q.device)
    kdn_recurrent_decode_multi(vid, DTYPES[q.dtype], N, T, H, dk, dv, mu, q, k, v,
                               alpha, beta, proc_noise, obs_noise, S0, p0, o, S, p,
                               stream)
    return o, S, p


def prefill_backward(variant, q, k, v, d_o, alpha=None, beta=None, proc_noise=None,
                     obs_noise=None, S0=None, p0=None, dS_out=None, dp_out=None, mu=1.0,
                     chunk=0, out=None, workspace=None, stream=None):
    """Gradients of :func:`prefill` (every variant) for the cotangents
    d_o [B,T,H,dv], dS_out [B,H,dk,dv] and (KDN) dp_out shaped as p0 (None:
    zero).  Returns a dict of float32 tensors: dq, dk, dv, dlog_alpha
    (alpha dL/dalpha: [B,T,H] for gated_deltanet, [B,T,H,dk] for kda and the
    KDNs, None for deltanet), dbeta (None for the KDNs), dS0, and for the KDNs
    dproc_noise, dobs_noise, dp0.  ``workspace``: a uint8 tensor of at least
    the queried size, or None to allocate one."""
    vid = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    iso = vid in (3, 4)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = DTYPES[q.dtype]
    dev = q.device
    if out is None:
        f = torch.float32
        new = lambda *shape: torch.empty(shape, dtype=f, device=dev)
        out = dict(dq=new(B, T, H, dk), dk=new(B, T, H, dk), dv=new(B, T, H, dv),
                   dlog_alpha=None if vid == 0 else (new(B, T, H) if vid == 1
                                                     else new(B, T, H, dk)),
                   dbeta=None if iso else new(B, T, H), dS0=new(B, H, dk, dv),
                   dproc_noise=new(B, T, H, dk) if iso else None,
                   dobs_noise=new(B, T, H) if iso else None,
                   dp0=(new(B, H, dk) if vid == 3 else new(B, H)) if iso else None)
    f32, pshape = torch.float32, _p_shape(vid, B, H, dk)
    la_shape = (B, T, H) if vid == 1 else (B, T, H, dk)
    _expect([("q", q, (B, T, H, dk), q.dtype), ("k", k, (B, T, H, dk), q.dtype),
             ("v", v, (B, T, H, dv), q.dtype), ("d_o", d_o, (B, T, H, dv), q.dtype)]
            + _gate_specs(vid, (B, T, H), dk, q.dtype, alpha, beta, proc_noise, obs_noise)
            + [("S0", S0, (B, H, dk, dv), f32), ("p0", p0, pshape, f32),
               ("dS_out", dS_out, (B, H, dk, dv), f32), ("dp_out", dp_out, pshape, f32),
               ("dq", out["dq"], (B, T, H, dk), f32), ("dk", out["dk"], (B, T, H, dk), f32),
               ("dv", out["dv"], (B, T, H, dv), f32),
               ("dlog_alpha", out["dlog_alpha"], la_shape, f32),
               ("dbeta", out["dbeta"], (B, T, H), f32),
               ("dproc_noise", out["dproc_noise"], (B, T, H, dk), f32),
               ("dobs_noise", out["dobs_noise"], (B, T, H), f32),
               ("dS0", out["dS0"], (B, H, dk, dv), f32), ("dp0", out["dp0"], pshape, f32)],
            q.device)
    if workspace is None:
        n = kdn_chunk_prefill_backward_workspace_size(vid, dt, B, T, H, dk, dv, chunk)
        workspace = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
    kdn_chunk_prefill_backward(vid, dt, B, T, H, dk, dv, chunk, mu, q, k, v, alpha, beta,
                               proc_noise, obs_noise, S0, p0, d_o, dS_out, dp_out,
                               out["dq"], out["dk"], out["dv"], out["dlog_alpha"],
                               out["dbeta"], out["dproc_noise"], out["dobs_noise"],
                               out["dS0"], out["dp0"], workspace, 0, stream)
    return out
