"""Python binding of libkda, the KDA operator for MI355X (gfx950).

The functions here carry the C entry points' names and only marshal arguments:
they check torch tensors (device, dtype, shape, contiguity), allocate outputs
and workspace with torch (device memory is plumbing), pass raw pointers and
the current HIP stream to libkda, and raise on a non-OK status.  Every step of
the operator runs in libkda's HIP kernels; there is no fallback.  If libkda.so
has not been built, every call raises.

    o, S_T = kda_chunk_fwd(q, k, v, theta, beta, S0=None)
    o      = kda_decode_step(q, k, v, theta, beta, S)        # S updated in place
    o, S_T = kda_chunk_fwd_gated(q, k, v, theta, beta, z)    # o * sigmoid(z)
    o, S_T = kda_chunk_fwd_noalloc(q, k, v, theta, beta, S0=None, o=o, S_T=S_T)
    o      = kda_decode_step_gated(q, k, v, theta, beta, S, z)
    g, gc  = kda_gate(theta)
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")
HEADER_PATH = os.path.join(_HERE, "..", "include", "kda.h")

KDA_BF16, KDA_F32 = 0, 1
KDA_CHUNK = 16
KDA_G_MIN = -5.0

_lib = None


class KdaError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load libkda.so (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it first "
                           "(python -m chunked_gated_delta_12_amd.build)")
    lib = ctypes.CDLL(path)
    c_int, c_size, vp, fp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p
    lib.kda_chunk_fwd.argtypes = [c_int] * 7 + [vp] * 3 + [fp] * 3 + [vp, fp, vp, c_size, vp]
    lib.kda_chunk_fwd.restype = c_int
    lib.kda_chunk_fwd_workspace_size.argtypes = [c_int] * 6 + [ctypes.POINTER(c_size)]
    lib.kda_chunk_fwd_workspace_size.restype = c_int
    lib.kda_chunk_fwd_auto_segments.argtypes = [c_int] * 5
    lib.kda_chunk_fwd_auto_segments.restype = c_int
    lib.kda_decode_step.argtypes = [c_int] * 5 + [vp] * 3 + [fp] * 3 + [vp, vp]
    lib.kda_decode_step.restype = c_int
    lib.kda_chunk_fwd_noalloc.argtypes = [c_int] * 7 + [vp] * 3 + [fp] * 3 + [vp, fp, vp]
    lib.kda_chunk_fwd_noalloc.restype = c_int
    lib.kda_chunk_fwd_gated.argtypes = [c_int] * 7 + [vp] * 3 + [fp] * 3 + [vp, vp, fp, vp, c_size, vp]
    lib.kda_chunk_fwd_gated.restype = c_int
    lib.kda_chunk_bwd.argtypes = [c_int] * 6 + [vp] * 3 + [fp] * 3 + [vp, fp] + [fp] * 6 + [vp, c_size, vp]
    lib.kda_chunk_bwd.restype = c_int
    lib.kda_chunk_bwd_workspace_size.argtypes = [c_int] * 5 + [ctypes.POINTER(c_size)]
    lib.kda_chunk_bwd_workspace_size.restype = c_int
    lib.kda_chunk_fwd_unbounded.argtypes = [c_int] * 6 + [vp] * 3 + [fp] * 3 + [vp, fp, vp]
    lib.kda_chunk_fwd_unbounded.restype = c_int
    lib.kda_decode_step_gated.argtypes = [c_int] * 5 + [vp] * 3 + [fp] * 3 + [vp, vp, vp]
    lib.kda_decode_step_gated.restype = c_int
    lib.kda_gate.argtypes = [c_int] * 4 + [fp, fp, fp, vp]
    lib.kda_gate.restype = c_int
    lib.kda_status_string.argtypes = [c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = c_int
    _lib = lib
    return lib


def header_functions(path: str = HEADER_PATH):
    """Names of the functions include/kda.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


def _check(fn, status):
    if status != 0:
        lib = load_library()
        raise KdaError(fn, status, lib.kda_last_error().decode() or lib.kda_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _need(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def kda_chunk_fwd_auto_segments(B, T, H, dk, dv) -> int:
    return int(load_library().kda_chunk_fwd_auto_segments(B, T, H, dk, dv))


def kda_chunk_fwd_workspace_size(B, T, H, dk, dv, segments=0) -> int:
    n = ctypes.c_size_t(0)
    _check("kda_chunk_fwd_workspace_size",
           load_library().kda_chunk_fwd_workspace_size(B, T, H, dk, dv, segments, ctypes.byref(n)))
    return int(n.value)


def kda_chunk_fwd(q, k, v, theta, beta, S0=None, *, segments=0, o=None, S_T=None,
                  want_state=True, workspace=None, stream=None):
    """Chunked prefill.  q, k [B,T,H,dk], v [B,T,H,dv] (bf16 or fp32), theta
    [B,T,H,dk] fp32, beta [B,T,H] fp32, S0 [B,H,dk,dv] fp32 or None.
    Returns (o, S_T); S_T is None when want_state is False."""
    return _chunk_fwd(q, k, v, theta, beta, S0, None, segments, o, S_T, want_state, workspace, stream)


def kda_chunk_fwd_gated(q, k, v, theta, beta, z, S0=None, *, segments=0, o=None, S_T=None,
                        want_state=True, workspace=None, stream=None):
    """kda_chunk_fwd with the output gate: o * sigmoid(z), z [B,T,H,dv] of q's dtype."""
    return _chunk_fwd(q, k, v, theta, beta, S0, z, segments, o, S_T, want_state, workspace, stream)


def kda_chunk_fwd_noalloc(q, k, v, theta, beta, S0=None, *, segments=0, o=None, S_T=None,
                          want_state=True, stream=None):
    """kda_chunk_fwd without a workspace: libkda uses its static per-device scratch
    (KDA_NOALLOC_SCRATCH_BYTES).  Pass o and S_T to make the call allocate nothing."""
    return _chunk_fwd(q, k, v, theta, beta, S0, None, segments, o, S_T, want_state, None, stream,
                      noalloc=True)


def kda_chunk_fwd_unbounded(q, k, v, theta, beta, S0=None, *, o=None, S_T=None, want_state=True,
                            stream=None):
    """The ablation of the bound: the recurrence with the unbounded gate
    g = -softplus(theta) and position-wise fp32 diagonal tiles (one segment)."""
    return _chunk_fwd(q, k, v, theta, beta, S0, None, 1, o, S_T, want_state, None, stream, unbounded=True)


def _chunk_fwd(q, k, v, theta, beta, S0, z, segments, o, S_T, want_state, workspace, stream,
               unbounded=False, noalloc=False):
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    _need(q, "q", dt, (B, T, H, dk), dev)
    _need(k, "k", dt, (B, T, H, dk), dev)
    _need(v, "v", dt, (B, T, H, dv), dev)
    _need(theta, "theta", torch.float32, (B, T, H, dk), dev)
    _need(beta, "beta", torch.float32, (B, T, H), dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (B, H, dk, dv), dev)
    if z is not None:
        _need(z, "z", dt, (B, T, H, dv), dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _need(o, "o", dt, (B, T, H, dv), dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if S_T is not None:
        _need(S_T, "S_T", torch.float32, (B, H, dk, dv), dev)
    nbytes = 0 if (unbounded or noalloc) else kda_chunk_fwd_workspace_size(B, T, H, dk, dv, segments)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if unbounded:
        st = lib.kda_chunk_fwd_unbounded(code, B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(theta),
                                         _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T), _stream(q, stream))
        _check("kda_chunk_fwd_unbounded", st)
    elif noalloc:
        st = lib.kda_chunk_fwd_noalloc(code, B, T, H, dk, dv, segments, _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(theta), _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T),
                                       _stream(q, stream))
        _check("kda_chunk_fwd_noalloc", st)
    elif z is None:
        st = lib.kda_chunk_fwd(code, B, T, H, dk, dv, segments, _ptr(q), _ptr(k), _ptr(v), _ptr(theta),
                               _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T), _ptr(workspace), ws_bytes,
                               _stream(q, stream))
        _check("kda_chunk_fwd", st)
    else:
        st = lib.kda_chunk_fwd_gated(code, B, T, H, dk, dv, segments, _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(theta), _ptr(beta), _ptr(S0), _ptr(z), _ptr(o), _ptr(S_T),
                                     _ptr(workspace), ws_bytes, _stream(q, stream))
        _check("kda_chunk_fwd_gated", st)
    return o, S_T


def kda_chunk_bwd_workspace_size(B, T, H, dk, dv) -> int:
    n = ctypes.c_size_t(0)
    _check("kda_chunk_bwd_workspace_size",
           load_library().kda_chunk_bwd_workspace_size(B, T, H, dk, dv, ctypes.byref(n)))
    return int(n.value)


def kda_chunk_bwd(q, k, v, theta, beta, do, S0=None, dS_T=None, *, want_dS0=True, workspace=None,
                  stream=None):
    """Backward pass of kda_chunk_fwd for L = sum <do, o> + <dS_T, S_T>.  Inputs as
    kda_chunk_fwd plus do [B,T,H,dv] (q's dtype) and dS_T [B,H,dk,dv] fp32 or None.
    Returns a dict of fp32 tensors dq, dk, dv, dtheta, dbeta and dS0 (None unless
    want_dS0)."""
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    _need(q, "q", dt, (B, T, H, dk), dev)
    _need(k, "k", dt, (B, T, H, dk), dev)
    _need(v, "v", dt, (B, T, H, dv), dev)
    _need(theta, "theta", torch.float32, (B, T, H, dk), dev)
    _need(beta, "beta", torch.float32, (B, T, H), dev)
    _need(do, "do", dt, (B, T, H, dv), dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (B, H, dk, dv), dev)
    if dS_T is not None:
        _need(dS_T, "dS_T", torch.float32, (B, H, dk, dv), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"dq": torch.empty((B, T, H, dk), **f32), "dk": torch.empty((B, T, H, dk), **f32),
         "dv": torch.empty((B, T, H, dv), **f32), "dtheta": torch.empty((B, T, H, dk), **f32),
         "dbeta": torch.empty((B, T, H), **f32),
         "dS0": torch.empty((B, H, dk, dv), **f32) if want_dS0 else None}
    nbytes = kda_chunk_bwd_workspace_size(B, T, H, dk, dv)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.kda_chunk_bwd(code, B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(theta), _ptr(beta), _ptr(S0),
                           _ptr(do), _ptr(dS_T), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dtheta"]),
                           _ptr(g["dbeta"]), _ptr(g["dS0"]), _ptr(workspace), ws_bytes, _stream(q, stream))
    _check("kda_chunk_bwd", st)
    return g


def kda_decode_step(q, k, v, theta, beta, S, *, o=None, stream=None):
    """One decode step.  q, k [B,H,dk], v [B,H,dv] (bf16 or fp32), theta [B,H,dk]
    fp32, beta [B,H] fp32, S [B,H,dk,dv] fp32 (updated in place).  Returns o."""
    return _decode_step(q, k, v, theta, beta, S, None, o, stream)


def kda_decode_step_gated(q, k, v, theta, beta, S, z, *, o=None, stream=None):
    """kda_decode_step with the output gate: o * sigmoid(z), z [B,H,dv] of q's dtype."""
    return _decode_step(q, k, v, theta, beta, S, z, o, stream)


def _decode_step(q, k, v, theta, beta, S, z, o, stream):
    lib = load_library()
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    _need(q, "q", dt, (B, H, dk), dev)
    _need(k, "k", dt, (B, H, dk), dev)
    _need(v, "v", dt, (B, H, dv), dev)
    _need(theta, "theta", torch.float32, (B, H, dk), dev)
    _need(beta, "beta", torch.float32, (B, H), dev)
    _need(S, "S", torch.float32, (B, H, dk, dv), dev)
    if z is not None:
        _need(z, "z", dt, (B, H, dv), dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=dt, device=dev)
    _need(o, "o", dt, (B, H, dv), dev)
    if z is None:
        st = lib.kda_decode_step(code, B, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(theta), _ptr(beta),
                                 _ptr(S), _ptr(o), _stream(q, stream))
        _check("kda_decode_step", st)
    else:
        st = lib.kda_decode_step_gated(code, B, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(theta),
                                       _ptr(beta), _ptr(S), _ptr(z), _ptr(o), _stream(q, stream))
        _check("kda_decode_step_gated", st)
    return o


def kda_gate(theta, *, g=True, g_cum=True, stream=None):
    """Bounded gate. theta [B,T,H,dk] fp32 -> (g, g_cum) fp32 (either may be skipped
    by passing False).  Pre-allocated tensors may be passed instead of True."""
    lib = load_library()
    B, T, H, dk = theta.shape
    dev = theta.device
    _need(theta, "theta", torch.float32, (B, T, H, dk), dev)
    if g is True:
        g = torch.empty_like(theta)
    if g_cum is True:
        g_cum = torch.empty_like(theta)
    g = g if isinstance(g, torch.Tensor) else None
    g_cum = g_cum if isinstance(g_cum, torch.Tensor) else None
    for name, t in (("g", g), ("g_cum", g_cum)):
        if t is not None:
            _need(t, name, torch.float32, (B, T, H, dk), dev)
    st = lib.kda_gate(B, T, H, dk, _ptr(theta), _ptr(g), _ptr(g_cum), _stream(theta, stream))
    _check("kda_gate", st)
    return g, g_cum


__all__ = ["kda_chunk_fwd", "kda_chunk_fwd_noalloc", "kda_chunk_fwd_gated", "kda_chunk_fwd_unbounded", "kda_chunk_bwd",
           "kda_chunk_bwd_workspace_size", "kda_decode_step",
           "kda_decode_step_gated", "kda_gate", "kda_chunk_fwd_workspace_size",
           "kda_chunk_fwd_auto_segments", "load_library", "header_functions", "KdaError",
           "KDA_BF16", "KDA_F32", "KDA_CHUNK", "KDA_G_MIN"]
