"""fp64 CPU oracle for the Kimi Delta Attention operator -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product (the HIP library and its binding) never
does, and this package imports nothing from the product.

The arithmetic lives in ``kda_oracle.c`` (plain C, double precision); this
module only marshals numpy arrays into it.  See that file's header for what is
computed and which passage of the pages each step follows.

Parity of every function here is pinned by ``tests/test_oracle_pins.py``
(hand examples, closed forms, invariants, an independent parallel form).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

G_MIN = -5.0  # the pages' fixed lower bound on the log-decay
CHUNK = 16    # the pages' chunk length


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/libkda_oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int)
        lib.kda_oracle_gate.argtypes = [ctypes.c_long, dp, dp]
        lib.kda_oracle_gate.restype = None
        lib.kda_oracle_output_gate.argtypes = [ctypes.c_long, dp, dp, dp]
        lib.kda_oracle_gate_softplus.argtypes = [ctypes.c_long, dp, dp]
        lib.kda_oracle_gate_softplus.restype = None
        lib.kda_oracle_backward.argtypes = [ctypes.c_int] * 5 + [dp] * 14
        lib.kda_oracle_backward.restype = ctypes.c_int
        lib.kda_oracle_gate_backward.argtypes = [ctypes.c_long, dp, dp, dp]
        lib.kda_oracle_gate_backward.restype = None
        lib.kda_oracle_output_gate.restype = None
        lib.kda_oracle_gate_cumsum.argtypes = [ctypes.c_int] * 4 + [dp, dp]
        lib.kda_oracle_gate_cumsum.restype = None
        lib.kda_oracle_recurrence.argtypes = (
            [ctypes.c_int] * 5 + [dp] * 6 + [ip, ctypes.c_int, dp, dp, ctypes.c_int])
        lib.kda_oracle_recurrence.restype = ctypes.c_int
        lib.kda_oracle_chunk_fwd.argtypes = lib.kda_oracle_recurrence.argtypes
        lib.kda_oracle_chunk_fwd.restype = ctypes.c_int
        lib.kda_oracle_decode_step.argtypes = [ctypes.c_int] * 4 + [dp] * 7 + [ctypes.c_int]
        lib.kda_oracle_decode_step.restype = ctypes.c_int
        _lib = lib
    return _lib


def _d(a):
    """Exact widening to a contiguous float64 numpy array (bf16/fp32 -> fp64 is exact)."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: widen on the host
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(n, 16))


def gate(theta):
    """g = g_min * sigmoid(theta), elementwise, float64."""
    th = _d(theta)
    g = np.empty_like(th)
    _load().kda_oracle_gate(th.size, _p(th), _p(g))
    return g


def gate_softplus(theta):
    """g = -softplus(theta) = -ln(1 + e^theta), elementwise, float64: the
    unbounded log-decay the bounded gate replaces (ablation of the bound)."""
    th = _d(theta)
    g = np.empty_like(th)
    _load().kda_oracle_gate_softplus(th.size, _p(th), _p(g))
    return g


def chunk_fwd_unbounded(q, k, v, theta, beta, S0=None, cols=None, nthreads=None):
    """The recurrence with the unbounded gate g = -softplus(theta)."""
    return recurrence(q, k, v, gate_softplus(theta), beta, S0, cols=cols, nthreads=nthreads)


def backward(q, k, v, g, beta, S0, do, dS_T=None):
    """Gradients of L = sum_t <do_t, o_t> + <dS_T, S_T> for the recurrence with log-decay
    g given directly: dict of dq, dk, dv, dg [as the inputs], dbeta [B,T,H], dS0 [B,H,dk,dv]."""
    q, k, v, g, beta, do = _d(q), _d(k), _d(v), _d(g), _d(beta), _d(do)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and g.shape == q.shape and v.shape == (B, T, H, dv)
    assert beta.shape == (B, T, H) and do.shape == (B, T, H, dv)
    S0, dS_T = _d(S0), _d(dS_T)
    out = {"dq": np.empty_like(q), "dk": np.empty_like(k), "dv": np.empty_like(v), "dg": np.empty_like(g),
           "dbeta": np.empty_like(beta), "dS0": np.empty((B, H, dk, dv))}
    st = _load().kda_oracle_backward(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta), _p(S0),
                                     _p(do), _p(dS_T), _p(out["dq"]), _p(out["dk"]), _p(out["dv"]),
                                     _p(out["dg"]), _p(out["dbeta"]), _p(out["dS0"]))
    if st:
        raise RuntimeError(f"kda_oracle_backward failed ({st})")
    return out


def chunk_bwd(q, k, v, theta, beta, S0, do, dS_T=None):
    """backward() with the bounded gate g = g_min sigmoid(theta): adds dtheta."""
    th = _d(theta)
    out = backward(q, k, v, gate(th), beta, S0, do, dS_T)
    dth = np.empty_like(th)
    _load().kda_oracle_gate_backward(th.size, _p(th), _p(out["dg"]), _p(dth))
    out["dtheta"] = dth
    return out


def output_gate(o, z):
    """o * sigmoid(z), elementwise, float64 (o and z of the same shape)."""
    o, z = _d(o), _d(z)
    assert o.shape == z.shape
    out = np.empty_like(o)
    _load().kda_oracle_output_gate(o.size, _p(o), _p(z), _p(out))
    return out


def gate_cumsum(g):
    """Chunk-local (16-token) inclusive prefix sum of g [B, T, H, dk] along T."""
    g = _d(g)
    B, T, H, dk = g.shape
    out = np.empty_like(g)
    _load().kda_oracle_gate_cumsum(B, T, H, dk, _p(g), _p(out))
    return out


def _run(fn, q, k, v, x, beta, S0, cols, nthreads):
    q, k, v, x, beta = _d(q), _d(k), _d(v), _d(x), _d(beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, T, H, dk) and x.shape == (B, T, H, dk)
    assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    S0 = _d(S0)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    if cols is not None:
        cols_arr = np.ascontiguousarray(cols, dtype=np.int32)
        nc = int(cols_arr.size)
        cp = cols_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int))
    else:
        cols_arr, nc, cp = None, dv, None
    o = np.empty((B, T, H, nc), dtype=np.float64)
    S_T = np.empty((B, H, dk, nc), dtype=np.float64)
    st = fn(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(x), _p(beta), _p(S0), cp,
            nc if cols is not None else 0, _p(o), _p(S_T),
            nthreads or default_threads())
    if st != 0:
        raise RuntimeError(f"oracle failed with status {st}")
    return o, S_T


def recurrence(q, k, v, g, beta, S0=None, cols=None, nthreads=None):
    """Token-by-token recurrence with log-decay g given. Returns (o, S_T) float64."""
    return _run(_load().kda_oracle_recurrence, q, k, v, g, beta, S0, cols, nthreads)


def chunk_fwd(q, k, v, theta, beta, S0=None, cols=None, nthreads=None):
    """Chunked prefill result: gate(theta) then the recurrence. Returns (o, S_T)."""
    return _run(_load().kda_oracle_chunk_fwd, q, k, v, theta, beta, S0, cols, nthreads)


def chunk_fwd_column_blocks(q, k, v, theta, beta, S0=None, nthreads=None):
    """chunk_fwd over every value column for few (batch, head) sequences: the
    columns are cut into blocks that run concurrently (each block is the column
    subset of the same recurrence, which evolves independently of the other
    columns), so all threads work even when B*H is small.  Returns (o, S_T)."""
    import concurrent.futures as cf
    q, k, v, theta, beta, S0 = _d(q), _d(k), _d(v), _d(theta), _d(beta), _d(S0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    n = nthreads or default_threads()
    nblk = max(1, min(n // max(1, B * H), dv))
    if nblk == 1:
        return chunk_fwd(q, k, v, theta, beta, S0, nthreads=n)
    g = gate(theta)
    blocks = [list(range(i * dv // nblk, (i + 1) * dv // nblk)) for i in range(nblk)]
    o = np.empty((B, T, H, dv))
    S_T = np.empty((B, H, dk, dv))

    def one(cols):
        ob, sb = recurrence(q, k, v, g, beta, S0, cols=cols, nthreads=B * H)
        o[..., cols] = ob
        S_T[..., cols] = sb

    with cf.ThreadPoolExecutor(max_workers=nblk) as ex:
        list(ex.map(one, blocks))
    return o, S_T


def decode_step(q, k, v, theta, beta, S, nthreads=None):
    """One decode step. q,k,theta [B,H,dk], v [B,H,dv], beta [B,H], S [B,H,dk,dv].
    Returns (o [B,H,dv], S_new) without modifying the caller's S."""
    q, k, v, theta, beta = _d(q), _d(k), _d(v), _d(theta), _d(beta)
    S = _d(S).copy()
    B, H, dk = q.shape
    dv = v.shape[-1]
    assert S.shape == (B, H, dk, dv) and beta.shape == (B, H)
    o = np.empty((B, H, dv), dtype=np.float64)
    st = _load().kda_oracle_decode_step(B, H, dk, dv, _p(q), _p(k), _p(v), _p(theta),
                                        _p(beta), _p(S), _p(o),
                                        nthreads or default_threads())
    if st != 0:
        raise RuntimeError(f"oracle failed with status {st}")
    return o, S
