"""Python wrapper around the fp64 C oracle (oracle/kda_oracle.c).

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  It never touches the
HIP library and the HIP library never touches it.

The oracle is the plain token-by-token recurrence of the gated delta rule
(reading of "From Numerical Stability to Load Balancing ..." section 2.1 and
"Demystifying Trillion-Parameter MoE Models ..." Breakthrough 1 part 1: a
fixed-shape state that is decayed and then written with key/value outer
products), with the bounded gate g = g_min * sigmoid(w) of the same pages'
section 2.2 / Breakthrough 1 part 2, or g = -softplus(w) when g_min = -inf.

All arrays are float64 numpy arrays in row-major layout:
  q, k, w [B,H,T,dk];  v [B,H,T,dv];  beta [B,H,T];  S0 [B,H,dk,dv] or None.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile kda_oracle.c into oracle/liboracle.so with gcc (plain C, -O2)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, _SRC,
                               "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # KDA_ORACLE_LIB: an already built copy of this oracle (the sanitizer test's instrumented build)
        lib = ctypes.CDLL(os.environ.get("KDA_ORACLE_LIB") or build())
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.kda_oracle_f64.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.c_double,
                                       i64, i64, i64, i64, i64, dp, dp, ctypes.c_int]
        lib.kda_oracle_f64.restype = ctypes.c_int
        lib.kda_oracle_spans_f64.argtypes = [dp, ctypes.c_double, i64, i64, i64, i64, i64, dp]
        lib.kda_oracle_spans_f64.restype = ctypes.c_int
        lib.kda_oracle_gate_array.argtypes = [dp, i64, ctypes.c_double, dp]
        lib.kda_oracle_gate_array.restype = ctypes.c_int
        lib.kda_oracle_bwd_f64.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.c_double, i64, i64, i64, i64, i64,
                                           dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.kda_oracle_bwd_f64.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def kda_reference(q, k, v, w, beta, S0=None, g_min=-5.0, nthreads=None):
    """Token-by-token fp64 forward. Returns (o [B,H,T,dv], S_final [B,H,dk,dv])."""
    q, k, v, w, beta, S0 = (_f64(x) for x in (q, k, v, w, beta, S0))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, H, T, dk) and w.shape == (B, H, T, dk)
    assert v.shape == (B, H, T, dv) and beta.shape == (B, H, T)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.empty((B, H, T, dv), dtype=np.float64)
    S = np.empty((B, H, dk, dv), dtype=np.float64)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    rc = _load().kda_oracle_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(S0),
                                float(g_min), B, H, T, dk, dv, _ptr(o), _ptr(S), int(nthreads))
    if rc != 0:
        raise ValueError("kda_oracle_f64 rejected its arguments")
    return o, S


def kda_backward(q, k, v, w, beta, S0, g_min, dO, dSf=None, nthreads=None):
    """fp64 gradients of <dO, o> + <dSf, S_final> by the adjoint of the token recurrence.
    Returns (dq, dk, dv, dw, dbeta, dS0)."""
    q, k, v, w, beta, S0, dO, dSf = (_f64(x) for x in (q, k, v, w, beta, S0, dO, dSf))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert dO.shape == (B, H, T, dv)
    out = dict(dq=np.zeros((B, H, T, dk)), dk=np.zeros((B, H, T, dk)), dv=np.zeros((B, H, T, dv)),
               dw=np.zeros((B, H, T, dk)), dbeta=np.zeros((B, H, T)), dS0=np.zeros((B, H, dk, dv)))
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    rc = _load().kda_oracle_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(S0), float(g_min),
                                    B, H, T, dk, dv, _ptr(dO), _ptr(dSf),
                                    _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dw"]),
                                    _ptr(out["dbeta"]), _ptr(out["dS0"]), int(nthreads))
    if rc != 0:
        raise ValueError("kda_oracle_bwd_f64 rejected its arguments")
    return out["dq"], out["dk"], out["dv"], out["dw"], out["dbeta"], out["dS0"]


def gate(w, g_min=-5.0):
    """Elementwise g(w): g_min*sigmoid(w), or -softplus(w) when g_min = -inf."""
    w = _f64(np.asarray(w))
    out = np.empty_like(w)
    rc = _load().kda_oracle_gate_array(_ptr(w), w.size, float(g_min), _ptr(out))
    if rc != 0:
        raise ValueError("kda_oracle_gate_array rejected its arguments")
    return out


def chunk_spans(w, g_min=-5.0, chunk=16):
    """spans [B,H,NC]: per chunk, min over key channels of the chunk-local sum of g."""
    w = _f64(w)
    B, H, T, dk = w.shape
    NC = (T + chunk - 1) // chunk
    out = np.empty((B, H, NC), dtype=np.float64)
    rc = _load().kda_oracle_spans_f64(_ptr(w), float(g_min), B, H, T, dk, chunk, _ptr(out))
    if rc != 0:
        raise ValueError("kda_oracle_spans_f64 rejected its arguments")
    return out


# Threshold on the chunk span below which a 16-token tile can no longer use
# reciprocal scaling safely: 16 * g_min with g_min = -5 ("From Numerical
# Stability ..." section 2.2; "Demystifying ..." Breakthrough 1 part 2).
SPAN_LIMIT = -80.0


def predicted_flags(w, g_min=-5.0, chunk=16, limit=SPAN_LIMIT):
    """Boolean [B,H,NC]: chunks whose span falls strictly below the limit."""
    return chunk_spans(w, g_min, chunk) < limit
