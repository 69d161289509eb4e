"""torch-facing wrappers over libkda.so.  Argument marshalling only: every
step of the computation runs in the library's HIP kernels.  torch provides the
device memory (outputs, workspace, statistics) and the stream."""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import KdaError, KdaOpts, KdaShape

_PATHS = {"auto": 0, "vector": 1, "fused": 3, "corr": 4}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.DTYPE_BF16
    if t.dtype == torch.float32:
        return _lib.DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr()) if t.numel() > 0 else None


def _check(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_stream(stream, *tensors):
    """Tell torch's caching allocator that `stream` uses these tensors: memory allocated on the
    current stream but written by kernels on another one must not be handed out again before
    that stream's work on it is done."""
    if stream == torch.cuda.current_stream(stream.device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def make_shape(B, H, T, dk, dv, dtype_code) -> KdaShape:
    return KdaShape(int(B), int(H), int(T), int(dk), int(dv), int(dtype_code), 0)


def workspace_bytes(B, H, T, dk, dv, dtype=torch.bfloat16, chunk=16, path: str = "auto") -> int:
    code = _lib.DTYPE_BF16 if dtype == torch.bfloat16 else _lib.DTYPE_F32
    opts = KdaOpts(0, 0, _PATHS[path], 0, None, None)
    return _lib.workspace_bytes(make_shape(B, H, T, dk, dv, code), chunk, opts)


def chunk_fwd(q, k, v, w, beta, S0=None, g_min: float = -5.0, chunk: int = 16, *,
              out=None, S_final=None, stats: bool = True, workspace=None, stream=None,
              disable_fallback: bool = False, force_fallback: int = 0,
              path: str = "auto", events=None, seg_steps: int = 0):
    """KDA chunked forward through kda_chunk_fwd_ex.

    q, k, w: [B,H,T,dk]; v: [B,H,T,dv]; beta: [B,H,T] (all bf16 or all fp32,
    on one GPU); S0: optional fp32 [B,H,dk,dv].  g_min = -inf selects the
    unbounded gate.  Returns (o, S_final, stats) with stats an int32[4] device
    tensor (see decode_stats) or None.  Asynchronous on `stream` (default: the
    current torch stream).  `events` = (begin, end) HipEvent pair recorded
    before the first kernel of the call and after its last.  `seg_steps` > 0
    fixes the matrix-core path's sequence segment length (in 32-token steps).
    `path`: "auto" (bf16 with dk = dv = 128: "corr"; otherwise "vector"), "vector" (fp32 vector
    kernel), "fused" (map pass, chaining, output pass) or "corr" (one pass
    over every segment, chaining, correction of the outputs of segments >= 1).
    `force_fallback` = 1 (or True) gives every chunk a flagged chunk's handling, 2 the per-pair
    factors on every chunk; `disable_fallback` lets flagged chunks take the plain tiles.
    """
    if q.dim() != 4:
        raise ValueError("q must be [B,H,T,dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must live on a GPU (the library has no CPU path)")
    _check(q, "q", (B, H, T, dk), dt, dev)
    _check(k, "k", (B, H, T, dk), dt, dev)
    _check(w, "w", (B, H, T, dk), dt, dev)
    _check(v, "v", (B, H, T, dv), dt, dev)
    _check(beta, "beta", (B, H, T), dt, dev)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    else:
        _check(out, "out", (B, H, T, dv), dt, dev)
    if S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    else:
        _check(S_final, "S_final", (B, H, dk, dv), torch.float32, dev)
    shape = make_shape(B, H, T, dk, dv, _dtype_code(q))
    opts = KdaOpts(int(bool(disable_fallback)), int(force_fallback), _PATHS[path], int(seg_steps),
                   events[0].handle if events else None, events[1].handle if events else None)
    plain = not (disable_fallback or force_fallback or path != "auto" or seg_steps or events)
    ws_need = _lib.workspace_bytes(shape, chunk, None if plain else opts)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    st = torch.empty(4, dtype=torch.int32, device=dev) if stats else None
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    _on_stream(stream, out, S_final, workspace, st)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(S0), ctypes.c_float(g_min), int(chunk),
            ctypes.byref(shape), _ptr(out), _ptr(S_final), _ptr(workspace), ws_len, _ptr(st),
            ctypes.c_void_p(stream.cuda_stream))
    with torch.cuda.device(dev):
        if plain:   # no option set: the plain entry point
            rc, where = _lib.load().kda_chunk_fwd(*args), "kda_chunk_fwd"
        else:
            rc, where = _lib.load().kda_chunk_fwd_ex(*args, ctypes.byref(opts)), "kda_chunk_fwd_ex"
    if rc != 0:
        raise KdaError(rc, where, _lib.last_hip_error() if rc == _lib.KDA_ERR_HIP else "")
    return out, S_final, st


def chunk_fwd_noalloc(q, k, v, w, beta, S0=None, g_min: float = -5.0, chunk: int = 16, *,
                      out=None, S_final=None, stats: bool = True, stream=None):
    """KDA chunked forward through kda_chunk_fwd_noalloc: the library takes the call's scratch from its
    own static device array (no workspace argument).  Same arguments as chunk_fwd without the options;
    where chunk_fwd takes the corrected matrix-core plan this takes the fused one (whose scratch fits
    the array), so the results equal chunk_fwd(..., path="fused") bit for bit and the automatic
    chunk_fwd to the rounding of the two plans.  out, S_final and stats are allocated here when not
    given (the C entry point itself allocates nothing).  Calls that overlap in time on one GPU share
    that array and race."""
    if q.dim() != 4:
        raise ValueError("q must be [B,H,T,dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must live on a GPU (the library has no CPU path)")
    _check(q, "q", (B, H, T, dk), dt, dev)
    _check(k, "k", (B, H, T, dk), dt, dev)
    _check(w, "w", (B, H, T, dk), dt, dev)
    _check(v, "v", (B, H, T, dv), dt, dev)
    _check(beta, "beta", (B, H, T), dt, dev)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    else:
        _check(out, "out", (B, H, T, dv), dt, dev)
    if S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    else:
        _check(S_final, "S_final", (B, H, dk, dv), torch.float32, dev)
    shape = make_shape(B, H, T, dk, dv, _dtype_code(q))
    st = torch.empty(4, dtype=torch.int32, device=dev) if stats else None
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    _on_stream(stream, out, S_final, st)
    with torch.cuda.device(dev):
        rc = _lib.load().kda_chunk_fwd_noalloc(
            _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(S0), ctypes.c_float(g_min), int(chunk),
            ctypes.byref(shape), _ptr(out), _ptr(S_final), _ptr(st), ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise KdaError(rc, "kda_chunk_fwd_noalloc", _lib.last_hip_error() if rc == _lib.KDA_ERR_HIP else "")
    return out, S_final, st


def decode_stats(st: torch.Tensor) -> dict:
    """int32[4] device tensor -> dict (synchronises)."""
    a = st.cpu()
    return {
        "n_chunks": int(a[0].item()) & 0xFFFFFFFF,
        "n_flagged": int(a[1].item()) & 0xFFFFFFFF,
        "n_nonfinite": int(a[2].item()) & 0xFFFFFFFF,
        "min_span": float(a[3:4].view(torch.float32).item()),
    }


def gate_prefix(w, g_min: float = -5.0, chunk: int = 16, stream=None):
    """Gate / in-chunk prefix stage alone: returns (g, G, span, flags) device tensors."""
    if not isinstance(w, torch.Tensor) or w.dim() != 4:
        raise ValueError("w must be a [B,H,T,dk] tensor")
    B, H, T, dk = w.shape
    dev = w.device
    if dev.type != "cuda":
        raise ValueError("w must live on a GPU (the library has no CPU path)")
    _check(w, "w", (B, H, T, dk), w.dtype, dev)
    _dtype_code(w)
    NC = (T + chunk - 1) // chunk
    g = torch.empty((B, H, T, dk), dtype=torch.float32, device=dev)
    G = torch.empty_like(g)
    span = torch.empty((B, H, NC), dtype=torch.float32, device=dev)
    flags = torch.empty((B, H, NC), dtype=torch.uint8, device=dev)
    shape = make_shape(B, H, T, dk, dk, _dtype_code(w))
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    _on_stream(stream, g, G, span, flags)
    with torch.cuda.device(dev):
        rc = _lib.load().kda_gate_prefix(_ptr(w), ctypes.c_float(g_min), int(chunk), ctypes.byref(shape),
                                         _ptr(g), _ptr(G), _ptr(span), _ptr(flags),
                                         ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise KdaError(rc, "kda_gate_prefix", _lib.last_hip_error() if rc == _lib.KDA_ERR_HIP else "")
    return g, G, span, flags


def decode(q, k, v, w, beta, S, g_min: float = -5.0, *, out=None, stream=None):
    """Recurrent decode through kda_decode: advances the fp32 state S [B,H,dk,dv] in place by the
    T tokens of q, k, w [B,H,T,dk], v [B,H,T,dv], beta [B,H,T] (T is typically 1) and returns
    o [B,H,T,dv].  Asynchronous on `stream` (default: the current torch stream)."""
    if q.dim() != 4:
        raise ValueError("q must be [B,H,T,dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must live on a GPU (the library has no CPU path)")
    _check(q, "q", (B, H, T, dk), dt, dev)
    _check(k, "k", (B, H, T, dk), dt, dev)
    _check(w, "w", (B, H, T, dk), dt, dev)
    _check(v, "v", (B, H, T, dv), dt, dev)
    _check(beta, "beta", (B, H, T), dt, dev)
    _check(S, "S", (B, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    else:
        _check(out, "out", (B, H, T, dv), dt, dev)
    shape = make_shape(B, H, T, dk, dv, _dtype_code(q))
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    _on_stream(stream, out)
    with torch.cuda.device(dev):
        rc = _lib.load().kda_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(S),
                                    ctypes.c_float(g_min), ctypes.byref(shape), _ptr(out),
                                    ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise KdaError(rc, "kda_decode", _lib.last_hip_error() if rc == _lib.KDA_ERR_HIP else "")
    return out


def chunk_bwd(q, k, v, w, beta, dO, S0=None, dS_final=None, g_min: float = -5.0, chunk: int = 16, *,
              want_dS0: bool = True, workspace=None, stream=None, events=None):
    """Gradients of the chunked forward through kda_chunk_bwd, given dO = dL/do [B,H,T,dv] (the
    inputs' dtype) and dS_final = dL/dS_final (fp32 [B,H,dk,dv] or None for zero).  Returns fp32
    (dq, dk, dv, dw, dbeta, dS0); dS0 is None when want_dS0 is False.  Asynchronous on `stream`.
    `events` = (begin, end) torch.cuda.Event pair recorded on `stream` around the library call (the
    library launches on that stream, so the pair brackets exactly its kernels)."""
    if q.dim() != 4:
        raise ValueError("q must be [B,H,T,dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must live on a GPU (the library has no CPU path)")
    _check(q, "q", (B, H, T, dk), dt, dev)
    _check(k, "k", (B, H, T, dk), dt, dev)
    _check(w, "w", (B, H, T, dk), dt, dev)
    _check(v, "v", (B, H, T, dv), dt, dev)
    _check(beta, "beta", (B, H, T), dt, dev)
    _check(dO, "dO", (B, H, T, dv), dt, dev)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if dS_final is not None:
        _check(dS_final, "dS_final", (B, H, dk, dv), torch.float32, dev)
    shape = make_shape(B, H, T, dk, dv, _dtype_code(q))
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty((B, H, T, dk), **f32)
    dk_ = torch.empty((B, H, T, dk), **f32)
    dv_ = torch.empty((B, H, T, dv), **f32)
    dw = torch.empty((B, H, T, dk), **f32)
    dbeta = torch.empty((B, H, T), **f32)
    dS0 = torch.empty((B, H, dk, dv), **f32) if want_dS0 else None
    need = _lib.bwd_workspace_bytes(shape, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, {need} needed")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    _on_stream(stream, dq, dk_, dv_, dw, dbeta, dS0, workspace)
    with torch.cuda.device(dev):
        if events is not None:
            events[0].record(stream)
        rc = _lib.load().kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(S0),
                                       ctypes.c_float(g_min), int(chunk), ctypes.byref(shape), _ptr(dO),
                                       _ptr(dS_final), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dw), _ptr(dbeta),
                                       _ptr(dS0), _ptr(workspace), ctypes.c_size_t(need),
                                       ctypes.c_void_p(stream.cuda_stream))
        if events is not None:
            events[1].record(stream)
    if rc != 0:
        raise KdaError(rc, "kda_chunk_bwd", _lib.last_hip_error() if rc == _lib.KDA_ERR_HIP else "")
    return dq, dk_, dv_, dw, dbeta, dS0


def is_unbounded(g_min: float) -> bool:
    return math.isinf(g_min) and g_min < 0
