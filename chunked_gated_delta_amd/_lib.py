"""ctypes view of libkda.so (include/kda.h).  Loading fails loudly when the
library has not been built; there is no other implementation to fall back to."""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
# KDA_LIB_PATH: another build of this library (the sanitizer test's host-only instrumented build)
LIB_PATH = os.environ.get("KDA_LIB_PATH") or os.path.join(PKG, "libkda.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "kda.h")

KDA_OK = 0
KDA_ERR_NULL = -1
KDA_ERR_SHAPE = -2
KDA_ERR_UNSUPPORTED = -3
KDA_ERR_ARG = -4
KDA_ERR_HIP = -5
KDA_ERR_SCRATCH = -6
NOALLOC_SCRATCH_BYTES = 64 << 20   # KDA_NOALLOC_SCRATCH_BYTES of include/kda.h

DTYPE_F32 = 0
DTYPE_BF16 = 1


class KdaShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("T", ctypes.c_int64),
                ("dk", ctypes.c_int64), ("dv", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class KdaStats(ctypes.Structure):
    _fields_ = [("n_chunks", ctypes.c_uint32), ("n_flagged", ctypes.c_uint32),
                ("n_nonfinite", ctypes.c_uint32), ("min_span", ctypes.c_float)]


class KdaOpts(ctypes.Structure):
    _fields_ = [("disable_fallback", ctypes.c_int32), ("force_fallback", ctypes.c_int32),
                ("path", ctypes.c_int32), ("seg_steps", ctypes.c_int32),
                ("ev_begin", ctypes.c_void_p), ("ev_end", ctypes.c_void_p)]


class KdaError(RuntimeError):
    def __init__(self, code: int, where: str, hip_text: str = ""):
        self.code = code
        msg = f"{where} failed with code {code}: {strerror(code)}"
        if hip_text:
            msg += f" [{hip_text}]"
        super().__init__(msg)


_lib = None


def declared_symbols() -> list[str]:
    """Names of the functions include/kda.h declares (parsed from the header)."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"KDA_API\s+[\w\s\*]+?\b(kda_\w+)\s*\(", text)))


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    vp, f32, i32, sz = ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    fwd_args = [vp, vp, vp, vp, vp, vp, f32, i32, ctypes.POINTER(KdaShape), vp, vp, vp, sz, vp, vp]
    lib.kda_chunk_fwd.argtypes = fwd_args
    lib.kda_chunk_fwd.restype = i32
    lib.kda_chunk_fwd_ex.argtypes = fwd_args + [ctypes.POINTER(KdaOpts)]
    lib.kda_chunk_fwd_ex.restype = i32
    lib.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, f32, i32, ctypes.POINTER(KdaShape), vp, vp, vp, vp]
    lib.kda_chunk_fwd_noalloc.restype = i32
    lib.kda_decode.argtypes = [vp, vp, vp, vp, vp, vp, f32, ctypes.POINTER(KdaShape), vp, vp]
    lib.kda_decode.restype = i32
    lib.kda_chunk_bwd.argtypes = [vp, vp, vp, vp, vp, vp, f32, i32, ctypes.POINTER(KdaShape), vp, vp,
                                  vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kda_chunk_bwd.restype = i32
    lib.kda_bwd_workspace_bytes.argtypes = [ctypes.POINTER(KdaShape), i32]
    lib.kda_bwd_workspace_bytes.restype = sz
    lib.kda_gate_prefix.argtypes = [vp, f32, i32, ctypes.POINTER(KdaShape), vp, vp, vp, vp, vp]
    lib.kda_gate_prefix.restype = i32
    lib.kda_workspace_bytes.argtypes = [ctypes.POINTER(KdaShape), i32]
    lib.kda_workspace_bytes.restype = sz
    lib.kda_workspace_bytes_ex.argtypes = [ctypes.POINTER(KdaShape), i32, ctypes.POINTER(KdaOpts)]
    lib.kda_workspace_bytes_ex.restype = sz
    lib.kda_strerror.argtypes = [i32]
    lib.kda_strerror.restype = ctypes.c_char_p
    lib.kda_last_hip_error.argtypes = []
    lib.kda_last_hip_error.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = i32
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().kda_strerror(int(code)).decode()


def last_hip_error() -> str:
    return load().kda_last_hip_error().decode()


def version() -> int:
    return load().kda_version()


def workspace_bytes(shape: KdaShape, chunk: int = 16, opts: KdaOpts | None = None) -> int:
    n = load().kda_workspace_bytes_ex(ctypes.byref(shape), int(chunk), None if opts is None else ctypes.byref(opts))
    if n == ctypes.c_size_t(-1).value:
        raise KdaError(KDA_ERR_SHAPE, "kda_workspace_bytes_ex")
    return n


def bwd_workspace_bytes(shape: KdaShape, chunk: int = 16) -> int:
    n = load().kda_bwd_workspace_bytes(ctypes.byref(shape), int(chunk))
    if n == ctypes.c_size_t(-1).value:
        raise KdaError(KDA_ERR_SHAPE, "kda_bwd_workspace_bytes")
    return n


class _Hip:
    """Minimal HIP event API through libamdhip64 (timing plumbing only)."""
    _h = None

    @classmethod
    def lib(cls):
        if cls._h is None:
            h = ctypes.CDLL("libamdhip64.so")
            h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            h.hipEventCreate.restype = ctypes.c_int
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            h.hipEventDestroy.restype = ctypes.c_int
            h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            h.hipEventSynchronize.restype = ctypes.c_int
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.restype = ctypes.c_int
            cls._h = h
        return cls._h


class HipEvent:
    """A raw hipEvent_t, recorded by the library around its main kernel."""

    def __init__(self):
        self.handle = ctypes.c_void_p()
        rc = _Hip.lib().hipEventCreate(ctypes.byref(self.handle))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")

    def synchronize(self):
        rc = _Hip.lib().hipEventSynchronize(self.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventSynchronize failed ({rc})")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        rc = _Hip.lib().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        try:
            if self.handle:
                _Hip.lib().hipEventDestroy(self.handle)
        except Exception:
            pass
