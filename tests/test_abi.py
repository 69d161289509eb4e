"""The C ABI on the host: the library loads, exports what include/kda.h
declares, and rejects invalid calls with the documented codes before any HIP
call (so these run without a GPU)."""
import ctypes
import math

import pytest

from chunked_gated_delta_amd import _lib
from chunked_gated_delta_amd._lib import KdaShape, KdaOpts

lib = _lib.load()
FAKE = 0x7F0000000000          # an aligned address validation never dereferences
ST = 1 << 40                   # per-tensor stride between fake buffers (no overlaps)


def ptrs(n=10):
    return [ctypes.c_void_p(FAKE + i * ST) for i in range(n)]


def shape(B=1, H=2, T=64, dk=128, dv=128, dtype=1, reserved=0):
    return KdaShape(B, H, T, dk, dv, dtype, reserved)


def call(sh=None, g_min=-5.0, chunk=16, ws_bytes=1 << 30, opts=None, **over):
    p = ptrs()
    args = dict(q=p[0], k=p[1], v=p[2], w=p[3], beta=p[4], S0=None, o=p[5], S_final=p[6],
                workspace=p[7], stats=p[8])
    args.update(over)
    sh = shape() if sh is None else sh
    return lib.kda_chunk_fwd_ex(args["q"], args["k"], args["v"], args["w"], args["beta"], args["S0"],
                                ctypes.c_float(g_min), chunk, ctypes.byref(sh), args["o"], args["S_final"],
                                args["workspace"], ws_bytes, args["stats"], None,
                                ctypes.byref(opts) if opts is not None else None)


def test_exports_every_declared_symbol():
    names = _lib.declared_symbols()
    assert {"kda_chunk_fwd", "kda_chunk_fwd_ex", "kda_workspace_bytes", "kda_strerror",
            "kda_version", "kda_gate_prefix", "kda_last_hip_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strings():
    assert _lib.version() == 110
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert len(_lib.strerror(code)) >= 2
    assert _lib.strerror(-99) == "unknown error code"
    assert isinstance(_lib.last_hip_error(), str)


def test_workspace_bytes():
    assert lib.kda_workspace_bytes(ctypes.byref(shape(dtype=0)), 16) == 0
    n = lib.kda_workspace_bytes(ctypes.byref(shape()), 16)
    assert n < (1 << 40)
    assert lib.kda_workspace_bytes(ctypes.byref(shape()), 24) == ctypes.c_size_t(-1).value
    assert lib.kda_workspace_bytes(ctypes.byref(shape(dk=48)), 16) == ctypes.c_size_t(-1).value
    assert lib.kda_workspace_bytes(None, 16) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("sh,code", [
    (shape(B=0), -2), (shape(H=0), -2), (shape(T=-1), -2), (shape(dk=0), -2), (shape(dv=-3), -2),
    (shape(dk=48), -3), (shape(dv=256), -3), (shape(dtype=7), -3), (shape(reserved=1), -4),
    (shape(B=1 << 30, H=1 << 30, T=1 << 30), -2)])
def test_shape_errors(sh, code):
    assert call(sh) == code


def test_null_shape():
    p = ptrs()
    assert lib.kda_chunk_fwd(p[0], p[1], p[2], p[3], p[4], None, ctypes.c_float(-5.0), 16, None,
                             p[5], p[6], p[7], 0, None, None) == -1


@pytest.mark.parametrize("name", ["q", "k", "v", "w", "beta", "o", "S_final"])
def test_null_pointers(name):
    assert call(**{name: None}) == -1


def test_null_inputs_allowed_when_empty():
    # T = 0 needs only S_final; this reaches the launch, so only check the NULL rule on S_final here
    assert call(shape(T=0), S_final=None, q=None, k=None, v=None, w=None, beta=None, o=None) == -1


@pytest.mark.parametrize("chunk", [0, 8, 15, 17, 48, 128])
def test_chunk_sizes(chunk):
    """16, 32 or 64 tokens per chunk; anything else is unsupported."""
    assert call(chunk=chunk) == -3


def test_chunk_32_64_only_on_the_vector_path():
    """32- and 64-token chunks run on the vector path (no workspace); the matrix-core paths take 16."""
    for chunk in (32, 64):
        assert lib.kda_workspace_bytes(ctypes.byref(shape(T=4096)), chunk) == 0
        for path in (3, 4):
            assert call(chunk=chunk, opts=KdaOpts(0, 0, path, 0, None, None)) == -3
            assert lib.kda_workspace_bytes_ex(ctypes.byref(shape()), chunk,
                                              ctypes.byref(KdaOpts(0, 0, path, 0, None, None))) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("g_min", [float("nan"), 0.5, 1e-30, float("inf")])
def test_bad_g_min(g_min):
    assert call(g_min=g_min) == -4


def test_misaligned_pointer():
    p = ptrs()
    assert call(q=ctypes.c_void_p(p[0].value + 2)) == -4
    assert call(S_final=ctypes.c_void_p(p[6].value + 8)) == -4


def test_overlaps_rejected():
    p = ptrs()
    assert call(o=p[0]) == -4                                   # output aliases q
    assert call(S_final=ctypes.c_void_p(p[2].value + 1024)) == -4   # S_final inside v
    assert call(workspace=p[5]) == -4                            # workspace aliases o
    assert call(stats=p[6]) == -4                                # stats aliases S_final
    assert call(S0=ctypes.c_void_p(p[6].value + 16)) == -4       # S0 partly overlaps S_final


def test_workspace_per_path():
    ex = lambda sh, path, seg=0: lib.kda_workspace_bytes_ex(ctypes.byref(sh), 16,
                                                            ctypes.byref(KdaOpts(0, 0, path, seg, None, None)))
    blk = 128 * 128 * 4                         # one X, M or S_start block (64 KiB)
    for path in (0, 1, 3, 4):                   # an empty sequence keeps nothing on any path
        assert ex(shape(T=0), path) == 0
    sh = shape(B=1, H=2, T=64)                  # 2 steps of 32 tokens per (b, h): one segment
    assert lib.kda_workspace_bytes(ctypes.byref(sh), 16) == 0        # automatic: fused, nothing kept
    assert ex(sh, 3) == 0
    assert ex(sh, 1) == 0
    for path in (2, 5, 7):                      # no such path (2 was the per-step records path)
        assert ex(sh, path) == ex(shape(T=0), path) == ctypes.c_size_t(-1).value
    # 128 steps per head, two heads: at most 16 segments of 8 steps; segment 0, which runs with its
    # outputs beside the maps, is 0.93x the others, so the plan is 8 steps, then 9-step segments (the
    # last takes the remaining 3): 15 segments
    sh = shape(B=1, H=2, T=4096)
    assert ex(sh, 3) == 3 * 2 * 15 * blk
    assert ex(sh, 3, seg=5) == 3 * 2 * 26 * blk                      # a forced length of 5 steps: 26 segments
    assert ex(sh, 3, seg=3) == ctypes.c_size_t(-1).value             # 43 segments: more than 32
    assert ex(shape(dk=64, dv=64), 3) == ctypes.c_size_t(-1).value   # no matrix-core path at d = 64
    assert ex(shape(dk=64, dv=64), 0) == 0
    # the fused kernels' views hold one segment of fewer than 2^18 steps: two heads of 2^23 tokens take
    # 32 segments of 8192 steps; 256 heads would keep one segment per sequence, 2^18 steps, so their
    # plan takes two (a segment 0 of 1.1x the other's length on the corrected plan, 0.93x on the fused
    # one), one step fewer keeps one segment (the corrected plan then keeps nothing)
    big_t = shape(T=1 << 23)
    assert ex(big_t, 0) == ex(big_t, 4) == 3 * 2 * 32 * blk + 2 * (1 << 18) * 8192
    wide = shape(B=1, H=256, T=1 << 23)
    assert ex(wide, 0) == ex(wide, 4) == 3 * 256 * 2 * blk + 256 * (1 << 18) * 8192
    assert ex(wide, 3) == 3 * 256 * 2 * blk
    assert ex(shape(B=1, H=256, T=(1 << 23) - 32), 0) == 0
    # a forced segment of 2^18 steps is refused; one step shorter gives two segments
    assert ex(big_t, 4, seg=1 << 18) == ex(big_t, 0, seg=1 << 18) == ctypes.c_size_t(-1).value
    assert ex(big_t, 4, seg=(1 << 18) - 1) == 3 * 2 * 2 * blk + 2 * (1 << 18) * 8192
    assert call(big_t, opts=KdaOpts(0, 0, 0, 1 << 18, None, None)) == -4
    assert call(sh, opts=KdaOpts(0, 0, 2, 0, None, None)) == -3
    # corrected plan: at most 16 segments of 8 steps (one pass holds every segment), its maps and
    # entering states, and the propagated queries of every step (8 KiB each)
    assert ex(shape(B=1, H=2, T=64), 4) == 0                          # one segment: nothing kept
    assert ex(sh, 4) == 3 * 2 * 16 * blk + 2 * 128 * 8192
    # automatic plan: the corrected one
    assert ex(sh, 0) == lib.kda_workspace_bytes(ctypes.byref(sh), 16) == ex(sh, 4) > ex(sh, 3)
    assert ex(sh, 4, seg=5) == 3 * 2 * 26 * blk + 2 * 128 * 8192
    assert ex(sh, 4, seg=3) == ctypes.c_size_t(-1).value
    assert ex(shape(dk=64, dv=64), 4) == ctypes.c_size_t(-1).value
    assert call(sh, ws_bytes=ex(sh, 3), opts=KdaOpts(0, 0, 4, 0, None, None)) == -4


def test_workspace_too_small():
    sh = shape(T=4096)                          # several segments per head: the fused path keeps its maps
    need = lib.kda_workspace_bytes(ctypes.byref(sh), 16)
    assert need > 0
    assert call(sh, ws_bytes=need - 1) == -4
    assert call(sh, workspace=None, ws_bytes=0) == -4


def test_opts_validation():
    assert call(opts=KdaOpts(1, 1, 0, 0, None, None)) == -4     # both knobs
    assert call(opts=KdaOpts(0, 3, 0, 0, None, None)) == -4     # force_fallback takes 0, 1 or 2
    assert call(opts=KdaOpts(0, -1, 0, 0, None, None)) == -4
    assert call(opts=KdaOpts(0, 0, 0, -1, None, None)) == -4    # negative segment length
    # a forced segment length giving more than 32 segments per sequence (33 steps of 32 tokens)
    assert call(sh=shape(T=33 * 32), opts=KdaOpts(0, 0, 0, 1, None, None)) == -4
    assert call(opts=KdaOpts(0, 0, 7, 0, None, None)) == -3     # unknown path


def decode_call(sh=None, g_min=-5.0, **over):
    p = ptrs()
    a = dict(q=p[0], k=p[1], v=p[2], w=p[3], beta=p[4], S=p[5], o=p[6])
    a.update(over)
    sh = shape() if sh is None else sh
    return lib.kda_decode(a["q"], a["k"], a["v"], a["w"], a["beta"], a["S"], ctypes.c_float(g_min),
                          ctypes.byref(sh), a["o"], None)


def test_decode_validation():
    assert decode_call(shape(B=0)) == -2
    assert decode_call(shape(dk=48)) == -3
    assert decode_call(g_min=float("nan")) == -4
    assert decode_call(S=None) == -1
    for name in ("q", "k", "v", "w", "beta", "o"):
        assert decode_call(**{name: None}) == -1, name
    p = ptrs()
    assert decode_call(S=ctypes.c_void_p(p[5].value + 4)) == -4        # misaligned state
    assert decode_call(o=ctypes.c_void_p(p[5].value + 1024)) == -4     # output inside the state
    assert decode_call(S=p[0]) == -4                                    # state aliases q
    # T = 0: nothing to do, no launch (so this runs without a GPU); only the state is required
    assert decode_call(shape(T=0), q=None, k=None, v=None, w=None, beta=None, o=None) == 0


def test_gate_prefix_validation():
    p = ptrs()
    sh = shape()
    f = lambda **kw: lib.kda_gate_prefix(kw.get("w", p[0]), ctypes.c_float(kw.get("g_min", -5.0)),
                                         kw.get("chunk", 16), ctypes.byref(kw.get("sh", sh)),
                                         kw.get("g", p[1]), kw.get("G", p[2]), kw.get("span", p[3]),
                                         kw.get("flags", p[4]), None)
    assert f(chunk=8) == -3
    assert f(chunk=48) == -3
    assert f(g_min=float("nan")) == -4
    assert f(w=None) == -1
    assert f(g=p[0]) == -4
    assert f(sh=shape(dk=100)) == -3


def bwd_call(sh=None, g_min=-5.0, chunk=16, ws_bytes=1 << 40, **over):
    p = ptrs(16)
    a = dict(q=p[0], k=p[1], v=p[2], w=p[3], beta=p[4], S0=None, dO=p[5], dSf=None, dq=p[6], dk=p[7],
             dv=p[8], dw=p[9], dbeta=p[10], dS0=p[11], workspace=p[12])
    a.update(over)
    sh = shape() if sh is None else sh
    return lib.kda_chunk_bwd(a["q"], a["k"], a["v"], a["w"], a["beta"], a["S0"], ctypes.c_float(g_min), chunk,
                             ctypes.byref(sh), a["dO"], a["dSf"], a["dq"], a["dk"], a["dv"], a["dw"], a["dbeta"],
                             a["dS0"], a["workspace"], ws_bytes, None)


def test_bwd_workspace_bytes():
    sh = shape(B=2, H=3, T=33, dk=64, dv=32)
    rec = 3 * 16 * 64 + 2 * 16 * 32 + 64                # per chunk: W, Ktil, Qbar, U0, P^T dO, e^Gam
    assert lib.kda_bwd_workspace_bytes(ctypes.byref(sh), 16) == 2 * 3 * 3 * (rec + 2 * 64 * 32) * 4
    assert lib.kda_bwd_workspace_bytes(ctypes.byref(sh), 32) == ctypes.c_size_t(-1).value
    assert lib.kda_bwd_workspace_bytes(ctypes.byref(shape(dv=48)), 16) == ctypes.c_size_t(-1).value
    assert lib.kda_bwd_workspace_bytes(None, 16) == ctypes.c_size_t(-1).value


def test_bwd_validation():
    assert bwd_call(shape(B=0)) == -2
    assert bwd_call(shape(dk=48)) == -3
    assert bwd_call(chunk=32) == -3
    assert bwd_call(g_min=float("nan")) == -4
    assert bwd_call(g_min=1.0) == -4
    for name in ("q", "k", "v", "w", "beta", "dO", "dq", "dk", "dv", "dw", "dbeta"):
        assert bwd_call(**{name: None}) == -1, name
    p = ptrs(16)
    assert bwd_call(ws_bytes=16) == -4                                      # workspace too small
    assert bwd_call(workspace=None) == -4
    assert bwd_call(dq=ctypes.c_void_p(p[6].value + 4)) == -4               # misaligned output
    assert bwd_call(dk=p[6]) == -4                                          # two outputs alias
    assert bwd_call(dv=p[5]) == -4                                          # output aliases dO
    assert bwd_call(dS0=p[0]) == -4                                         # output aliases q
    # T = 0 with no dS0 wanted: nothing to do, no launch, no pointers needed
    assert bwd_call(shape(T=0), q=None, k=None, v=None, w=None, beta=None, dO=None, dq=None, dk=None, dv=None,
                    dw=None, dbeta=None, dS0=None, workspace=None, ws_bytes=0) == 0


def test_noalloc_rejects_calls_beyond_its_scratch():
    """kda_chunk_fwd_noalloc refuses, before any HIP call, a call whose automatic plan needs more than
    the static array holds, and validates everything else as kda_chunk_fwd does."""
    assert _lib.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert "#define KDA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)" in open(_lib.HEADER).read()
    p = ptrs()
    big = shape(B=1, H=128, T=65536)            # 128 heads x 3 segments x 192 KiB = 72 MiB
    assert lib.kda_workspace_bytes(ctypes.byref(big), 16) > _lib.NOALLOC_SCRATCH_BYTES
    na = lambda sh, g_min=-5.0, chunk=16, S_final=p[6]: lib.kda_chunk_fwd_noalloc(
        p[0], p[1], p[2], p[3], p[4], None, ctypes.c_float(g_min), chunk, ctypes.byref(sh), p[5], S_final,
        p[8], None)
    assert na(big) == _lib.KDA_ERR_SCRATCH == -6
    assert na(shape(), chunk=48) == -3
    assert na(shape(dk=48)) == -3
    assert na(shape(), g_min=1.0) == -4
    assert na(shape(), S_final=None) == -1
    # the entry point takes the fused plan where the automatic one is the corrected plan: the headline
    # shape fits the array with the former (52 MiB), not with the latter (its 8 KiB per step of queries)
    headline = shape(B=1, H=16, T=65536)
    fused = lambda sh: lib.kda_workspace_bytes_ex(ctypes.byref(sh), 16, ctypes.byref(KdaOpts(0, 0, 3, 0, None, None)))
    assert 0 < fused(headline) <= _lib.NOALLOC_SCRATCH_BYTES < lib.kda_workspace_bytes(ctypes.byref(headline), 16)
    assert fused(big) > _lib.NOALLOC_SCRATCH_BYTES
    # every head count up to 113 fits at any length (the plan holds at most 256 + B*H segment triples),
    # 114 does not, and from 129 heads on the plan has one segment per sequence and keeps nothing
    for H in (1, 16, 32, 85, 100, 113):
        for T in (65536, 1 << 20):
            assert fused(shape(B=1, H=H, T=T)) <= _lib.NOALLOC_SCRATCH_BYTES, (H, T)
    assert fused(shape(B=1, H=114, T=65536)) > _lib.NOALLOC_SCRATCH_BYTES
    assert fused(shape(B=1, H=129, T=65536)) == fused(shape(B=3, H=100, T=1 << 20)) == 0
