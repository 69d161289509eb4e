"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import math
import sys

import numpy as np

from chunked_gated_delta_amd import inputs as gen
from oracle import oracle as orc

# Acceptance: max |x - ref| / max |ref| per output tensor.
#   fp32 workloads: 1e-5 on o and S_final;
#   bf16 inputs with fp32 accumulation and state: 2e-2 on o, 1e-2 on S_final.
TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-2)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    num = np.max(np.abs(x - ref))
    if not np.isfinite(num):
        return math.inf
    return float(num / den) if den > 0 else float(num)


def gpu_run(inp_t, g_min, **kw):
    import torch
    from chunked_gated_delta_amd import chunk_fwd
    o, S, st = chunk_fwd(inp_t["q"], inp_t["k"], inp_t["v"], inp_t["w"], inp_t["beta"], inp_t["S0"],
                         g_min=g_min, **kw)
    torch.cuda.synchronize()
    return o, S, st


def oracle_run(inp_np, g_min, nthreads=8):
    f = gen.all_to_f64(inp_np)
    return orc.kda_reference(f["q"], f["k"], f["v"], f["w"], f["beta"], f["S0"], g_min, nthreads=nthreads)


def compare(wl, seed=0, path="auto", mutate=None, **kw):
    """numpy-seeded inputs for workload wl -> (err_o, err_S, stats, o, S, o_ref, S_ref)."""
    import torch
    from chunked_gated_delta_amd import decode_stats
    inp = gen.make_numpy(wl, seed)
    if mutate:
        mutate(inp)
    say(f"[case] {wl} seed={seed} path={path} kw={kw}")
    t = gen.numpy_to_torch(inp, "cuda")
    try:
        o, S, st = gpu_run(t, wl.g_min, path=path, **kw)
    except Exception as e:  # the requested path does not take this configuration
        from chunked_gated_delta_amd import KdaError
        if isinstance(e, KdaError) and e.code == -3 and path != "auto":
            import pytest
            pytest.skip(f"path {path} does not support {wl}")
        raise
    o_ref, S_ref = oracle_run(inp, wl.g_min)
    o_np = o.float().cpu().numpy()
    S_np = S.cpu().numpy()
    stats = decode_stats(st) if st is not None else None
    return rel_err(o_np, o_ref), rel_err(S_np, S_ref), stats, o_np, S_np, o_ref, S_ref


_MFMA = None


def mfma_available() -> bool:
    """Whether the library's matrix-core path takes bf16, dk = dv = 128."""
    global _MFMA
    if _MFMA is None:
        import torch
        from chunked_gated_delta_amd import KdaError, chunk_fwd
        x = torch.zeros((1, 1, 16, 128), dtype=torch.bfloat16, device="cuda")
        b = torch.zeros((1, 1, 16), dtype=torch.bfloat16, device="cuda")
        try:
            chunk_fwd(x, x, x, x, b, path="corr")
            torch.cuda.synchronize()
            _MFMA = True
        except KdaError as e:
            if e.code != -3:
                raise
            _MFMA = False
    return _MFMA


def need_path(path):
    import pytest
    if path in ("fused", "corr") and not mfma_available():
        pytest.skip("the loaded library has no matrix-core path")
