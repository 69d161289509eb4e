"""Chunk sizes 32 and 64 (the vector path): the same function as the 16-token chunk form and as the
fp64 token recurrence, whatever the chunk size, with each chunk taking the reciprocal tiles when its
span is at or above -80 and per-pair factors otherwise.  The flagged set is checked against the
oracle's own spans ("From Numerical Stability to Load Balancing ..." section 2.3: the chunk size is
co-designed with the lower bound; 64 x -5 = -320 leaves every chunk of a bounded gate flagged)."""
import math

import numpy as np
import pytest

from chunked_gated_delta_amd import inputs as gen
from oracle import oracle as orc
from kda_testutil import TOL, compare, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

BF16 = gen.WORKLOADS["bf16_4k"]
F32 = gen.WORKLOADS["tiny_f32"]


def check(wl, chunk, seed, **kw):
    eo, es, st, *_ = compare(wl, seed=seed, path="auto", chunk=chunk, **kw)
    tol_o, tol_s = TOL[wl.dtype]
    say(f"   chunk={chunk} err_o={eo:.3e} (tol {tol_o})  err_S={es:.3e} (tol {tol_s})  stats={st}")
    assert eo <= tol_o and es <= tol_s
    assert st["n_nonfinite"] == 0
    assert st["n_chunks"] == wl.B * wl.H * ((wl.T + chunk - 1) // chunk)
    return st


def oracle_flags(wl, seed, chunk):
    """Flagged chunks from the oracle's fp64 spans, and the spans within 1e-3 of -80 (ties that fp32
    may decide either way)."""
    inp = gen.make_numpy(wl, seed)
    spans = orc.chunk_spans(gen.all_to_f64(inp)["w"], wl.g_min, chunk)
    return int(np.sum(spans < -80.0)), int(np.sum(np.abs(spans + 80.0) < 1e-3)), float(np.min(spans))


@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("T", [1, 31, 64, 100, 257])
def test_f32_ragged(chunk, T):
    check(F32.with_(T=T, s0_sd=0.3), chunk, seed=300 + T)


@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("dk,dv", [(32, 64), (128, 128), (64, 32)])
def test_f32_dims(chunk, dk, dv):
    check(F32.with_(T=150, dk=dk, dv=dv), chunk, seed=310 + dk + dv)


@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("g_min", [-1.0, -2.5, -5.0])
def test_bf16_headline_dims(chunk, g_min):
    """d = 128 bf16 inputs at three lower bounds: -1 keeps even 64-token spans above -80 (dense tiles),
    -5 flags every 32- and 64-token chunk (per-pair factors), -2.5 mixes the two at 32 tokens."""
    wl = BF16.with_(B=1, H=2, T=700, g_min=g_min, s0_sd=0.2)
    st = check(wl, chunk, seed=320)
    n_flag, n_tie, mn = oracle_flags(wl, 320, chunk)
    assert abs(st["n_flagged"] - n_flag) <= n_tie, (st, n_flag, n_tie)
    assert math.isclose(st["min_span"], mn, rel_tol=1e-4, abs_tol=1e-3)


@pytest.mark.parametrize("chunk", [32, 64])
def test_unbounded_gate(chunk):
    check(gen.WORKLOADS["unbounded"].with_(B=1, H=2, T=300), chunk, seed=330)


@pytest.mark.parametrize("chunk", [32, 64])
def test_forced_and_disabled_fallback(chunk):
    """Forcing the per-pair factors on every chunk leaves the result; disabling them on a chunk past the
    bound lets its reciprocal factors overflow (the failure the bound exists to prevent)."""
    wl = BF16.with_(B=1, H=1, T=256, g_min=-1.0)
    check(wl, chunk, seed=340, force_fallback=True)
    wl = BF16.with_(B=1, H=1, T=256, g_min=-8.0)
    _, _, st, *_ = compare(wl, seed=341, path="auto", chunk=chunk, disable_fallback=True)
    say(f"   disabled fallback: stats={st}")
    assert st["n_flagged"] > 0 and st["n_nonfinite"] > 0


@pytest.mark.parametrize("chunk", [32, 64])
def test_chunk_sizes_agree(chunk):
    """Chunk 16 (matrix-core path) and chunk 32/64 (vector path) on one input: the same function."""
    from kda_testutil import gpu_run, rel_err
    wl = BF16.with_(B=1, H=2, T=500, g_min=-2.0)
    t = gen.numpy_to_torch(gen.make_numpy(wl, 350), "cuda")
    o16, S16, _ = gpu_run(t, wl.g_min, chunk=16)
    oc, Sc, _ = gpu_run(t, wl.g_min, chunk=chunk)
    assert rel_err(oc.float().cpu().numpy(), o16.float().cpu().numpy()) < 2e-2
    assert rel_err(Sc.cpu().numpy(), S16.cpu().numpy()) < 1e-2
