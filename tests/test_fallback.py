"""Unbounded gates and deep lower bounds: chunks whose span falls below -80 are detected and take
a flagged chunk's handling (on the fused path the tiles referenced to the chunk's token 7 when both
8-token halves span at least -80, per-position factors otherwise); the flagged set is the one the
oracle predicts, outputs match the oracle, turning the fallback off shows the overflow, and forcing
either form everywhere still matches."""
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

UNB = gen.WORKLOADS["unbounded"]
PATHS = ["vector", "fused", "corr"]


@pytest.mark.parametrize("path", PATHS)
def test_unbounded_detects_and_falls_back(path):
    wl = UNB.with_(B=1, H=3, T=640)
    eo, es, st, o, S, o_ref, S_ref = compare(wl, seed=0, path=path)
    w = gen.make_numpy(wl, 0)["w"]
    spans = orc.chunk_spans(w, wl.g_min, 16)
    pred = spans < -80.0
    ties = np.abs(spans + 80.0) <= 1e-3
    say(f"   err_o={eo:.3e} err_S={es:.3e} stats={st} predicted={int(pred.sum())} ties={int(ties.sum())}")
    assert pred.mean() > 0.3
    assert abs(st["n_flagged"] - int(pred.sum())) <= int(ties.sum())
    assert abs(st["min_span"] - spans.min()) <= 1e-4 * abs(spans.min())
    assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1]
    assert st["n_nonfinite"] == 0


@pytest.mark.parametrize("path", PATHS)
def test_disabling_fallback_shows_overflow(path):
    """With the fallback off, a chunk whose span passes ln(max float) = 88.7 makes
    exp(-G) overflow and the outputs turn non-finite (the failure the pages describe)."""
    wl = UNB.with_(B=1, H=2, T=640)
    spans = orc.chunk_spans(gen.make_numpy(wl, 0)["w"], wl.g_min, 16)
    assert spans.min() < -89.0
    _, _, st, o, *_ = compare(wl, seed=0, path=path, disable_fallback=True)
    say(f"   stats={st}")
    assert st["n_nonfinite"] > 0
    assert not np.all(np.isfinite(o))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("g_min", [-5.0, -math.inf])
@pytest.mark.parametrize("force", [1, 2])
def test_forced_fallback_matches(path, g_min, force):
    """force 1: every chunk takes a flagged chunk's handling (on the fused path the tiles referenced to
    the chunk's token 7, or per-pair factors where a half spans below -80); force 2: per-pair factors."""
    wl = UNB.with_(B=1, H=2, T=300, g_min=g_min, w_mu=0.0 if g_min == -5.0 else 3.0)
    eo, es, st, *_ = compare(wl, seed=1, path=path, force_fallback=force)
    say(f"   err_o={eo:.3e} err_S={es:.3e} stats={st}")
    assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1]
    assert st["n_nonfinite"] == 0


@pytest.mark.parametrize("path,seg", [("vector", 0), ("fused", 0), ("fused", 3), ("corr", 0), ("corr", 3)])
def test_nonfinite_count_matches_outputs(path, seg):
    """With the fallback off, the overflowing chunks make outputs non-finite from that chunk on; the
    count the forward reports is exactly the number of non-finite entries of o and S_final it
    returns, on every path and segment plan.  The corrected plan counts in three places: segment 0's
    outputs in its pass, the corrected outputs of the later segments in the correction, and S_final
    in the chaining."""
    wl = UNB.with_(B=1, H=2, T=640)
    kw = dict(disable_fallback=True)
    if seg:
        kw["seg_steps"] = seg   # 7 segments of 3 steps
    _, _, st, o, S, *_ = compare(wl, seed=0, path=path, **kw)
    n = int((~np.isfinite(o)).sum() + (~np.isfinite(S)).sum())
    say(f"   stats={st} non-finite in o and S_final: {n}")
    assert n > 0 and st["n_nonfinite"] == n


def half_spans(w, g_min):
    """Per 16-token chunk, the minimum over channels of the spans of its two 8-token halves (fp64)."""
    g = orc.gate(w, g_min)
    B, H, T, D = g.shape
    n = T // 16
    L = np.cumsum(g[:, :, :16 * n].reshape(B, H, n, 16, D), axis=3)
    return np.minimum(L[:, :, :, 7, :], L[:, :, :, 15, :] - L[:, :, :, 7, :]).min(-1)


@pytest.mark.parametrize("g_min,mix", [(-8.0, False), (-12.0, True), (-20.0, True)])
def test_flagged_chunk_forms(g_min, mix):
    """Lower bounds past 16 x -5: at -8 every flagged chunk's halves stay within -80, so every step takes
    the midpoint-referenced tiles; at -12 a fifth of the chunks have a half past -80, so steps with
    per-pair chunks mix with midpoint steps; at -20 nearly every step takes the per-pair blocks.  Flags
    follow the oracle's spans and the result the oracle."""
    wl = gen.WORKLOADS["bf16_4k"].with_(B=1, H=2, T=1000, g_min=g_min, s0_sd=0.2)
    w = gen.make_numpy(wl, 7)["w"]
    spans = orc.chunk_spans(w, g_min, 16)
    hs = half_spans(w, g_min)
    flagged = spans[:, :, :hs.shape[2]] < -80.0
    per_pair = flagged & (hs < -80.0)
    say(f"   flagged {int(flagged.sum())} of {flagged.size}, halves past -80 {int(per_pair.sum())}")
    assert flagged.mean() > 0.9
    assert per_pair.any() == mix
    eo, es, st, *_ = compare(wl, seed=7, path="fused")
    ties = np.abs(spans + 80.0) <= 1e-3
    say(f"   err_o={eo:.3e} err_S={es:.3e} stats={st}")
    assert abs(st["n_flagged"] - int((spans < -80.0).sum())) <= int(ties.sum())
    assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1]
    assert st["n_nonfinite"] == 0


def test_unbounded_f32():
    wl = gen.WORKLOADS["tiny_f32"].with_(H=2, T=160, g_min=-math.inf, w_mu=3.0, w_sd=3.0)
    eo, es, st, *_ = compare(wl, seed=2, path="vector")
    say(f"   err_o={eo:.3e} err_S={es:.3e} stats={st}")
    assert st["n_flagged"] > 0
    assert eo <= TOL["f32"][0] and es <= TOL["f32"][1]


@pytest.mark.parametrize("path", ["fused", "corr", "vector"])
def test_gates_at_the_bound(path):
    """Every gate at g_min = -5 on some channels (w = 30 there, so sigmoid(w) = 1): those channels' 16-token
    spans are -80 up to the rounding of their sums, the edge the bound promises never to pass.  The
    fused path then runs its kernel without the flagged-chunk forms; the reciprocal factors reach e^80
    and everything stays finite and matches the oracle.  Spans within 1e-3 of -80 count as ties."""
    wl = gen.WORKLOADS["bf16_4k"].with_(B=1, H=2, T=200, s0_sd=0.2)

    def mutate(inp):
        inp["w"][..., ::7] = 30.0   # every seventh channel at the bound (exact in bf16)

    eo, es, st, *_ = compare(wl, seed=11, path=path, mutate=mutate)
    inp = gen.make_numpy(wl, 11)
    mutate(inp)
    spans = orc.chunk_spans(gen.all_to_f64(inp)["w"], wl.g_min, 16)
    ties = np.abs(spans + 80.0) <= 1e-3
    say(f"   err_o={eo:.3e} err_S={es:.3e} stats={st} oracle min span {spans.min():.6f} ties {int(ties.sum())}")
    assert abs(spans.min() + 80.0) < 1e-9          # the oracle's span sits on the bound
    assert abs(st["n_flagged"] - int((spans < -80.0).sum())) <= int(ties.sum())
    assert st["n_nonfinite"] == 0
    assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1]
