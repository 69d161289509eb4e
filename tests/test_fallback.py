"""Unbounded gates: chunks whose span falls below -80 are detected and take the
per-position path; the flagged set is the one the oracle predicts, outputs
match the oracle, turning the fallback off shows the overflow, and forcing it
everywhere still matches."""
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
PATHS = ["vector", "mfma", "fused"]


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
def test_forced_fallback_matches(path, g_min):
    wl = UNB.with_(B=1, H=2, T=300, g_min=g_min, w_mu=0.0 if g_min == -5.0 else 3.0)
    eo, es, st, *_ = compare(wl, seed=1, path=path, force_fallback=True)
    say(f"   err_o={eo:.3e} err_S={es:.3e} stats={st}")
    assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1]
    assert st["n_nonfinite"] == 0


def test_unbounded_f32():
    wl = gen.WORKLOADS["tiny_f32"].with_(H=2, T=160, g_min=-math.inf, w_mu=3.0, w_sd=3.0)
    eo, es, st, *_ = compare(wl, seed=2, path="vector")
    say(f"   err_o={eo:.3e} err_S={es:.3e} stats={st}")
    assert st["n_flagged"] > 0
    assert eo <= TOL["f32"][0] and es <= TOL["f32"][1]
