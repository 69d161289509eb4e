"""GPU parity over a fixed, seeded list of mixed configurations: batch and head counts, lengths from
1 to 3000 tokens (ragged), automatic and forced segment plans, every gate kind (bounded at -5, -8
and -1, no decay, unbounded) and an initial state or none, on the automatic path (the corrected
plan) and the fused plan, each against the fp64 oracle.  The list is drawn once from a fixed seed,
so every run checks the same cases."""
import numpy as np
import pytest

from chunked_gated_delta_amd import inputs as gen
from kda_testutil import TOL, compare, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _cases(n=24, seed=20261202):
    rng = np.random.default_rng(seed)
    gates = [(-5.0, 0.0, 2.0), (-8.0, 4.0, 1.0), (-1.0, -2.0, 1.0), (0.0, 0.0, 1.0), (-np.inf, 3.0, 3.0)]
    out = []
    for i in range(n):
        g_min, w_mu, w_sd = gates[i % len(gates)]
        out.append(dict(B=int(rng.integers(1, 4)), H=int(rng.integers(1, 7)), T=int(rng.integers(1, 3001)),
                        seg=int(rng.choice([0, 0, 1, 2, 3, 5, 7])), g_min=g_min, w_mu=w_mu, w_sd=w_sd,
                        s0=bool(rng.integers(0, 2)), seed=int(rng.integers(0, 1 << 30))))
    return out


CASES = _cases()


@pytest.mark.parametrize("path", ["auto", "fused"])
@pytest.mark.parametrize("i", range(len(CASES)))
def test_mixed_configuration(i, path):
    c = CASES[i]
    wl = gen.WORKLOADS["bf16_4k"].with_(B=c["B"], H=c["H"], T=c["T"], g_min=c["g_min"], w_mu=c["w_mu"],
                                        w_sd=c["w_sd"], s0_sd=0.3 if c["s0"] else None)
    n = (c["T"] + 31) // 32
    seg = c["seg"] if c["seg"] and (n + c["seg"] - 1) // c["seg"] <= 32 else 0   # at most 32 segments
    eo, es, st, *_ = compare(wl, seed=c["seed"], path=path, seg_steps=seg)
    tol_o, tol_s = TOL["bf16"]
    say(f"   seg_steps={seg} err_o={eo:.3e} err_S={es:.3e} stats={st}")
    assert eo <= tol_o and es <= tol_s
    assert st["n_nonfinite"] == 0
    assert st["n_chunks"] == wl.B * wl.H * ((wl.T + 15) // 16)
