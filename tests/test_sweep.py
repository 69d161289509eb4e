"""Chunk-size / g_min co-design sweep on the headline shape (B=1 H=16 T=65536 d=128, w ~ N(0, 2)).

For chunk in {16, 32, 64} and g_min in {-3, -5, -8}: the fraction of chunks whose span falls below
-80 (whose reciprocal factor e^{-G} could pass e^{80} and which must take the per-pair blocks) and
the minimum span, from the GPU gate/prefix stage and pinned to the oracle's spans; and, for the
16-token chunks the forward evaluates, the forward's time and its error against the oracle on
sampled heads.  The pages' rule is that chunk * |g_min| <= 80 keeps every chunk dense; the sweep
checks that the measured flags follow it.  Results go to gpurun_out/sweep_gmin_chunk.json."""
import json
import os

import numpy as np
import pytest

from chunked_gated_delta_amd import inputs as gen
from oracle import oracle as orc
from kda_testutil import TOL, rel_err, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from chunked_gated_delta_amd import chunk_fwd, decode_stats, gate_prefix  # noqa: E402

CHUNKS = [16, 32, 64]
GMINS = [-3.0, -5.0, -8.0]
HEADS = [(0, 0), (0, 11)]   # sampled heads for the error column


def test_gmin_chunk_sweep():
    wl = gen.WORKLOADS["headline"]
    t = gen.make_torch(wl, seed=0, device="cuda")
    w64_heads = {bh: t["w"][bh[0]:bh[0] + 1, bh[1]:bh[1] + 1].float().cpu().numpy().astype(np.float64) for bh in HEADS}
    rows = []
    for g_min in GMINS:
        for chunk in CHUNKS:
            _, _, span, flags = gate_prefix(t["w"], g_min, chunk=chunk)
            torch.cuda.synchronize()
            sp = span.cpu().numpy()
            frac = float(flags.cpu().numpy().mean())
            # pin: the sampled heads' spans match the oracle's
            for (b, h), w64 in w64_heads.items():
                ref = orc.chunk_spans(w64, g_min, chunk)[0, 0]
                assert np.max(np.abs(sp[b, h] - ref)) <= 2e-5 * max(1.0, np.max(np.abs(ref)))
            row = {"chunk": chunk, "g_min": g_min, "flagged_fraction": frac, "min_span": float(sp.min()),
                   "chunk_times_gmin": chunk * g_min}
            if chunk * g_min >= -80.0:
                assert frac == 0.0 and sp.min() >= -80.0 - 1e-3   # the pages' rule: nothing to flag
            if chunk == 16:
                o, S, st = chunk_fwd(t["q"], t["k"], t["v"], t["w"], t["beta"], None, g_min=g_min)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(3):
                    chunk_fwd(t["q"], t["k"], t["v"], t["w"], t["beta"], None, g_min=g_min, out=o, S_final=S)
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / 3
                d = decode_stats(st)
                assert d["n_flagged"] == int(flags.cpu().numpy().sum()) or abs(d["n_flagged"] - flags.sum().item()) <= 2
                errs = []
                for (b, h) in HEADS:
                    f = {n: t[n][b:b + 1, h:h + 1].float().cpu().numpy().astype(np.float64)
                         for n in ("q", "k", "v", "w", "beta")}
                    o_ref, S_ref = orc.kda_reference(f["q"], f["k"], f["v"], f["w"], f["beta"], None, g_min)
                    errs.append((rel_err(o[b:b + 1, h:h + 1].float().cpu().numpy(), o_ref),
                                 rel_err(S[b:b + 1, h:h + 1].cpu().numpy(), S_ref)))
                eo, es = max(e[0] for e in errs), max(e[1] for e in errs)
                assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1] and d["n_nonfinite"] == 0
                row.update({"forward_ms": ms, "tokens_per_s": wl.B * wl.T / (ms * 1e-3), "err_o": eo, "err_S": es,
                            "n_flagged_forward": d["n_flagged"]})
            say("   " + json.dumps(row))
            rows.append(row)
    # more tokens per chunk, or a deeper g_min, never flags fewer chunks
    by = {(r["chunk"], r["g_min"]): r["flagged_fraction"] for r in rows}
    for g_min in GMINS:
        assert by[(16, g_min)] <= by[(32, g_min)] <= by[(64, g_min)]
    for chunk in CHUNKS:
        assert by[(chunk, -3.0)] <= by[(chunk, -5.0)] <= by[(chunk, -8.0)]
    out = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out")
    if os.path.isdir(out):
        with open(os.path.join(out, "sweep_gmin_chunk.json"), "w") as fh:
            json.dump(rows, fh, indent=1)
