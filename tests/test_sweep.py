"""Chunk-size / g_min co-design sweep on the headline shape (B=1 H=16 T=65536 d=128, w ~ N(0, 2)).

For chunk in {16, 32, 64} and g_min in {-3, -5, -8} the forward runs at that chunk size (16: the
matrix-core path, and the vector path beside it; 32 and 64: the vector path, whose tiles take any
chunk size), each chunk taking the
reciprocal exp(+-G) tiles when its span is at or above -80 and per-pair factors otherwise ("From
Numerical Stability to Load Balancing ..." section 2.3: the tile size is co-designed with the lower
bound; "Architecture Analysis ..." section 5: the bound is to be scanned under the target precision).
For each cell: the flagged fraction and minimum span the forward reports, checked chunk by chunk
against the oracle's fp64 spans of every head (a span within 1e-3 of -80 may fall either way in
fp32); the forward's kernel time after warm-up (HIP events on the launch stream); and its error against
the fp64 oracle on two sampled heads.  Results go to gpurun_out/sweep_gmin_chunk.json."""
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

from chunked_gated_delta_amd import HipEvent, chunk_fwd, decode_stats  # noqa: E402

CHUNKS = [16, 32, 64]
# (chunk, path): the automatic path takes the matrix cores at chunk 16 and the vector kernel at 32 and
# 64; chunk 16 on the vector kernel as well, so that one kernel's time is seen at every chunk size
CASES = [(16, "auto"), (16, "vector"), (32, "auto"), (64, "auto")]
GMINS = [-3.0, -5.0, -8.0]
HEADS = [(0, 0), (0, 11)]   # sampled heads for the error columns


def test_gmin_chunk_sweep():
    wl = gen.WORKLOADS["headline"]
    t = gen.make_torch(wl, seed=0, device="cuda")
    q, k, v, w, beta = (t[n] for n in ("q", "k", "v", "w", "beta"))
    w64 = w.float().cpu().numpy().astype(np.float64)
    heads = {bh: {n: t[n][bh[0]:bh[0] + 1, bh[1]:bh[1] + 1].float().cpu().numpy().astype(np.float64)
                  for n in ("q", "k", "v", "w", "beta")} for bh in HEADS}
    o = torch.empty_like(v)
    S = torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
    rows = []
    for g_min in GMINS:
        ref = {bh: orc.kda_reference(f["q"], f["k"], f["v"], f["w"], f["beta"], None, g_min) for bh, f in heads.items()}
        for chunk, path in CASES:
            fused = chunk == 16 and path == "auto"
            kw = dict(g_min=g_min, chunk=chunk, out=o, S_final=S, path=path)
            for _ in range(20 if fused else 2):
                chunk_fwd(q, k, v, w, beta, None, **kw)
            evs = [(HipEvent(), HipEvent()) for _ in range(20 if fused else 3)]
            for ev in evs:
                _, _, st = chunk_fwd(q, k, v, w, beta, None, events=ev, **kw)
            torch.cuda.synchronize()
            ms = float(np.median([b.elapsed_ms(e) for b, e in evs]))
            d = decode_stats(st)
            spans = orc.chunk_spans(w64, g_min, chunk)
            n_flag = int(np.sum(spans < -80.0))
            n_tie = int(np.sum(np.abs(spans + 80.0) < 1e-3))
            say(f"[case] chunk={chunk} path={path} g_min={g_min}: {ms:.3f} ms, stats {d}, oracle flags {n_flag} (ties {n_tie})")
            assert d["n_chunks"] == wl.B * wl.H * ((wl.T + chunk - 1) // chunk)
            assert abs(d["n_flagged"] - n_flag) <= n_tie
            assert abs(d["min_span"] - float(spans.min())) <= 1e-4 * abs(float(spans.min())) + 1e-3
            assert d["n_nonfinite"] == 0
            errs = [(rel_err(o[b:b + 1, h:h + 1].float().cpu().numpy(), ref[(b, h)][0]),
                     rel_err(S[b:b + 1, h:h + 1].cpu().numpy(), ref[(b, h)][1])) for (b, h) in HEADS]
            eo, es = max(e[0] for e in errs), max(e[1] for e in errs)
            assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1]
            row = {"chunk": chunk, "g_min": g_min, "chunk_times_gmin": chunk * g_min,
                   "path": "matrix cores (bf16 MFMA)" if fused else "vector (fp32)",
                   "flagged_fraction": d["n_flagged"] / d["n_chunks"], "oracle_flagged": n_flag, "ties": n_tie,
                   "min_span": d["min_span"], "forward_ms": ms, "tokens_per_s": wl.B * wl.T / (ms * 1e-3),
                   "err_o": eo, "err_S": es}
            say("   " + json.dumps(row))
            rows.append(row)
    # more tokens per chunk, or a deeper g_min, never flags fewer chunks
    by = {(r["chunk"], r["g_min"]): r["flagged_fraction"] for r in rows}
    for r in rows:   # both kernels flag the same chunks
        assert r["flagged_fraction"] == by[(r["chunk"], r["g_min"])]
    for g_min in GMINS:
        assert by[(16, g_min)] <= by[(32, g_min)] <= by[(64, g_min)]
    for chunk in CHUNKS:
        assert by[(chunk, -3.0)] <= by[(chunk, -5.0)] <= by[(chunk, -8.0)]
    # the pages' rule: a chunk of C tokens never overflows when C * g_min >= -80
    for r in rows:
        if r["chunk_times_gmin"] >= -80.0:
            assert r["flagged_fraction"] == 0.0
    out = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out")
    if os.path.isdir(out):
        with open(os.path.join(out, "sweep_gmin_chunk.json"), "w") as fh:
            json.dump(rows, fh, indent=1)
