"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, element by element, at sizes the oracle finishes in
seconds, spanning several chunks and ragged tails."""
import math

import numpy as np
import pytest

from chunked_gated_delta_amd import inputs as gen
from oracle import oracle as orc
from kda_testutil import TOL, compare, rel_err, say, gpu_run, need_path

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

BF16 = gen.WORKLOADS["bf16_4k"]
PATHS = ["vector", "fused", "corr"]


def mfma_ok(wl):
    return wl.dtype == "bf16" and wl.dk == 128 and wl.dv == 128


def paths_for(wl):
    return [p for p in PATHS if p == "vector" or mfma_ok(wl)]


def check(wl, path, seed=0, **kw):
    if path in ("fused", "corr") and not mfma_ok(wl):
        pytest.skip("matrix-core path covers bf16 with dk = dv = 128")
    eo, es, st, *_ = compare(wl, seed=seed, path=path, **kw)
    tol_o, tol_s = TOL[wl.dtype]
    say(f"   err_o={eo:.3e} (tol {tol_o})  err_S={es:.3e} (tol {tol_s})  stats={st}")
    assert eo <= tol_o and es <= tol_s
    assert st["n_nonfinite"] == 0
    assert st["n_chunks"] == wl.B * wl.H * ((wl.T + 15) // 16)
    return st


def test_tiny_f32_workload():
    """The fp32 workload in full: B1 H1 T64 d32, max relative error <= 1e-5."""
    check(gen.WORKLOADS["tiny_f32"], "vector")


@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 100])
def test_f32_ragged_lengths(T):
    check(gen.WORKLOADS["tiny_f32"].with_(T=T, H=2), "vector", seed=T)


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 32), (32, 128), (128, 64), (64, 64)])
def test_f32_dims(dk, dv):
    check(gen.WORKLOADS["tiny_f32"].with_(T=80, dk=dk, dv=dv), "vector", seed=dk + dv)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T", [1, 15, 16, 17, 31, 32, 33, 63, 300])
def test_bf16_ragged_lengths(path, T):
    check(BF16.with_(B=1, H=3, T=T), path, seed=100 + T)


@pytest.mark.parametrize("path", PATHS)
def test_bf16_several_heads_batches(path):
    check(BF16.with_(B=2, H=3, T=520), path, seed=7)


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 32), (32, 64)])
def test_bf16_other_dims(dk, dv):
    check(BF16.with_(B=1, H=2, T=200, dk=dk, dv=dv), "vector", seed=dk * dv)


@pytest.mark.parametrize("path", PATHS)
def test_bf16_initial_state_and_decay_stress(path):
    """Decay-stress distributions (w ~ N(6,1): spans near -80) with S0 ~ N(0, 0.1)."""
    st = check(gen.WORKLOADS["decay_stress"].with_(H=2, T=1024), path, seed=3)
    assert st["n_flagged"] == 0 and -80.0 <= st["min_span"] < -79.0


@pytest.mark.parametrize("path", PATHS)
def test_beta_zero_is_pure_decay(path):
    """beta = 0: no writes, the state only decays.  Slow decay (w ~ N(-3, 1)) keeps the
    true state inside fp32's range over the whole sequence, so the relative metric is meaningful."""
    wl = BF16.with_(B=1, H=2, T=96, s0_sd=0.5, w_mu=-3.0, w_sd=1.0)
    check(wl, path, seed=5, mutate=lambda inp: inp["beta"].fill(0.0))


@pytest.mark.parametrize("path", PATHS)
def test_beta_one_retrieval(path):
    """beta = 1 and q = k: each read returns the value just written."""
    wl = BF16.with_(B=1, H=2, T=130)

    def mut(inp):
        inp["beta"].fill(1.0)
        inp["q"][...] = inp["k"]
    eo, es, st, o, S, o_ref, S_ref = compare(wl, seed=9, path=path, mutate=mut)
    assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1]
    v = gen.make_numpy(wl, 9)["v"].astype(np.float64)
    assert rel_err(o, v) < 2e-2


@pytest.mark.parametrize("path", PATHS)
def test_zero_gate_no_decay(path):
    """g_min = 0: no forgetting at all (a degenerate gate)."""
    check(BF16.with_(B=1, H=2, T=64, g_min=0.0), path, seed=4)


@pytest.mark.parametrize("path", PATHS)
def test_bounded_gate_other_gmin(path):
    """g_min = -8: spans may pass -80 and those chunks take the per-position path."""
    wl = BF16.with_(B=1, H=2, T=512, g_min=-8.0, w_mu=4.0, w_sd=1.0)
    st = check(wl, path, seed=12)
    pred = orc.predicted_flags(gen.make_numpy(wl, 12)["w"], -8.0)
    assert st["n_flagged"] == int(pred.sum()) and st["n_flagged"] > 0


def test_empty_sequence():
    from chunked_gated_delta_amd import chunk_fwd, decode_stats
    dev = "cuda"
    z = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=dev)
    b = torch.empty((1, 2, 0), dtype=torch.bfloat16, device=dev)
    S0 = torch.randn((1, 2, 128, 128), device=dev)
    o, S, st = chunk_fwd(z, z, z, z, b, S0)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 128) and torch.equal(S, S0)
    d = decode_stats(st)
    assert d["n_chunks"] == 0 and math.isinf(d["min_span"])
    o, S, _ = chunk_fwd(z, z, z, z, b, None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S).item() == 0


# ---------------------------------------------------------------- stage: gate and in-chunk prefix

@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("g_min,mu,sd", [(-5.0, 0.0, 2.0), (-5.0, 6.0, 1.0), (-math.inf, 3.0, 3.0), (-3.0, 0.0, 2.0)])
def test_gate_prefix_stage(g_min, mu, sd, chunk):
    from chunked_gated_delta_amd import gate_prefix
    wl = BF16.with_(B=1, H=2, T=333, w_mu=mu, w_sd=sd, g_min=g_min)
    inp = gen.make_numpy(wl, 21)
    say(f"[case] gate_prefix {wl} chunk={chunk}")
    w_t = gen.numpy_to_torch(inp, "cuda")["w"]
    g, G, span, flags = gate_prefix(w_t, g_min, chunk=chunk)
    torch.cuda.synchronize()
    w64 = inp["w"].astype(np.float64)
    g_ref = orc.gate(w64, g_min)
    assert np.max(np.abs(g.cpu().numpy() - g_ref)) <= 2e-6 * max(1.0, np.max(np.abs(g_ref)))
    T = wl.T
    G_ref = np.empty_like(g_ref)
    for n in range(0, T, chunk):
        G_ref[:, :, n:n + chunk] = np.cumsum(g_ref[:, :, n:n + chunk], axis=2)
    assert np.max(np.abs(G.cpu().numpy() - G_ref)) <= 2e-5 * max(1.0, np.max(np.abs(G_ref)))
    sp_ref = orc.chunk_spans(w64, g_min, chunk)
    assert np.max(np.abs(span.cpu().numpy() - sp_ref)) <= 2e-5 * max(1.0, np.max(np.abs(sp_ref)))
    fl = flags.cpu().numpy().astype(bool)
    pred = sp_ref < -80.0
    decided = np.abs(sp_ref + 80.0) > 1e-3        # ties within 1e-3 of -80 may go either way
    assert np.array_equal(fl[decided], pred[decided])


# ---------------------------------------------------------------- state carry, determinism, in-place

@pytest.mark.parametrize("path", PATHS)
def test_chaining_is_bitwise(path):
    from chunked_gated_delta_amd import chunk_fwd
    need_path(path)
    wl = BF16.with_(B=1, H=2, T=400, s0_sd=0.2)
    t = gen.numpy_to_torch(gen.make_numpy(wl, 33), "cuda")
    say(f"[case] chaining {wl} path={path}")
    o, S, _ = chunk_fwd(t["q"], t["k"], t["v"], t["w"], t["beta"], t["S0"], path=path)
    T1 = 192
    sl = lambda x, a, b: x[:, :, a:b].contiguous()
    o1, S1, _ = chunk_fwd(*(sl(t[n], 0, T1) for n in ("q", "k", "v", "w", "beta")), t["S0"], path=path)
    o2, S2, _ = chunk_fwd(*(sl(t[n], T1, wl.T) for n in ("q", "k", "v", "w", "beta")), S1, path=path)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], dim=2), o)
    assert torch.equal(S2, S)


@pytest.mark.parametrize("path", PATHS)
def test_deterministic_and_in_place_state(path):
    from chunked_gated_delta_amd import chunk_fwd
    need_path(path)
    wl = BF16.with_(B=1, H=2, T=150, s0_sd=0.2)
    t = gen.numpy_to_torch(gen.make_numpy(wl, 44), "cuda")
    say(f"[case] determinism {wl} path={path}")
    args = [t[n] for n in ("q", "k", "v", "w", "beta")]
    oa, Sa, _ = chunk_fwd(*args, t["S0"], path=path)
    ob, Sb, _ = chunk_fwd(*args, t["S0"], path=path)
    state = t["S0"].clone()
    oc, Sc, _ = chunk_fwd(*args, state, S_final=state, path=path)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(Sa, Sb)
    assert torch.equal(oa, oc) and torch.equal(Sa, state)


# ---------------------------------------------------------------- vector vs matrix-core agreement

def test_paths_agree():
    wl = BF16.with_(B=1, H=2, T=700)
    need_path("corr")
    inp = gen.make_numpy(wl, 55)
    t = gen.numpy_to_torch(inp, "cuda")
    say(f"[case] path agreement {wl}")
    ov, Sv, _ = gpu_run(t, wl.g_min, path="vector")
    om, Sm, _ = gpu_run(t, wl.g_min, path="corr")
    assert rel_err(om.float().cpu().numpy(), ov.float().cpu().numpy()) < 2e-2
    assert rel_err(Sm.cpu().numpy(), Sv.cpu().numpy()) < 1e-2
