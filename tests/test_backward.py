"""Backward of the chunked forward (kda_chunk_bwd): gradients of <dO, o> + <dS_final, S_final> with
respect to q, k, v, w, beta and S0, against the fp64 oracle's adjoint of the token recurrence
(itself pinned to central finite differences in test_oracle.py).

Tolerance: the kernel computes in fp32 from the same (dtype-rounded) inputs and cotangents that
the oracle gets exactly, for bf16 and fp32 workloads alike, so the only error is fp32 rounding:
dot products of at most 128 terms (worst case about 128 * 6e-8 = 8e-6 relative to the sum of
magnitudes, typically a few 1e-7 for these zero-mean terms), then the reverse chain of chunk
states, which the decay factors (all <= 1) keep from growing.  Measured errors sit near 1e-6 up to
4000 tokens and on the 65536-token shape; the tests hold every gradient to BWD_TOL = 2e-5 of its
largest entry, the worst-case dot-product bound with a factor of two for the chain."""
import numpy as np
import pytest

from chunked_gated_delta_amd import inputs as gen
from kda_testutil import rel_err, say
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from chunked_gated_delta_amd import chunk_bwd  # noqa: E402

BWD_TOL = 2e-5
NAMES = ("dq", "dk", "dv", "dw", "dbeta", "dS0")


def run_case(wl, seed, with_dSf=True, want_dS0=True):
    inp = gen.make_numpy(wl, seed)
    cot = gen.make_cotangents(wl, seed, with_dSf=with_dSf)
    say(f"[case] bwd {wl} seed={seed} dSf={with_dSf} dS0={want_dS0}")
    t = gen.numpy_to_torch(inp, "cuda")
    td = gen.torch_dtype(wl.dtype)
    dO = torch.from_numpy(cot["dO"]).to("cuda", td).contiguous()
    dSf = None if cot["dSf"] is None else torch.from_numpy(cot["dSf"]).cuda().contiguous()
    got = chunk_bwd(t["q"], t["k"], t["v"], t["w"], t["beta"], dO, S0=t["S0"], dS_final=dSf,
                    g_min=wl.g_min, want_dS0=want_dS0)
    torch.cuda.synchronize()
    got = [None if x is None else x.cpu().numpy() for x in got]
    f = gen.all_to_f64(inp)
    ref = orc.kda_backward(f["q"], f["k"], f["v"], f["w"], f["beta"], f["S0"], wl.g_min,
                           cot["dO"].astype(np.float64),
                           None if cot["dSf"] is None else cot["dSf"].astype(np.float64), nthreads=8)
    return got, ref


def check(wl, seed, tol=None, **kw):
    tol = dict(tol or {})
    got, ref = run_case(wl, seed, **kw)
    errs = {}
    for name, g, r in zip(NAMES, got, ref):
        if g is None:
            continue
        assert g.shape == r.shape, name
        assert np.isfinite(g).all(), f"{name} has non-finite entries"
        errs[name] = rel_err(g, r)
    say("   " + "  ".join(f"{n}={e:.2e}" for n, e in errs.items()) + f"  (tol {BWD_TOL}, {tol})")
    for n, e in errs.items():
        t = tol.get(n, BWD_TOL)
        assert e <= t, f"{n}: {e:.3e} > {t}"
    return got, ref


F32 = gen.WORKLOADS["tiny_f32"]
BF16 = gen.WORKLOADS["bf16_4k"]


def test_f32_one_chunk():
    check(F32.with_(T=16), seed=400)


@pytest.mark.parametrize("T", [1, 15, 17, 77, 160])
def test_f32_ragged(T):
    """Lengths below, at and past a chunk, and several chunks with a ragged tail."""
    check(F32.with_(B=1, H=2, T=T, dk=64, dv=64, s0_sd=0.5), seed=410 + T)


@pytest.mark.parametrize("dk,dv", [(32, 128), (128, 32), (64, 128), (128, 64), (128, 128)])
def test_f32_dims(dk, dv):
    check(F32.with_(B=1, H=2, T=83, dk=dk, dv=dv, s0_sd=0.3), seed=420 + dk + dv)


@pytest.mark.parametrize("dk,dv", [(32, 64), (64, 32), (64, 128)])
def test_bf16_dims(dk, dv):
    """bf16 inputs at the smaller key and value widths (each width has its own kernel instances)."""
    check(BF16.with_(B=1, H=2, T=83, dk=dk, dv=dv, s0_sd=0.3), seed=425 + dk + dv)


def test_bf16_multi_head():
    check(BF16.with_(B=2, H=3, T=203, s0_sd=0.5), seed=430)


def test_bf16_without_state_gradients():
    """No S0, no dS_final, dS0 not wanted."""
    check(BF16.with_(B=1, H=2, T=130), seed=431, with_dSf=False, want_dS0=False)


def test_unbounded_gate():
    """g = -softplus(w) with strongly negative log-decays: the pair-by-pair factors stay <= 1."""
    wl = gen.WORKLOADS["unbounded"].with_(B=1, H=2, T=150, s0_sd=0.5)
    check(wl, seed=440)


@pytest.mark.parametrize("g_min", [-8.0, -0.5])
def test_other_bounds(g_min):
    """A bound whose forward chunks get flagged (-8) and a mild one."""
    check(BF16.with_(B=1, H=2, T=100, g_min=g_min, s0_sd=0.5), seed=450)


@pytest.mark.parametrize("w_mu,what", [(4.0, "every chunk past the span limit (pair-by-pair terms)"),
                                       (-4.0, "no chunk near it (products of e^{+-G} factors)"),
                                       (1.0, "a mix of both kinds of chunk")])
def test_span_paths(w_mu, what):
    """g_min = -8: chunks whose span is below -80 take the pair-by-pair terms, the others the dense
    products; both against the oracle, separately and mixed in one sequence.

    With every chunk decaying by about e^{-126} (w_mu = 4), dg per token is a small difference of
    in-chunk terms, and the chunk form's fp32 rounding reaches about 3e-5 of max |dw| (a float32 numpy
    model of the same formulas gives 3.0e-5 on these inputs, its float64 twin 1e-13 against the oracle);
    dw is held to 1e-4 there, every other gradient to BWD_TOL."""
    tol = {"dw": 1e-4} if w_mu > 2 else None
    check(F32.with_(B=1, H=2, T=150, dk=64, dv=64, g_min=-8.0, w_mu=w_mu, w_sd=1.0, s0_sd=0.5), seed=455, tol=tol)


def test_long_f32():
    """A few hundred chunks of reverse state chain."""
    check(F32.with_(B=1, H=1, T=4000, dk=128, dv=128, s0_sd=0.5), seed=460)


def test_long_ragged_bf16():
    """A few hundred chunks with a ragged last one (3001 = 187 * 16 + 9) on two heads."""
    check(BF16.with_(B=1, H=2, T=3001, s0_sd=0.5), seed=465)


def test_zero_length():
    """T = 0: dS0 = dS_final, nothing else to write."""
    wl = F32.with_(B=2, H=2, T=0, dk=64, dv=32)
    got, ref = run_case(wl, 470)
    assert np.array_equal(got[5], gen.make_cotangents(wl, 470)["dSf"])


def test_repeat_is_deterministic_up_to_atomics():
    """Two calls agree to fp32 rounding (value-column blocks are summed with atomics)."""
    wl = BF16.with_(B=1, H=2, T=96, s0_sd=0.5)
    a, _ = run_case(wl, 480)
    b, _ = run_case(wl, 480)
    for n, x, y in zip(NAMES, a, b):
        assert rel_err(x, y) <= 1e-6, n


def test_headline_shape_tail_window():
    """Full-size shape (B1 H16 T65536 d128 bf16): on two sampled heads, the gradients of the last
    W tokens depend on the rest only through the state entering the window, so the oracle forward
    gives that state and the oracle backward over the window gives exact gradients for it."""
    wl = gen.WORKLOADS["headline"]
    seed, W = 490, 512
    inp = gen.make_torch(wl, seed, "cuda")
    g = torch.Generator(device="cuda").manual_seed(seed + 1)
    dO = torch.randn((wl.B, wl.H, wl.T, wl.dv), generator=g, device="cuda").to(gen.torch_dtype(wl.dtype))
    dSf = torch.randn((wl.B, wl.H, wl.dk, wl.dv), generator=g, device="cuda")
    say(f"[case] bwd headline tail window W={W}")
    got = chunk_bwd(inp["q"], inp["k"], inp["v"], inp["w"], inp["beta"], dO, S0=inp["S0"], dS_final=dSf,
                    g_min=wl.g_min, want_dS0=False)
    torch.cuda.synchronize()
    for h in (0, wl.H - 1):
        f = gen.head_to_f64(inp, 0, h)
        cut = wl.T - W
        pre = {k: (None if v is None else v[:, :, :cut]) for k, v in f.items() if k != "S0"}
        _, S_cut = orc.kda_reference(pre["q"], pre["k"], pre["v"], pre["w"], pre["beta"], f["S0"], wl.g_min,
                                     nthreads=1)
        win = {k: v[:, :, cut:] for k, v in f.items() if k != "S0"}
        dO_w = dO[0:1, h:h + 1, cut:].float().cpu().numpy().astype(np.float64)
        dSf_h = dSf[0:1, h:h + 1].cpu().numpy().astype(np.float64)
        ref = orc.kda_backward(win["q"], win["k"], win["v"], win["w"], win["beta"], S_cut, wl.g_min, dO_w,
                               dSf_h, nthreads=1)
        for name, x, r in zip(NAMES[:5], got[:5], ref[:5]):
            xs = x[0:1, h:h + 1, cut:].cpu().numpy()
            e = rel_err(xs, r)
            say(f"   head {h} {name}: {e:.2e}")
            assert np.isfinite(xs).all() and e <= BWD_TOL, name
    for x in got[:5]:
        assert torch.isfinite(x).all()


def test_rejects_other_chunk_sizes():
    wl = F32.with_(T=20)
    inp = gen.numpy_to_torch(gen.make_numpy(wl, 1), "cuda")
    dO = torch.zeros((1, 1, 20, 32), device="cuda")
    from chunked_gated_delta_amd import KdaError
    with pytest.raises(KdaError):
        chunk_bwd(inp["q"], inp["k"], inp["v"], inp["w"], inp["beta"], dO, chunk=32)
