"""Recurrent decode (kda_decode): the per-token recurrence on a resident fp32 state, advanced in
place.  Parity against the fp64 oracle (which is the same recurrence), and agreement with the
chunked forward run from the same state."""
import numpy as np
import pytest

from chunked_gated_delta_amd import inputs as gen
from kda_testutil import TOL, rel_err, say, oracle_run

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from chunked_gated_delta_amd import chunk_fwd, decode  # noqa: E402

BF16 = gen.WORKLOADS["bf16_4k"]
F32 = gen.WORKLOADS["tiny_f32"]


def run_decode(wl, seed, s0_sd=0.5, steps=None):
    """Decode wl's T tokens from S0 ~ N(0, s0_sd), in calls of `steps` tokens (all at once when
    None); returns (o, S) from the GPU and (o_ref, S_ref) from the oracle."""
    wl = wl.with_(s0_sd=s0_sd)
    inp = gen.make_numpy(wl, seed)
    say(f"[case] decode {wl} seed={seed} steps={steps}")
    t = gen.numpy_to_torch(inp, "cuda")
    S = t["S0"].clone()
    T = wl.T
    steps = steps or T
    outs = []
    for a in range(0, T, steps):
        b = min(T, a + steps)
        sl = lambda x: x[:, :, a:b].contiguous()
        outs.append(decode(sl(t["q"]), sl(t["k"]), sl(t["v"]), sl(t["w"]), sl(t["beta"]), S, g_min=wl.g_min))
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=2).float().cpu().numpy()
    o_ref, S_ref = oracle_run(inp, wl.g_min)
    return o, S.cpu().numpy(), o_ref, S_ref


def check(wl, seed, **kw):
    o, S, o_ref, S_ref = run_decode(wl, seed, **kw)
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    tol_o, tol_s = TOL[wl.dtype]
    say(f"   err_o={eo:.3e} (tol {tol_o})  err_S={es:.3e} (tol {tol_s})")
    assert np.isfinite(o).all() and np.isfinite(S).all()
    assert eo <= tol_o and es <= tol_s


@pytest.mark.parametrize("T", [1, 2, 7])
def test_bf16_single_call(T):
    check(BF16.with_(B=2, H=3, T=T), seed=300 + T)


def test_bf16_token_by_token():
    """Forty calls of one token each carry the state through HBM between calls."""
    check(BF16.with_(B=1, H=2, T=40), seed=310, steps=1)


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 64), (128, 128), (32, 64)])
def test_f32_dims(dk, dv):
    check(F32.with_(B=1, H=2, T=5, dk=dk, dv=dv), seed=dk + dv)


def test_f32_token_by_token():
    check(F32.with_(B=2, H=2, T=12), seed=320, steps=1)


def test_unbounded_gate():
    """g = -softplus(w): per token there is no reciprocal, so nothing to flag."""
    check(gen.WORKLOADS["unbounded"].with_(B=1, H=2, T=9), seed=330)


def test_no_decay():
    check(BF16.with_(B=1, H=2, T=6, g_min=0.0), seed=340)


def test_matches_chunked_forward():
    """Decoding a prompt's last tokens from the chunked forward's state gives the same outputs and
    final state as running the chunked forward over the whole sequence."""
    wl = BF16.with_(B=1, H=4, T=300, s0_sd=0.3)
    inp = gen.numpy_to_torch(gen.make_numpy(wl, 350), "cuda")
    o_all, S_all, _ = chunk_fwd(inp["q"], inp["k"], inp["v"], inp["w"], inp["beta"], inp["S0"], g_min=wl.g_min)
    cut = 290
    pre = lambda x: x[:, :, :cut].contiguous()
    post = lambda x: x[:, :, cut:].contiguous()
    _, S_pre, _ = chunk_fwd(pre(inp["q"]), pre(inp["k"]), pre(inp["v"]), pre(inp["w"]), pre(inp["beta"]), inp["S0"],
                            g_min=wl.g_min)
    S = S_pre.clone()
    outs = [decode(post(inp["q"])[:, :, i:i + 1].contiguous(), post(inp["k"])[:, :, i:i + 1].contiguous(),
                   post(inp["v"])[:, :, i:i + 1].contiguous(), post(inp["w"])[:, :, i:i + 1].contiguous(),
                   post(inp["beta"])[:, :, i:i + 1].contiguous(), S, g_min=wl.g_min) for i in range(wl.T - cut)]
    torch.cuda.synchronize()
    o_dec = torch.cat(outs, dim=2).float().cpu().numpy()
    eo = rel_err(o_dec, o_all[:, :, cut:].float().cpu().numpy())
    es = rel_err(S.cpu().numpy(), S_all.cpu().numpy())
    say(f"   decode vs chunked: err_o={eo:.3e} err_S={es:.3e}")
    assert eo < 2e-2 and es < 1e-2


def test_full_size_batch():
    """A serving-size batch, B=64 H=16 d=128, one token: parity on sampled heads."""
    wl = BF16.with_(B=64, H=16, T=1, s0_sd=0.5)
    t = gen.make_torch(wl, seed=360, device="cuda")
    S = t["S0"].clone()
    o = decode(t["q"], t["k"], t["v"], t["w"], t["beta"], S, g_min=wl.g_min)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (37, 9), (63, 15)]:
        f = {n: t[n][b:b + 1, h:h + 1].float().cpu().numpy().astype(np.float64) for n in ("q", "k", "v", "w", "beta")}
        S0 = t["S0"][b:b + 1, h:h + 1].cpu().numpy().astype(np.float64)
        from oracle import oracle as orc
        o_ref, S_ref = orc.kda_reference(f["q"], f["k"], f["v"], f["w"], f["beta"], S0, wl.g_min)
        eo = rel_err(o[b:b + 1, h:h + 1].float().cpu().numpy(), o_ref)
        es = rel_err(S[b:b + 1, h:h + 1].cpu().numpy(), S_ref)
        say(f"   head ({b},{h}): err_o={eo:.3e} err_S={es:.3e}")
        assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1]
