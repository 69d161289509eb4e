"""Concurrent calls on separate streams: the library keeps no state between calls beyond per-device
kernel attributes, so forwards (and a decode step) issued on two torch streams at once, each with its
own workspace and outputs, give exactly what the same calls give one after the other."""
import pytest

from chunked_gated_delta_amd import inputs as gen
from kda_testutil import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

NAMES = ("q", "k", "v", "w", "beta")


def _workspace(wl):
    from chunked_gated_delta_amd import workspace_bytes
    n = workspace_bytes(wl.B, wl.H, wl.T, wl.dk, wl.dv, gen.torch_dtype(wl.dtype))
    return torch.empty(max(1, n), dtype=torch.uint8, device="cuda")


def test_forwards_on_two_streams():
    from chunked_gated_delta_amd import chunk_fwd, decode_stats
    # two different shapes and gates: a multi-segment bf16 forward and an unbounded-gate one
    wls = [gen.WORKLOADS["bf16_4k"].with_(B=1, H=4, T=3000, s0_sd=0.3),
           gen.WORKLOADS["unbounded"].with_(B=2, H=3, T=1500)]
    inps = [gen.make_torch(wl, seed=31 + i, device="cuda") for i, wl in enumerate(wls)]
    wss = [_workspace(wl) for wl in wls]
    say(f"[case] two streams: {wls[0]} and {wls[1]}")
    seq = []
    for wl, t, ws in zip(wls, inps, wss):
        o, S, st = chunk_fwd(*(t[n] for n in NAMES), t["S0"], g_min=wl.g_min, workspace=ws)
        torch.cuda.synchronize()
        seq.append((o.clone(), S.clone(), decode_stats(st)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full_like(r[0], float("nan")) for r in seq]
    Ss = [torch.full_like(r[1], float("nan")) for r in seq]
    torch.cuda.synchronize()
    for rep in range(3):
        sts = []
        for i, (wl, t, ws, s) in enumerate(zip(wls, inps, wss, streams)):
            with torch.cuda.stream(s):
                sts.append(chunk_fwd(*(t[n] for n in NAMES), t["S0"], g_min=wl.g_min, out=outs[i], S_final=Ss[i],
                                     workspace=ws, stream=s)[2])
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], seq[i][0]) and torch.equal(Ss[i], seq[i][1]), (rep, i)
            assert decode_stats(sts[i]) == seq[i][2], (rep, i)
            outs[i].fill_(float("nan"))
            Ss[i].fill_(float("nan"))
        torch.cuda.synchronize()
    say("   3 rounds of concurrent calls equal to the sequential ones")


def test_forward_and_decode_on_two_streams():
    """A long forward on one stream while a decode loop advances resident states on another."""
    from chunked_gated_delta_amd import chunk_fwd, decode
    wl = gen.WORKLOADS["bf16_4k"].with_(B=1, H=16, T=8192)
    wd = gen.WORKLOADS["bf16_4k"].with_(B=8, H=8, T=1)
    t = gen.make_torch(wl, seed=41, device="cuda")
    ws = _workspace(wl)
    toks = [gen.make_torch(wd, seed=50 + i, device="cuda") for i in range(8)]
    g = torch.Generator(device="cuda").manual_seed(9)
    S0 = 0.3 * torch.randn((wd.B, wd.H, wd.dk, wd.dv), generator=g, device="cuda")
    say(f"[case] forward {wl} beside a decode loop of {len(toks)} tokens on {wd.B * wd.H} heads")
    o_ref, S_ref, _ = chunk_fwd(*(t[n] for n in NAMES), t["S0"], g_min=wl.g_min, workspace=ws)
    Sd_ref = S0.clone()
    od_ref = [decode(*(x[n] for n in NAMES), Sd_ref, g_min=wd.g_min).clone() for x in toks]
    torch.cuda.synchronize()
    o_ref, S_ref = o_ref.clone(), S_ref.clone()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    o = torch.empty_like(o_ref)
    S = torch.empty_like(S_ref)
    Sd = S0.clone()
    od = []
    torch.cuda.synchronize()
    with torch.cuda.stream(sa):
        chunk_fwd(*(t[n] for n in NAMES), t["S0"], g_min=wl.g_min, out=o, S_final=S, workspace=ws, stream=sa)
    with torch.cuda.stream(sb):
        for x in toks:
            od.append(decode(*(x[n] for n in NAMES), Sd, g_min=wd.g_min, stream=sb))
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    assert torch.equal(Sd, Sd_ref)
    assert all(torch.equal(a, b) for a, b in zip(od, od_ref))
    say("   forward and decode loop equal to the sequential calls")
