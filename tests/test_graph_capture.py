"""HIP graph capture of the library's calls.  The forward (automatic plan: statistics reset, segment
pass, chaining, correction), the recurrent decode step (the launch-bound serving loop, where capture
pays) and the backward are each captured once into a torch CUDA graph (a hipGraph on ROCm) on the
capture stream, after an eager warm-up, and the graph is replayed several times.  Between replays
the program does eager work of its own (fills, a reduction over many blocks) and synchronises; every
replay must reproduce the eager call bit for bit, which the kernels allow (no floating-point atomics,
a fixed launch order).  No call records a memset node: the statistics are reset by a kernel."""
import pytest

from chunked_gated_delta_amd import inputs as gen
from kda_testutil import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

REPLAYS = 4


def _eager_work():
    """Eager work of the program between replays: a multi-block reduction and a copy."""
    x = torch.randn(1 << 20, device="cuda")
    y = x.clone()
    return float((x - y).abs().sum())


def _capture(fn):
    """Warm fn up eagerly on a side stream, then capture it; returns (graph, fn's result in the graph)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


def test_forward_graph_replays():
    from chunked_gated_delta_amd import chunk_fwd, decode_stats, workspace_bytes
    wl = gen.WORKLOADS["bf16_4k"].with_(B=1, H=4, T=2000, s0_sd=0.3)   # 7 segments per head
    say(f"[case] forward under graph capture {wl}")
    t = gen.make_torch(wl, seed=11, device="cuda")
    args = [t[n] for n in ("q", "k", "v", "w", "beta")]
    ws = torch.empty(max(1, workspace_bytes(wl.B, wl.H, wl.T, wl.dk, wl.dv, torch.bfloat16)), dtype=torch.uint8,
                     device="cuda")
    o_ref, S_ref, st_ref = chunk_fwd(*args, t["S0"], g_min=wl.g_min, workspace=ws)
    torch.cuda.synchronize()
    o_ref, S_ref, st_ref = o_ref.clone(), S_ref.clone(), decode_stats(st_ref)
    o = torch.empty_like(o_ref)
    S = torch.empty_like(S_ref)
    g, (_, _, st) = _capture(lambda: chunk_fwd(*args, t["S0"], g_min=wl.g_min, out=o, S_final=S, workspace=ws))
    for i in range(REPLAYS):
        o.fill_(float("nan"))
        S.fill_(float("nan"))
        ws.fill_(0xAB)                       # the graph must not depend on the workspace's contents
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        stats = decode_stats(st)
        say(f"   replay {i}: o equal {torch.equal(o, o_ref)}, S_final equal {torch.equal(S, S_ref)}, stats {stats}")
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
        assert stats == st_ref
        _eager_work()


def test_decode_graph_serving_loop():
    """A serving loop: the captured decode step advances a resident state by one token per replay,
    with each step's token copied into the graph's static inputs beforehand; the outputs and the
    state after every step equal the eager loop's."""
    from chunked_gated_delta_amd import decode
    wl = gen.WORKLOADS["bf16_4k"].with_(B=4, H=8, T=1)
    say(f"[case] decode under graph capture, {wl.B * wl.H} heads, {REPLAYS + 2} steps")
    gen_ = torch.Generator(device="cuda").manual_seed(5)
    steps = [gen.make_torch(wl, seed=100 + i, device="cuda") for i in range(REPLAYS + 2)]
    S0 = 0.3 * torch.randn((wl.B, wl.H, wl.dk, wl.dv), generator=gen_, device="cuda")
    names = ("q", "k", "v", "w", "beta")
    # eager loop
    S_e = S0.clone()
    o_e = []
    for x in steps:
        o_e.append(decode(*(x[n] for n in names), S_e, g_min=wl.g_min).clone())
        S_e_i = S_e.clone()
        x["S_after"] = S_e_i
    torch.cuda.synchronize()
    # graph loop: static inputs, the same resident state, one replay per token
    static = {n: torch.empty_like(steps[0][n]) for n in names}
    o_g = torch.empty_like(o_e[0])
    S_g = S0.clone()
    for n in names:
        static[n].copy_(steps[0][n])
    # the warm-up call inside _capture advances S_g once: restart from S0 afterwards
    g, _ = _capture(lambda: decode(*(static[n] for n in names), S_g, g_min=wl.g_min, out=o_g))
    S_g.copy_(S0)
    for i, x in enumerate(steps):
        for n in names:
            static[n].copy_(x[n])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e[i]), i
        assert torch.equal(S_g, x["S_after"]), i
        _eager_work()
    say(f"   {len(steps)} replays equal to the eager loop")


def test_backward_graph_replays():
    from chunked_gated_delta_amd import chunk_bwd
    wl = gen.WORKLOADS["bf16_4k"].with_(B=1, H=2, T=300, s0_sd=0.3)
    say(f"[case] backward under graph capture {wl}")
    t = gen.make_torch(wl, seed=21, device="cuda")
    gen_ = torch.Generator(device="cuda").manual_seed(3)
    dO = torch.randn((wl.B, wl.H, wl.T, wl.dv), generator=gen_, device="cuda").to(torch.bfloat16)
    dSf = torch.randn((wl.B, wl.H, wl.dk, wl.dv), generator=gen_, device="cuda")
    args = [t[n] for n in ("q", "k", "v", "w", "beta")]
    ref = [x.clone() for x in chunk_bwd(*args, dO, S0=t["S0"], dS_final=dSf, g_min=wl.g_min)]
    torch.cuda.synchronize()
    g, outs = _capture(lambda: chunk_bwd(*args, dO, S0=t["S0"], dS_final=dSf, g_min=wl.g_min))
    for i in range(REPLAYS):
        for x in outs:
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eq = [torch.equal(a, b) for a, b in zip(outs, ref)]
        say(f"   replay {i}: dq, dk, dv, dw, dbeta, dS0 equal {eq}")
        assert all(eq)
        _eager_work()
