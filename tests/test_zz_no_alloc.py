"""kda_chunk_fwd_noalloc through the C ABI: the scratch-free entry point gives exactly what the
workspace entry point gives for the same plan (the fused plan where the automatic plan is the
corrected one, whose queries would not fit the array), on calls in a row that reuse the library's
static array (the second and later calls smaller than the first); it agrees with the automatic
kda_chunk_fwd and with the fp64 oracle to the parity tolerance."""
import ctypes

import numpy as np
import pytest

from chunked_gated_delta_amd import inputs as gen
from kda_testutil import TOL, rel_err, say, oracle_run

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _noalloc_call(t, wl, o, S, st):
    """One raw kda_chunk_fwd_noalloc call on the current stream (no allocation in the entry point)."""
    from chunked_gated_delta_amd import _lib
    from chunked_gated_delta_amd.api import _dtype_code, _ptr, make_shape
    shape = make_shape(wl.B, wl.H, wl.T, wl.dk, wl.dv, _dtype_code(t["q"]))
    stream = torch.cuda.current_stream()
    return _lib.load().kda_chunk_fwd_noalloc(
        _ptr(t["q"]), _ptr(t["k"]), _ptr(t["v"]), _ptr(t["w"]), _ptr(t["beta"]), _ptr(t["S0"]),
        ctypes.c_float(wl.g_min), 16, ctypes.byref(shape), _ptr(o), _ptr(S), _ptr(st),
        ctypes.c_void_p(stream.cuda_stream))


def _check_against_workspace_entry(wl, seed, with_oracle):
    from chunked_gated_delta_amd import chunk_fwd, decode_stats, workspace_bytes
    inp = gen.make_numpy(wl, seed)
    t = gen.numpy_to_torch(inp, "cuda")
    mfma = wl.dtype == "bf16" and wl.dk == wl.dv == 128
    plan = "fused" if mfma else "auto"
    need = workspace_bytes(wl.B, wl.H, wl.T, wl.dk, wl.dv, gen.torch_dtype(wl.dtype), path=plan)
    say(f"[case] noalloc {wl} seed={seed} plan={plan} scratch={need} bytes")
    o = torch.empty_like(t["v"])
    S = torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
    st = torch.empty(4, dtype=torch.int32, device="cuda")
    rc = _noalloc_call(t, wl, o, S, st)
    assert rc == 0, rc
    o_ref, S_ref, st_ref = chunk_fwd(t["q"], t["k"], t["v"], t["w"], t["beta"], t["S0"], g_min=wl.g_min, path=plan)
    o_auto, S_auto, st_auto = chunk_fwd(t["q"], t["k"], t["v"], t["w"], t["beta"], t["S0"], g_min=wl.g_min)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    assert decode_stats(st) == decode_stats(st_ref)
    st_a = decode_stats(st_auto)
    assert {k: st_a[k] for k in ("n_chunks", "n_flagged", "n_nonfinite")} == \
        {k: decode_stats(st)[k] for k in ("n_chunks", "n_flagged", "n_nonfinite")}
    eo = rel_err(o.float().cpu().numpy(), o_auto.float().cpu().numpy())
    es = rel_err(S.cpu().numpy(), S_auto.cpu().numpy())
    say(f"   against the automatic plan: err_o={eo:.3e} err_S={es:.3e}")
    assert eo <= TOL[wl.dtype][0] and es <= TOL[wl.dtype][1]
    if with_oracle:
        o64, S64 = oracle_run(inp, wl.g_min)
        eo, es = rel_err(o.float().cpu().numpy(), o64), rel_err(S.cpu().numpy(), S64)
        say(f"   oracle: err_o={eo:.3e} err_S={es:.3e}")
        assert eo <= TOL[wl.dtype][0] and es <= TOL[wl.dtype][1]
    return need


def test_noalloc_calls_in_a_row():
    bf16 = gen.WORKLOADS["bf16_4k"]
    # first call: 16 heads of 8192 tokens, 16 segments each (48 MiB of the 64 MiB array)
    n1 = _check_against_workspace_entry(bf16.with_(B=1, H=16, T=8192), seed=71, with_oracle=False)
    # second call, smaller: 4 heads with an initial state and a ragged tail (4 segments each)
    n2 = _check_against_workspace_entry(bf16.with_(B=1, H=4, T=1000, s0_sd=0.3), seed=72, with_oracle=True)
    assert 0 < n2 < n1
    # third: a one-segment plan (no scratch at all), and the fp32 vector path
    _check_against_workspace_entry(bf16.with_(B=1, H=2, T=100), seed=73, with_oracle=True)
    _check_against_workspace_entry(gen.WORKLOADS["tiny_f32"], seed=74, with_oracle=True)
    # the first shape again, after the smaller calls left their contents in the array
    _check_against_workspace_entry(bf16.with_(B=1, H=16, T=8192), seed=75, with_oracle=False)


def test_noalloc_rejects_more_than_its_scratch():
    from chunked_gated_delta_amd import KdaError, chunk_fwd_noalloc
    wl = gen.WORKLOADS["bf16_4k"].with_(B=1, H=128, T=2048)   # 128 heads x 3 segments x 192 KiB = 72 MiB
    t = {n: torch.zeros(s, dtype=torch.bfloat16, device="cuda") for n, s in
         (("q", (1, 128, 2048, 128)), ("k", (1, 128, 2048, 128)), ("v", (1, 128, 2048, 128)),
          ("w", (1, 128, 2048, 128)), ("beta", (1, 128, 2048)))}
    say(f"[case] noalloc rejection {wl}")
    with pytest.raises(KdaError) as e:
        chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["w"], t["beta"])
    assert e.value.code == -6
