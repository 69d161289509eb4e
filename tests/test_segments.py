"""Sequence segments of the matrix-core path.  Each (b, h) sequence is cut into
segments.  Each segment's affine state map S_end = M S_start + X is computed in
parallel, and the maps are then chained.  A forced segment length
(`seg_steps`, in 32-token steps) exercises plans with many segments at sizes the
oracle finishes in seconds.  The ragged tail always falls in the last segment."""
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


SEG_PATHS = ["fused", "corr"]


def check(wl, seed, path, **kw):
    need_path(path)
    eo, es, st, *_ = compare(wl, seed=seed, path=path, **kw)
    tol_o, tol_s = TOL[wl.dtype]
    say(f"   err_o={eo:.3e} (tol {tol_o})  err_S={es:.3e} (tol {tol_s})  stats={st}")
    assert eo <= tol_o and es <= tol_s
    assert st["n_nonfinite"] == 0
    assert st["n_chunks"] == wl.B * wl.H * ((wl.T + 15) // 16)
    return st


@pytest.mark.parametrize("path", SEG_PATHS)
@pytest.mark.parametrize("T,seg", [(64, 1), (300, 1), (300, 2), (300, 3), (1000, 1), (1000, 5), (1000, 7)])
def test_forced_segments(T, seg, path):
    check(BF16.with_(B=1, H=2, T=T), seed=200 + T + seg, path=path, seg_steps=seg)


@pytest.mark.parametrize("T,seg", [(320, 3), (1440, 20), (1450, 20)])
def test_correction_workgroup_boundaries(T, seg):
    """The corrected plan's correction runs 16 steps per workgroup: T = 320 with segments of 3 steps
    leaves a last segment of one step; segments of 20 steps take two workgroups each, the second
    covering 4 steps, and the last segment (5 steps; 6 with the 10-token tail of T = 1450) leaves the
    second workgroup of its segment empty.  S0 present, so every correction is non-zero."""
    check(BF16.with_(B=1, H=2, T=T, s0_sd=0.5), seed=400 + T + seg, path="corr", seg_steps=seg)


@pytest.mark.parametrize("path", SEG_PATHS)
@pytest.mark.parametrize("seg", [1, 4])
def test_segments_with_initial_state(seg, path):
    """Decay-stress gates with S0 ~ N(0, 0.1): the first segment starts from S0."""
    st = check(gen.WORKLOADS["decay_stress"].with_(H=2, T=1000), seed=3, path=path, seg_steps=seg)
    assert st["n_flagged"] == 0


@pytest.mark.parametrize("path", SEG_PATHS)
@pytest.mark.parametrize("B,H", [(1, 3), (3, 5), (2, 8)])
def test_chaining_block_order_over_heads(B, H, path):
    """The chaining pass spreads the eight 16-column slices of every head over its grid in an
    XCD-aware order; with S0 present and B*H not a multiple of 8 (and one that is), every head's
    slices must still pick up that head's own S0, M_j and X_j."""
    check(BF16.with_(B=B, H=H, T=330, s0_sd=0.5), seed=30 + 7 * B + H, path=path, seg_steps=3)


def test_statistics_fold_over_many_heads():
    """300 heads (B3 H100), segments of 2 steps, g_min = -8: segment 0 runs inside the map pass and
    leaves one statistics record per head, which the chaining pass folds with a strided loop over
    more heads than its workgroup has threads; the call's counters must still count every chunk and
    exactly the flagged ones."""
    wl = BF16.with_(B=3, H=100, T=160, g_min=-8.0, w_mu=0.0, w_sd=1.0, s0_sd=0.3)   # 1928 of 3000 flagged
    st = check(wl, seed=19, path="fused", seg_steps=2)
    pred = orc.predicted_flags(gen.make_numpy(wl, 19)["w"], -8.0)
    assert st["n_flagged"] == int(pred.sum()) and 0 < st["n_flagged"] < pred.size


@pytest.mark.parametrize("path", SEG_PATHS)
def test_segments_no_decay(path):
    """g_min = 0: nothing is forgotten, so each segment transition is a pure
    product of (I - beta k k^T) factors, far from zero.  A nonzero S0 flows
    through every transition."""
    check(BF16.with_(B=1, H=2, T=640, g_min=0.0, s0_sd=0.5), seed=14, path=path, seg_steps=2)


@pytest.mark.parametrize("path", SEG_PATHS)
def test_segments_pure_decay(path):
    """beta = 0: X = 0 and M = diag(prod e^g), so the state is S0, decayed.  The decay is
    slow (w ~ N(-5, 0.5), about -0.034 per token), so the decayed S0 stays well inside fp32's range."""
    wl = BF16.with_(B=1, H=2, T=800, s0_sd=0.5, w_mu=-5.0, w_sd=0.5)
    check(wl, seed=15, path=path, seg_steps=3, mutate=lambda inp: inp["beta"].fill(0.0))


@pytest.mark.parametrize("path", SEG_PATHS)
def test_segments_with_flagged_chunks(path):
    """g_min = -8: chunks past the span limit take the per-position path inside segments."""
    wl = BF16.with_(B=1, H=2, T=700, g_min=-8.0, w_mu=4.0, w_sd=1.0)
    st = check(wl, seed=16, path=path, seg_steps=3)
    pred = orc.predicted_flags(gen.make_numpy(wl, 16)["w"], -8.0)
    assert st["n_flagged"] == int(pred.sum()) and st["n_flagged"] > 0


@pytest.mark.parametrize("path", SEG_PATHS)
def test_automatic_plan_several_heads(path):
    """B2 H4 T2048: the automatic plan cuts each sequence into 8 segments of 8 steps."""
    check(BF16.with_(B=2, H=4, T=2048), seed=17, path=path)


@pytest.mark.parametrize("path", ["auto", "fused"])
def test_automatic_plan_odd_head_count(path):
    """B3 H5 (15 heads) T8229 with S0: the corrected (automatic) plan takes 17 segments per head (255
    workgroups in its pass), a first segment of 17 steps and a last one of a single, ragged step; the
    fused plan 18 segments (17 workgroups per head in each pass)."""
    check(BF16.with_(B=3, H=5, T=8229, s0_sd=0.3), seed=21, path=path)


@pytest.mark.parametrize("path", SEG_PATHS)
def test_segment_plans_agree(path):
    """Different segment plans change only the rounding."""
    need_path(path)
    wl = BF16.with_(B=1, H=2, T=900, s0_sd=0.3)
    t = gen.numpy_to_torch(gen.make_numpy(wl, 18), "cuda")
    say(f"[case] segment plans {wl} path={path}")
    outs = [gpu_run(t, wl.g_min, path=path, seg_steps=s) for s in (0, 2, 3, 29)]
    o0, S0_, _ = outs[0]
    for o, S, _ in outs[1:]:
        assert rel_err(o.float().cpu().numpy(), o0.float().cpu().numpy()) < 1e-2
        assert rel_err(S.cpu().numpy(), S0_.cpu().numpy()) < 5e-3


@pytest.mark.parametrize("path", SEG_PATHS)
def test_in_place_state_with_many_segments(path):
    """S_final == S0 (the in-place update kda.h allows) with at least three segments: the last
    segment's S_final write must not reach the first segment's read of S0."""
    from chunked_gated_delta_amd import chunk_fwd
    need_path(path)
    wl = BF16.with_(B=1, H=2, T=700, s0_sd=0.3)
    inp = gen.make_numpy(wl, 61)
    t = gen.numpy_to_torch(inp, "cuda")
    say(f"[case] in-place state {wl} path={path} seg_steps=3 (8 segments)")
    args = [t[n] for n in ("q", "k", "v", "w", "beta")]
    oa, Sa, _ = chunk_fwd(*args, t["S0"], path=path, seg_steps=3)
    state = t["S0"].clone()
    ob, _, _ = chunk_fwd(*args, state, S_final=state, path=path, seg_steps=3)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(Sa, state)
    o_ref, S_ref = orc.kda_reference(*(gen.all_to_f64(inp)[n] for n in ("q", "k", "v", "w", "beta", "S0")), wl.g_min)
    assert rel_err(ob.float().cpu().numpy(), o_ref) <= TOL["bf16"][0]
    assert rel_err(state.cpu().numpy(), S_ref) <= TOL["bf16"][1]
