"""The corrected segment plan, written out in numpy (CPU, float64).

The matrix-core forward cuts each (b, h) sequence into segments and relies on the outputs being
affine in a segment's entering state: with S_t = X_t + M_t S_start the state entering chunk t of
the segment (X from a zero state with the real values, M from the identity with none),
    O_t = [Qbar X_t + P T diag(beta)(V - Kbar X_t)] + [Qbar M_t - P T diag(beta) Kbar M_t] S_start
        = O_t(from zero) + Qtil_t S_start.
This model runs the plan on the 16-token chunk form ("From Numerical Stability to Load Balancing ..."
section 2.1: in-chunk blocks with exp(G_r - G_j) scaling, the WY solve T = (I + A)^{-1}, the
chunk-to-chunk state update) in float64: segment 0 exactly from S0; every later segment from a zero
state, with its transition M, its Qtil per chunk and its map (X, M); the maps chained from segment 0's
leaving state; each later segment's outputs corrected by Qtil S_start.  It must agree with the
oracle's token recurrence to float64 rounding, which checks the identity the kernels use, for every
gate kind and with an initial state.  It is a model of the formulas, not a second oracle: nothing
here is compared with the GPU."""
import numpy as np
import pytest

from chunked_gated_delta_amd import inputs as gen
from oracle import oracle as orc

C = 16


def _gate(w, g_min):
    if np.isfinite(g_min):
        return g_min / (1.0 + np.exp(-w))
    return -np.logaddexp(0.0, w)   # -softplus(w)


def chunk_operands(q, k, beta, g):
    """One chunk's operands: Qbar, Kbar, Ktil, P, T and the chunk total Gam (float64)."""
    G = np.cumsum(g, axis=0)
    gam = G[-1]
    e = np.exp(np.minimum(G[:, None, :] - G[None, :, :], 0.0))   # exp(G_r - G_j) for j <= r
    A = np.tril(np.einsum("rc,jc,rjc->rj", k, k, e), -1)
    P = np.tril(np.einsum("rc,jc,rjc->rj", q, k, e))
    T = np.linalg.inv(np.eye(len(k)) + beta[:, None] * A)
    return dict(Qbar=q * np.exp(G), Kbar=k * np.exp(G), Ktil=k * np.exp(gam - G), P=P, T=T, gam=gam, beta=beta)


def chunk_step(op, S, v):
    """Outputs and leaving state of one chunk from entering state S (v = None: no values)."""
    R = -op["beta"][:, None] * (op["Kbar"] @ S)
    if v is not None:
        R = R + op["beta"][:, None] * v
    U = op["T"] @ R
    O = op["Qbar"] @ S + op["P"] @ U
    return O, np.exp(op["gam"])[:, None] * S + op["Ktil"].T @ U


def corrected_plan(q, k, v, w, beta, S0, g_min, seg_chunks):
    """The plan for one head: (o, S_final)."""
    T, dk = q.shape
    dv = v.shape[1]
    n = (T + C - 1) // C
    pad = n * C - T
    pd = lambda x: np.concatenate([x, np.zeros((pad,) + x.shape[1:])]) if pad else x
    q, k, v, beta = pd(q), pd(k), pd(v), pd(beta)
    g = pd(_gate(w, g_min))   # tokens past the end: no decay, no write, no read
    ops = [chunk_operands(q[c * C:(c + 1) * C], k[c * C:(c + 1) * C], beta[c * C:(c + 1) * C], g[c * C:(c + 1) * C])
           for c in range(n)]
    vs = [v[c * C:(c + 1) * C] for c in range(n)]
    bounds = [(s, min(s + seg_chunks, n)) for s in range(0, n, seg_chunks)]
    o = np.zeros((n * C, dv))
    # segment 0, exactly
    S = S0.copy()
    for c in range(*bounds[0]):
        o[c * C:(c + 1) * C], S = chunk_step(ops[c], S, vs[c])
    S_start = [None, S]
    # later segments: outputs from zero, Qtil per chunk, the map (X, M)
    qtil, maps = {}, []
    for a, b in bounds[1:]:
        X, M = np.zeros((dk, dv)), np.eye(dk)
        for c in range(a, b):
            o[c * C:(c + 1) * C], X_next = chunk_step(ops[c], X, vs[c])
            # the transition: the same step with M for S and no values; its outputs are Qtil,
            # Qbar M + P T diag(beta)(-Kbar M)
            qtil[c], M = chunk_step(ops[c], M, None)
            X = X_next
        maps.append((X, M))
    # chaining: S_start(j + 1) = M_j S_start(j) + X_j
    for X, M in maps:
        S_start.append(M @ S_start[-1] + X)
    # correction of the later segments
    for j, (a, b) in enumerate(bounds[1:], start=1):
        for c in range(a, b):
            o[c * C:(c + 1) * C] += qtil[c] @ S_start[j]
    return o[:T], S_start[-1]


CASES = [
    ("bounded", -5.0, 0.0, 2.0),
    ("slow decay", -1.0, -6.0, 1.0),
    ("no decay", 0.0, 0.0, 1.0),
    ("unbounded", -np.inf, 3.0, 3.0),
]


@pytest.mark.parametrize("name,g_min,w_mu,w_sd", CASES)
@pytest.mark.parametrize("T,seg_chunks", [(200, 3), (333, 4), (64, 1)])
def test_corrected_plan_equals_token_recurrence(name, g_min, w_mu, w_sd, T, seg_chunks):
    """Segments of `seg_chunks` 16-token chunks (ragged ends), S0 present; o and S_final of the plan
    against the oracle's token recurrence."""
    wl = gen.WORKLOADS["tiny_f32"].with_(B=1, H=2, T=T, dk=32, dv=64, g_min=g_min, w_mu=w_mu, w_sd=w_sd, s0_sd=0.5)
    inp = gen.make_numpy(wl, seed=T + seg_chunks)
    f = {n: inp[n].astype(np.float64) for n in ("q", "k", "v", "w", "beta", "S0")}
    o_ref, S_ref = orc.kda_reference(f["q"], f["k"], f["v"], f["w"], f["beta"], f["S0"], g_min)
    for h in range(wl.H):
        o, S = corrected_plan(f["q"][0, h], f["k"][0, h], f["v"][0, h], f["w"][0, h], f["beta"][0, h],
                              f["S0"][0, h], g_min, seg_chunks)
        eo = np.max(np.abs(o - o_ref[0, h])) / np.max(np.abs(o_ref[0, h]))
        es = np.max(np.abs(S - S_ref[0, h])) / np.max(np.abs(S_ref[0, h]))
        assert eo < 1e-10 and es < 1e-10, (name, h, eo, es)


def test_correction_is_not_trivial():
    """The check has teeth: with slow decay and S0 present, dropping the correction (outputs from a
    zero state only) misses the oracle by far more than rounding."""
    wl = gen.WORKLOADS["tiny_f32"].with_(B=1, H=1, T=200, dk=32, dv=64, g_min=-1.0, w_mu=-6.0, w_sd=1.0, s0_sd=0.5)
    inp = gen.make_numpy(wl, seed=5)
    f = {n: inp[n].astype(np.float64) for n in ("q", "k", "v", "w", "beta", "S0")}
    o_ref, _ = orc.kda_reference(f["q"], f["k"], f["v"], f["w"], f["beta"], f["S0"], -1.0)
    args = (f["q"][0, 0], f["k"][0, 0], f["v"][0, 0], f["w"][0, 0], f["beta"][0, 0])
    o_plan, _ = corrected_plan(*args, f["S0"][0, 0], -1.0, 3)
    # the same plan without the correction: segment 0 from S0, every later segment's outputs from
    # its own zero state, which is what one-segment runs of each part give
    o_zero = np.concatenate([corrected_plan(*(x[a:a + 48] for x in args), f["S0"][0, 0] if a == 0 else np.zeros((32, 64)),
                                            -1.0, 3)[0] for a in range(0, 200, 48)])
    e_plan = np.max(np.abs(o_plan - o_ref[0, 0])) / np.max(np.abs(o_ref[0, 0]))
    e_zero = np.max(np.abs(o_zero - o_ref[0, 0])) / np.max(np.abs(o_ref[0, 0]))
    assert e_plan < 1e-10 and e_zero > 1e-2
