"""The 16-token chunk form of the backward, written out in numpy (CPU).

The GPU backward differentiates the chunk form of the forward ("From Numerical Stability to Load
Balancing ..." section 2.1: in-chunk blocks, the WY solve, the chunk-to-chunk state update), not the
token recurrence the oracle differentiates.  This model evaluates the same reverse-mode formulas as
the kernels, chunk by chunk, in a chosen float type:
  - in float64 it must agree with the oracle's adjoint of the token recurrence, which checks the
    derivation itself (every term of dq, dk, dv, dw, dbeta, dS0);
  - in float32 it shows how far rounding alone moves dw when every chunk decays strongly: the bound
    the GPU test uses for that regime rests on this figure.
It is a model of the formulas, not a second oracle: nothing here is compared with the GPU."""
import numpy as np
import pytest

from chunked_gated_delta_amd import inputs as gen
from oracle import oracle as orc

C = 16


def _gate(w, g_min):
    s = 1.0 / (1.0 + np.exp(-w))
    if np.isfinite(g_min):
        return g_min * s, g_min * s * (1.0 - s)
    return -np.log1p(np.exp(w)), -s


def chunk_backward(q, k, v, w, beta, S0, dO, dSf, g_min, dt):
    """Reverse mode of the chunk form for one head; returns (dq, dk, dv, dw, dbeta, dS0) in float64."""
    T, dk = q.shape
    q, k, v, beta, S0, dO, dSf = (x.astype(dt) for x in (q, k, v, beta, S0, dO, dSf))
    g, gd = (x.astype(dt) for x in _gate(w.astype(np.float64), g_min))
    NC = (T + C - 1) // C
    pad = NC * C - T

    def padded(x):   # rows past the end: zero k, q, v, beta, dO and gate
        return np.concatenate([x, np.zeros((pad,) + x.shape[1:], dt)]) if pad else x

    q, k, v, beta, g, dO = map(padded, (q, k, v, beta, g, dO))

    def chunk(n, S):
        sl = slice(n * C, n * C + C)
        G = np.cumsum(g[sl], axis=0, dtype=dt)
        gam = G[-1]
        kk, qq, bb = k[sl], q[sl], beta[sl]
        e = np.exp(np.minimum(G[:, None, :] - G[None, :, :], 0)).astype(dt)   # e^{G_r - G_j}, j <= r
        X = np.tril(np.einsum("rc,jc,rjc->rj", kk, kk, e), -1).astype(dt)
        P = np.tril(np.einsum("rc,jc,rjc->rj", qq, kk, e)).astype(dt)
        Tm = np.linalg.inv(np.eye(C, dtype=dt) + bb[:, None] * X).astype(dt)
        Kbar, Qbar = kk * np.exp(G).astype(dt), qq * np.exp(G).astype(dt)
        Ktil = kk * np.exp(gam - G).astype(dt)
        E = v[sl] - Kbar @ S
        R = bb[:, None] * E
        U = Tm @ R
        return dict(sl=sl, G=G, gam=gam, kk=kk, qq=qq, bb=bb, e=e, X=X, P=P, T=Tm, Kbar=Kbar, Qbar=Qbar,
                    Ktil=Ktil, E=E, R=R, U=U)

    states, S = [], S0.copy()
    for n in range(NC):
        states.append(S)
        f = chunk(n, S)
        S = (np.exp(f["gam"]).astype(dt)[:, None] * S + f["Ktil"].T @ f["U"]).astype(dt)

    out = {x: np.zeros(s, dt) for x, s in (("dq", q.shape), ("dk", k.shape), ("dv", v.shape), ("dg", g.shape),
                                           ("db", beta.shape))}
    dS = dSf.copy()
    for n in reversed(range(NC)):
        S = states[n]
        f = chunk(n, S)
        sl, kk, qq, G, bb = f["sl"], f["kk"], f["qq"], f["G"], f["bb"]
        dOc = dO[sl]
        dU = f["P"].T @ dOc + f["Ktil"] @ dS
        dR = f["T"].T @ dU
        dT = dU @ f["R"].T
        dA = np.tril(-(f["T"].T @ dT @ f["T"].T), -1)
        dP = np.tril(dOc @ f["U"].T)
        out["dv"][sl] = bb[:, None] * dR
        out["db"][sl] = (dR * f["E"]).sum(1) + (dA * f["X"]).sum(1)
        wa = bb[:, None] * dA
        # pair terms: t[r][j][c] = (wa k_r + wp q_r) k_j e^{G_r - G_j}
        t = (wa[:, :, None] * kk[:, None, :] + dP[:, :, None] * qq[:, None, :]) * kk[None, :, :] * f["e"]
        dkc = np.einsum("rj,jc,rjc->rc", wa, kk, f["e"]) + np.einsum("rj,rc,rjc->jc", wa, kk, f["e"]) \
            + np.einsum("rj,rc,rjc->jc", dP, qq, f["e"])
        dqc = np.einsum("rj,jc,rjc->rc", dP, kk, f["e"])
        dG = t.sum(1) - t.sum(0)
        eg, et = np.exp(G).astype(dt), np.exp(f["gam"] - G).astype(dt)
        dQbar, dKbar, dKtil = dOc @ S.T, -bb[:, None] * (dR @ S.T), f["U"] @ dS.T
        dqc = dqc + dQbar * eg
        dkc = dkc + dKbar * eg + dKtil * et
        dG = dG + dQbar * qq * eg + dKbar * kk * eg
        kt = dKtil * kk * et                                     # the Ktil share, summed over earlier rows
        before = np.concatenate([np.zeros((1, dk), dt), np.cumsum(kt, axis=0, dtype=dt)[:-1]])
        after = np.cumsum(dG[::-1], axis=0, dtype=dt)[::-1]
        out["dg"][sl] = np.exp(f["gam"]).astype(dt) * (dS * S).sum(1) + before + after
        out["dq"][sl], out["dk"][sl] = dqc, dkc
        dS = (np.exp(f["gam"]).astype(dt)[:, None] * dS + f["Qbar"].T @ dOc - f["Kbar"].T @ (bb[:, None] * dR)).astype(dt)
    f64 = lambda x: x[:T].astype(np.float64)
    return (f64(out["dq"]), f64(out["dk"]), f64(out["dv"]), f64(out["dg"][:T] * gd), f64(out["db"]),
            dS.astype(np.float64))


def _case(wl, seed):
    inp = gen.make_numpy(wl, seed)
    cot = gen.make_cotangents(wl, seed)
    f = gen.all_to_f64(inp)
    ref = orc.kda_backward(f["q"], f["k"], f["v"], f["w"], f["beta"], f["S0"], wl.g_min,
                           cot["dO"].astype(np.float64), cot["dSf"].astype(np.float64), nthreads=1)
    args = [f[x][0, 0] for x in ("q", "k", "v", "w", "beta", "S0")] + [cot["dO"][0, 0].astype(np.float64),
                                                                       cot["dSf"][0, 0].astype(np.float64)]
    return args, [r[0, 0] for r in ref]


def _rel(x, r):
    return float(np.max(np.abs(x - r)) / np.max(np.abs(r)))


BASE = gen.WORKLOADS["tiny_f32"].with_(B=1, H=1, T=70, dk=32, dv=32, s0_sd=0.5)


@pytest.mark.parametrize("g_min,w_mu", [(-5.0, 0.0), (-8.0, 4.0), (-float("inf"), 3.0), (0.0, 0.0)])
def test_float64_chunk_form_equals_token_adjoint(g_min, w_mu):
    """Bounded, strongly decaying, unbounded and zero gates, ragged last chunk: every gradient of the
    chunk form agrees with the adjoint of the token recurrence to rounding."""
    wl = BASE.with_(g_min=g_min, w_mu=w_mu, w_sd=1.0)
    args, ref = _case(wl, 11)
    got = chunk_backward(*args, wl.g_min, np.float64)
    for name, x, r in zip(("dq", "dk", "dv", "dw", "dbeta", "dS0"), got, ref):
        if np.max(np.abs(r)) == 0:
            assert np.max(np.abs(x)) < 1e-12, name
        else:
            assert _rel(x, r) < 1e-10, name


def test_float32_rounding_of_dw_under_strong_decay():
    """g_min = -8 with every chunk's span near -126: the chunk form's own fp32 rounding of dw stays
    below 1e-4 of its largest entry (the GPU test's bound for this regime), and in a moderate regime
    below 2e-5 (the general bound)."""
    wl = gen.WORKLOADS["tiny_f32"].with_(B=1, H=1, T=150, dk=64, dv=64, g_min=-8.0, w_mu=4.0, w_sd=1.0, s0_sd=0.5)
    args, ref = _case(wl, 455)
    e_strong = _rel(chunk_backward(*args, wl.g_min, np.float32)[3], ref[3])
    wl2 = wl.with_(w_mu=1.0)
    args2, ref2 = _case(wl2, 455)
    e_mod = _rel(chunk_backward(*args2, wl2.g_min, np.float32)[3], ref2[3])
    assert e_strong < 1e-4 and e_mod < 2e-5, (e_strong, e_mod)
