"""Pins for the fp64 oracle, each checked against something other than the oracle itself.

Every check here is independent of the oracle's own loop structure: a dense
product-of-transitions form, closed forms of special cases, invariants of the
delta rule, the constants the pages print, and mutation runs that plant a
mistake in a private copy of the oracle source and require a pin to catch it.
"""
import math
import os
import subprocess
import ctypes

import numpy as np
import pytest

from oracle import oracle as orc
from chunked_gated_delta_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "printed_constants.txt")


# ---------------------------------------------------------------- helpers (independent of the oracle)

def np_gate(w, g_min):
    """Gate written directly from its definition, for the brute-force forms only."""
    w = np.asarray(w, np.float64)
    if math.isinf(g_min):
        return -(np.maximum(w, 0.0) + np.log1p(np.exp(-np.abs(w))))
    return g_min / (1.0 + np.exp(-w))


def rand_case(T, dk, dv, seed, w_mu=0.0, w_sd=2.0, s0=True, beta=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal(T))) if beta is None else np.full(T, float(beta))
    w = rng.normal(w_mu, w_sd, (T, dk))
    S0 = rng.standard_normal((dk, dv)) * 0.5 if s0 else None
    return q, k, v, w, b, S0


def run1(q, k, v, w, b, S0, g_min=-5.0):
    """Oracle on one (b,h): 2-D inputs in, 2-D outputs back."""
    o, S = orc.kda_reference(q[None, None], k[None, None], v[None, None], w[None, None],
                             b[None, None], None if S0 is None else S0[None, None], g_min, nthreads=1)
    return o[0, 0], S[0, 0]


def brute_quadratic(q, k, v, w, b, S0, g_min):
    """o_t = sum_{j<=t} b_j (q_t^T A_t...A_{j+1} k_j) v_j + q_t^T A_t...A_1 S0,
    A_s = (I - b_s k_s k_s^T) Diag(e^{g_s}); S_T = A_T...A_1 S0 + sum_j A_T...A_{j+1} b_j k_j v_j^T.
    Dense products of transition matrices, no recurrence."""
    T, dk = q.shape
    dv = v.shape[1]
    g = np_gate(w, g_min)
    A = [(np.eye(dk) - b[s] * np.outer(k[s], k[s])) @ np.diag(np.exp(g[s])) for s in range(T)]
    S0 = np.zeros((dk, dv)) if S0 is None else S0
    o = np.zeros((T, dv))
    for t in range(T):
        M = np.eye(dk)
        for j in range(t, -1, -1):
            o[t] += b[j] * (q[t] @ M @ k[j]) * v[j]
            M = M @ A[j]
        o[t] += q[t] @ M @ S0
    M = np.eye(dk)
    S = np.zeros((dk, dv))
    for j in range(T - 1, -1, -1):
        S += b[j] * np.outer(M @ k[j], v[j])
        M = M @ A[j]
    S += M @ S0
    return o, S


def rel(x, ref):
    return np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300)


# ---------------------------------------------------------------- whole recurrence

@pytest.mark.parametrize("T,dk,dv,seed,g_min", [
    (1, 4, 3, 0, -5.0), (17, 8, 5, 1, -5.0), (40, 6, 6, 2, -5.0),
    (33, 5, 7, 3, -math.inf), (24, 8, 4, 4, -1.0), (20, 3, 9, 5, 0.0)])
def test_brute_force_quadratic_form(T, dk, dv, seed, g_min):
    q, k, v, w, b, S0 = rand_case(T, dk, dv, seed, w_mu=1.0 if math.isinf(g_min) else 0.0)
    o, S = run1(q, k, v, w, b, S0, g_min)
    o_ref, S_ref = brute_quadratic(q, k, v, w, b, S0, g_min)
    assert rel(o, o_ref) < 1e-12
    assert rel(S, S_ref) < 1e-12


def test_brute_force_zero_state_ragged():
    q, k, v, w, b, _ = rand_case(37, 8, 8, 11, s0=False)
    o, S = run1(q, k, v, w, b, None)
    o_ref, S_ref = brute_quadratic(q, k, v, w, b, None, -5.0)
    assert rel(o, o_ref) < 1e-12 and rel(S, S_ref) < 1e-12


# ---------------------------------------------------------------- decay path: beta = 0 is gated linear attention with no writes

def test_beta_zero_closed_form():
    T, dk, dv = 50, 16, 8
    q, k, v, w, _, S0 = rand_case(T, dk, dv, 21, beta=0.0)
    b = np.zeros(T)
    o, S = run1(q, k, v, w, b, S0)
    G = np.cumsum(np_gate(w, -5.0), axis=0)            # global prefix, per key channel
    o_ref = np.stack([(q[t] * np.exp(G[t])) @ S0 for t in range(T)])
    S_ref = np.exp(G[-1])[:, None] * S0
    assert rel(o, o_ref) < 1e-13
    assert rel(S, S_ref) < 1e-13


# ---------------------------------------------------------------- write + decay: one-hot distinct keys (no erase) is closed-form GLA

def test_one_hot_keys_gla_closed_form():
    T, dk, dv = 24, 32, 6
    rng = np.random.default_rng(7)
    perm = rng.permutation(dk)[:T]
    k = np.zeros((T, dk)); k[np.arange(T), perm] = 1.0
    q = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    b = rng.uniform(0.1, 0.9, T)
    w = rng.normal(0.0, 2.0, (T, dk))
    o, S = run1(q, k, v, w, b, None)
    G = np.cumsum(np_gate(w, -5.0), axis=0)
    o_ref = np.zeros((T, dv))
    for t in range(T):
        for j in range(t + 1):
            c = perm[j]
            o_ref[t] += b[j] * q[t, c] * np.exp(G[t, c] - G[j, c]) * v[j]
    assert rel(o, o_ref) < 1e-13
    S_ref = np.zeros((dk, dv))
    for j in range(T):
        c = perm[j]
        S_ref[c] += b[j] * np.exp(G[-1, c] - G[j, c]) * v[j]
    assert rel(S, S_ref) < 1e-13


# ---------------------------------------------------------------- delta correction: retrieval invariant

def test_retrieval_invariant_beta_one():
    """beta_t = 1 and unit k_t: after the write, S_t^T k_t = v_t; reading with q = k returns v."""
    T, dk, dv = 64, 16, 8
    q, k, v, w, _, S0 = rand_case(T, dk, dv, 31)
    b = np.ones(T)
    o, _ = run1(k, k, v, w, b, S0)
    assert np.max(np.abs(o - v)) < 1e-12


def test_partial_retrieval_identity():
    """k_t^T S_t = (1 - beta_t) k_t^T Diag(e^{g_t}) S_{t-1} + beta_t v_t^T, with S_{t-1} from a prefix run."""
    T, dk, dv = 30, 8, 5
    q, k, v, w, b, S0 = rand_case(T, dk, dv, 41)
    g = np_gate(w, -5.0)
    for t in (0, 7, 29):
        if t == 0:
            S_prev = S0
        else:
            _, S_prev = run1(q[:t], k[:t], v[:t], w[:t], b[:t], S0)
        o, _ = run1(k[:t + 1], k[:t + 1], v[:t + 1], w[:t + 1], b[:t + 1], S0)
        lhs = o[t]
        rhs = (1 - b[t]) * ((k[t] * np.exp(g[t])) @ S_prev) + b[t] * v[t]
        assert np.max(np.abs(lhs - rhs)) < 1e-12


# ---------------------------------------------------------------- textbook reduction: dk = 1 is a first-order time-varying recurrence

def test_scalar_key_product_form():
    T, dv = 45, 4
    rng = np.random.default_rng(5)
    ks = rng.choice([-1.0, 1.0], T)
    qs = rng.standard_normal(T)
    v = rng.standard_normal((T, dv))
    b = rng.uniform(0, 1, T)
    w = rng.normal(0, 2, T)
    S0 = rng.standard_normal((1, dv))
    o, S = run1(qs[:, None], ks[:, None], v, w[:, None], b, S0)
    a = (1 - b) * np.exp(np_gate(w, -5.0))   # S_t = a_t S_{t-1} + b_t k_t v_t
    o_ref = np.zeros((T, dv))
    for t in range(T):
        s = np.prod(a[:t + 1]) * S0[0]
        for j in range(t + 1):
            s = s + np.prod(a[j + 1:t + 1]) * b[j] * ks[j] * v[j]
        o_ref[t] = qs[t] * s
    assert rel(o, o_ref) < 1e-13
    assert rel(S[0], o_ref[-1] / qs[-1]) < 1e-12


# ---------------------------------------------------------------- state carry and linearity

def test_chaining_bitwise():
    T, dk, dv = 70, 8, 8
    q, k, v, w, b, S0 = rand_case(T, dk, dv, 51)
    o, S = run1(q, k, v, w, b, S0)
    for T1 in (16, 33):
        o1, S1 = run1(q[:T1], k[:T1], v[:T1], w[:T1], b[:T1], S0)
        o2, S2 = run1(q[T1:], k[T1:], v[T1:], w[T1:], b[T1:], S1)
        assert np.array_equal(np.concatenate([o1, o2]), o)
        assert np.array_equal(S2, S)


def test_linearity_in_state_and_values():
    T, dk, dv = 40, 8, 6
    q, k, v, w, b, S0 = rand_case(T, dk, dv, 61)
    o, S = run1(q, k, v, w, b, S0)
    oa, Sa = run1(q, k, v, w, b, None)
    ob, Sb = run1(q, k, np.zeros_like(v), w, b, S0)
    assert rel(o, oa + ob) < 1e-13
    assert rel(S, Sa + Sb) < 1e-13


def test_state_norm_growth_bound():
    """For beta in [0,1], unit k and g <= 0 the transition is a contraction, so
    ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t|| ("From Numerical Stability ..." section 2.3
    asks for the state-matrix norm to stay stable on long inputs)."""
    T, dk, dv = 48, 8, 8
    q, k, v, w, b, S0 = rand_case(T, dk, dv, 71)
    prev = np.linalg.norm(S0)
    for t in range(1, T + 1):
        _, S = run1(q[:t], k[:t], v[:t], w[:t], b[:t], S0)
        cur = np.linalg.norm(S)
        assert cur <= prev + b[t - 1] * np.linalg.norm(v[t - 1]) + 1e-12
        prev = cur


# ---------------------------------------------------------------- gate and printed constants

def _golden():
    rows = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, val, tol, _src = [x.strip() for x in line.split("|", 3)]
        rows[name] = (float(val), float(tol))
    return rows


def close(x, printed, tol):
    return abs(x - printed) <= tol * abs(printed) if tol > 0 else x == printed


def test_printed_constants_from_gate():
    gold = _golden()
    g_min = -5.0
    g_sat = orc.gate([1e4], g_min)[0]              # sigmoid saturates: g reaches g_min
    assert g_sat == -5.0
    assert close(math.exp(g_sat), *gold["step_decay_lower"])
    span16 = float(np.sum(orc.gate(np.full(16, 1e4), g_min)))
    assert close(span16, *gold["tile_span_16"])
    assert close(math.exp(-span16), *gold["exp_plus_80"])
    assert close(math.exp(span16), *gold["exp_minus_80"])
    assert math.exp(-span16) < gold["normal_max"][0]
    smallest_normal = float(np.finfo(np.float32).tiny)  # bf16 shares fp32's exponent range
    orders = math.log10(math.exp(span16) / smallest_normal)
    assert close(orders, *gold["bf16_headroom_orders"])
    span15 = float(np.sum(orc.gate(np.full(15, 1e4), g_min)))
    assert close(-span15, *gold["reciprocal_15_steps_log"])
    assert 1.0 - math.exp(g_sat) > gold["forgetting_at_gmin"][0]
    # the unbounded example: a step of -40 repeated over 16 tokens
    w40 = 40.0  # softplus(40) = 40 up to 4e-18
    g40 = orc.gate([w40], -math.inf)[0]
    assert close(round(g40), *gold["unbounded_step"])
    span_unb = float(np.sum(orc.gate(np.full(16, w40), -math.inf)))
    assert close(round(span_unb), *gold["unbounded_chunk_log"])
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(np.exp(-span_unb)))   # reciprocal overflows in fp32/bf16


def test_gate_special_values():
    assert orc.gate([0.0], -5.0)[0] == -2.5                 # sigmoid(0) = 1/2
    assert orc.gate([0.0], -math.inf)[0] == pytest.approx(-math.log(2.0), abs=1e-16)
    assert orc.gate([-1e4], -5.0)[0] == 0.0 or orc.gate([-1e4], -5.0)[0] > -1e-300
    x = np.linspace(-30, 30, 121)
    gb = orc.gate(x, -5.0)
    assert np.all(gb <= 0) and np.all(gb >= -5.0)
    assert np.all(np.diff(gb) <= 0)                          # more gate input -> more decay
    gu = orc.gate(x, -math.inf)
    assert np.all(gu < 0) and np.all(np.diff(gu) < 0)
    # the unbounded gate is not bounded below; the bounded one never passes g_min
    assert orc.gate([100.0], -math.inf)[0] < -99.0
    # symmetry of the logistic function: g(w) + g(-w) = g_min
    assert np.max(np.abs(orc.gate(x, -5.0) + orc.gate(-x, -5.0) + 5.0)) < 1e-14


@pytest.mark.parametrize("name", ["tiny_f32", "bf16_4k", "decay_stress", "million", "headline"])
def test_gate_range_and_span_on_bounded_workloads(name):
    """g stays in (-5, 0) and every 16-token span stays at or above -80 on sampled
    inputs of each bounded workload (sampled: one head, first 2048 tokens)."""
    wl = gen.WORKLOADS[name]
    small = wl.with_(B=1, H=1, T=min(wl.T, 2048))
    inp = gen.make_numpy(small, seed=0)
    g = orc.gate(inp["w"].astype(np.float64), wl.g_min)
    assert np.all(g < 0.0) and np.all(g > -5.0)
    spans = orc.chunk_spans(inp["w"], wl.g_min, 16)
    assert np.all(spans >= -80.0)
    if name == "decay_stress":                      # spans approach the bound
        assert spans.min() < -79.5


def test_unbounded_workload_flags_a_large_share_of_chunks():
    wl = gen.WORKLOADS["unbounded"].with_(B=1, H=2, T=4096)
    inp = gen.make_numpy(wl, seed=0)
    flags = orc.predicted_flags(inp["w"], wl.g_min, 16)
    frac = flags.mean()
    assert 0.45 < frac < 0.70, frac
    spans = orc.chunk_spans(inp["w"], wl.g_min, 16)
    assert spans.min() < -88.8                     # some chunks really overflow fp32 reciprocals


def test_spans_match_definition_on_ragged_tail():
    rng = np.random.default_rng(3)
    w = rng.normal(0, 2, (1, 2, 37, 5))
    spans = orc.chunk_spans(w, -5.0, 16)
    g = np_gate(w, -5.0)
    assert spans.shape == (1, 2, 3)
    for h in range(2):
        for n in range(3):
            ref = g[0, h, 16 * n:16 * (n + 1)].sum(axis=0).min()
            assert abs(spans[0, h, n] - ref) < 1e-13


def test_multithreaded_equals_single_threaded():
    wl = gen.WORKLOADS["bf16_4k"].with_(B=2, H=3, T=80, dk=16, dv=8)
    inp = gen.make_numpy(wl.with_(s0_sd=0.1), seed=1)
    args = [inp[x].astype(np.float64) for x in ("q", "k", "v", "w", "beta")]
    o1, S1 = orc.kda_reference(*args, S0=inp["S0"], nthreads=1)
    o4, S4 = orc.kda_reference(*args, S0=inp["S0"], nthreads=4)
    assert np.array_equal(o1, o4) and np.array_equal(S1, S4)
    for b in range(2):
        for h in range(3):
            o, S = run1(*(a[b, h] for a in args), inp["S0"][b, h].astype(np.float64))
            assert np.array_equal(o, o1[b, h]) and np.array_equal(S, S1[b, h])


def test_empty_sequence_returns_initial_state():
    S0 = np.random.default_rng(0).standard_normal((1, 1, 4, 3))
    z = np.zeros((1, 1, 0, 4))
    o, S = orc.kda_reference(z, z, np.zeros((1, 1, 0, 3)), z, np.zeros((1, 1, 0)), S0)
    assert o.shape == (1, 1, 0, 3) and np.array_equal(S, S0)


# ---------------------------------------------------------------- mutation runs: plant a mistake in a copy of the oracle

MUTATIONS = {
    "erase_sign": ("u[j] = beta[t] * (vt[j] - kS[j]);", "u[j] = beta[t] * (vt[j] + kS[j]);"),
    "no_beta_on_v": ("u[j] = beta[t] * (vt[j] - kS[j]);", "u[j] = vt[j] - beta[t] * kS[j];"),
    "gate_sign": ("return g_min * sigmoid(w);", "return g_min * sigmoid(-w);"),
    "decay_exp_missing": ("double d = exp(g[c]);", "double d = 1.0 + g[c];"),
    "read_uses_k": ("const double qc = qt[c];", "const double qc = kt[c];"),
    "write_transposed_index": ("row[j] += kc * u[j];", "row[j] += kt[j % dk] * u[c % dv];"),
}


def _build_mutant(tmp_path, name):
    src = open(os.path.join(os.path.dirname(orc.__file__), "kda_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, name
    path = tmp_path / f"mut_{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"mut_{name}.so"
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-o", str(so), str(path), "-lm", "-lpthread"])
    lib = ctypes.CDLL(str(so))
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.kda_oracle_f64.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.c_double, i64, i64, i64, i64, i64, dp, dp, ctypes.c_int]
    return lib


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(tmp_path, name):
    lib = _build_mutant(tmp_path, name)
    T, dk, dv = 20, 6, 6
    q, k, v, w, b, S0 = rand_case(T, dk, dv, 99)
    arrs = [np.ascontiguousarray(x, np.float64) for x in (q, k, v, w, b, S0)]
    o = np.empty((T, dv))
    S = np.empty((dk, dv))
    ptr = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    rc = lib.kda_oracle_f64(*[ptr(a) for a in arrs], -5.0, 1, 1, T, dk, dv, ptr(o), ptr(S), 1)
    assert rc == 0
    o_ref, S_ref = brute_quadratic(q, k, v, w, b, S0, -5.0)
    assert rel(o, o_ref) > 1e-6 or rel(S, S_ref) > 1e-6, f"pin failed to catch mutation {name}"


# ---------------------------------------------------------------- backward (adjoint) pins

def _fd_grads(args, g_min, dO, dSf, h=1e-6):
    """Central finite differences of <dO, o> + <dSf, S_final> with respect to every input."""
    def loss(a):
        o, S = orc.kda_reference(*a, g_min, nthreads=1)
        return float((o * dO).sum() + (S * dSf).sum())
    out = []
    for ai, x in enumerate(args):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            ap = [a.copy() for a in args]
            am = [a.copy() for a in args]
            ap[ai][idx] += h
            am[ai][idx] -= h
            fd[idx] = (loss(ap) - loss(am)) / (2 * h)
        out.append(fd)
    return out


def _bwd_case(seed, T=7, dk=4, dv=3):
    rng = np.random.default_rng(seed)
    q, k, w = (rng.normal(size=(1, 2, T, dk)) for _ in range(3))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(1, 2, T, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.normal(size=(1, 2, T))))
    S0 = 0.3 * rng.normal(size=(1, 2, dk, dv))
    dO = rng.normal(size=(1, 2, T, dv))
    dSf = rng.normal(size=(1, 2, dk, dv))
    return [q, k, v, w, beta, S0], dO, dSf


@pytest.mark.parametrize("g_min", [-5.0, -8.0, -math.inf, 0.0])
def test_backward_matches_finite_differences(g_min):
    """The adjoint recurrence against central differences of the forward oracle, every input."""
    args, dO, dSf = _bwd_case(7)
    grads = orc.kda_backward(*args, g_min, dO, dSf, nthreads=1)
    fds = _fd_grads(args, g_min, dO, dSf)
    for name, g, fd in zip(("q", "k", "v", "w", "beta", "S0"), grads, fds):
        scale = max(1e-12, np.max(np.abs(fd)))
        assert np.max(np.abs(g - fd)) / scale < 1e-6, name


def test_backward_closed_form_no_writes():
    """beta = 0 and a zero gate: o_t = S0^T q_t, so dq_t = S0 do_t, dS0 = sum_t q_t do_t^T + dSf, and
    dk = dv = dbeta = 0 except dbeta_t = do-weighted error, which the next pin covers."""
    rng = np.random.default_rng(3)
    T, dk, dv = 9, 5, 4
    q = rng.normal(size=(1, 1, T, dk))
    k = rng.normal(size=(1, 1, T, dk))
    v = rng.normal(size=(1, 1, T, dv))
    w = rng.normal(size=(1, 1, T, dk))
    beta = np.zeros((1, 1, T))
    S0 = rng.normal(size=(1, 1, dk, dv))
    dO = rng.normal(size=(1, 1, T, dv))
    dSf = rng.normal(size=(1, 1, dk, dv))
    dq, dk_, dv_, dw, db, dS0 = orc.kda_backward(q, k, v, w, beta, S0, 0.0, dO, dSf, nthreads=1)
    assert np.allclose(dq[0, 0], dO[0, 0] @ S0[0, 0].T, atol=1e-12)
    assert np.allclose(dS0[0, 0], q[0, 0].T @ dO[0, 0] + dSf[0, 0], atol=1e-12)
    assert np.allclose(dk_, 0.0) and np.allclose(dv_, 0.0) and np.allclose(dw, 0.0)
    # dbeta_t = (v_t - S0^T k_t) . (S0^T-side adjoint): with S constant, du_t = (dSf + sum_{t'>=t} q do^T)^T k_t
    dS = dSf[0, 0] + np.zeros_like(S0[0, 0])
    want = np.zeros(T)
    for t in range(T - 1, -1, -1):
        dS = dS + np.outer(q[0, 0, t], dO[0, 0, t])
        want[t] = (dS.T @ k[0, 0, t]) @ (v[0, 0, t] - S0[0, 0].T @ k[0, 0, t])
    assert np.allclose(db[0, 0], want, atol=1e-10)


BWD_MUTATIONS = {
    "read_adjoint_dropped": ("for (int64_t j = 0; j < dv; ++j) dS[c * dv + j] += qt[c] * dot[j];", ""),
    "erase_adjoint_sign": ("du[j] = -beta[t] * du[j];   /* z */", "du[j] = beta[t] * du[j];   /* z */"),
    "gate_derivative": ("return g_min * s * (1.0 - s);", "return g_min * s;"),
    "decay_adjoint_missing": ("dS[c * dv + j] *= eg[c];", "dS[c * dv + j] *= 1.0;"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_backward_planted_mistakes_are_caught(tmp_path, name):
    src = open(os.path.join(os.path.dirname(orc.__file__), "kda_oracle.c")).read()
    old, new = BWD_MUTATIONS[name]
    assert src.count(old) == 1, name
    path = tmp_path / f"bmut_{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"bmut_{name}.so"
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-o", str(so), str(path), "-lm", "-lpthread"])
    lib = ctypes.CDLL(str(so))
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.kda_oracle_bwd_f64.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.c_double, i64, i64, i64, i64, i64,
                                       dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
    args, dO, dSf = _bwd_case(11)
    B, H, T, dk = args[0].shape
    dv = args[2].shape[-1]
    outs = [np.zeros((B, H, T, dk)), np.zeros((B, H, T, dk)), np.zeros((B, H, T, dv)), np.zeros((B, H, T, dk)),
            np.zeros((B, H, T)), np.zeros((B, H, dk, dv))]
    ptr = lambda a: np.ascontiguousarray(a).ctypes.data_as(dp)
    arrs = [np.ascontiguousarray(a, np.float64) for a in args]
    rc = lib.kda_oracle_bwd_f64(*[ptr(a) for a in arrs], -5.0, B, H, T, dk, dv, ptr(dO), ptr(dSf),
                                *[ptr(o) for o in outs], 1)
    assert rc == 0
    fds = _fd_grads(args, -5.0, dO, dSf)
    worst = max(np.max(np.abs(g - fd)) / max(1e-12, np.max(np.abs(fd))) for g, fd in zip(outs, fds))
    assert worst > 1e-4, f"finite differences failed to catch backward mutation {name}"
