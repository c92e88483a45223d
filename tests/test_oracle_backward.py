"""Pins of the fp64 backward oracle (CPU only).

The pages define no backward, so the gradients are pinned to what the
mathematics fixes:
  B1  central differences of the C recurrence (an independent forward),
      along random directions for every input, fixed-length and packed;
  B2  one token from a zero state: closed forms of every gradient;
  B3  a frozen state (beta = 0): closed forms in cumulative decay products,
      including the gate parameters;
  B4  clamped elements pass no gradient to g, dt_bias or A_log.
tests/test_oracle_mutants.py plants mistakes in the backward and checks that
one of these fails.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as obwd


def rand_case(rng, B, T, H, K, V, lb=-4.0, N=None, state=True, dfinal=True):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    g = rng.standard_normal((B, T, H, K))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    A_log = np.log(rng.uniform(0.5, 4.0, H))
    dt_bias = 0.3 * rng.standard_normal((H, K))
    Nn = N or B
    init = 0.3 * rng.standard_normal((Nn, H, K, V)) if state else None
    dout = rng.standard_normal((B, T, H, V))
    dfin = rng.standard_normal((Nn, H, K, V)) if dfinal else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, scale=K ** -0.5, A_log=A_log,
                dt_bias=dt_bias, lower_bound=lb, initial_state=init, dout=dout,
                dfinal=dfin, cu_seqlens=None)


def loss(d):
    """L = <dout, out> + <dfinal, final> through the C recurrence (fp64)."""
    o, f = oracle.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["A_log"],
                      d["dt_bias"], d["lower_bound"], initial_state=d["initial_state"],
                      cu_seqlens=d["cu_seqlens"], nthreads=1)
    val = float(np.sum(o * d["dout"]))
    if d["dfinal"] is not None:
        val += float(np.sum(f * d["dfinal"]))
    return val


def grads(d, impl=None):
    impl = impl or obwd
    return impl.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["A_log"],
                    d["dt_bias"], d["lower_bound"], d["dout"], initial_state=d["initial_state"],
                    dfinal=d["dfinal"], cu_seqlens=d["cu_seqlens"])


WRT = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
       ("A_log", "dA_log"), ("dt_bias", "ddt_bias"), ("initial_state", "dinitial_state")]


def check_fd(d, impl=None, h=1e-5, tol=1e-6, seed=0):
    """Directional central differences for every input against the gradients."""
    gr = grads(d, impl)
    rng = np.random.default_rng(seed)
    margin = obwd.clamp_margin(d["g"], d["dt_bias"], d["A_log"], d["lower_bound"]).min()
    assert margin > 100 * h, "a rate term sits on the clamp; pick another seed"
    for name, gname in WRT:
        x = d[name]
        if x is None:
            continue
        dirn = rng.standard_normal(np.shape(x))
        dp, dm = dict(d), dict(d)
        dp[name] = x + h * dirn
        dm[name] = x - h * dirn
        fd = (loss(dp) - loss(dm)) / (2 * h)
        an = float(np.sum(gr[gname] * dirn))
        assert abs(fd - an) <= tol * max(1.0, abs(fd)), (name, fd, an)


# B1: central differences, fixed-length batch with states
@pytest.mark.parametrize("K,V,T,H,B", [(8, 8, 7, 2, 2), (16, 12, 13, 1, 1)])
def test_b1_finite_differences(K, V, T, H, B):
    d = rand_case(np.random.default_rng(11), B, T, H, K, V)
    check_fd(d)


def test_b1_finite_differences_packed():
    rng = np.random.default_rng(12)
    d = rand_case(rng, 1, 17, 2, 8, 8, N=3)
    d["cu_seqlens"] = np.array([0, 5, 5, 17], dtype=np.int32)   # an empty sequence too
    check_fd(d)


def test_b1_finite_differences_no_states():
    d = rand_case(np.random.default_rng(13), 1, 9, 1, 8, 8, state=False, dfinal=False)
    check_fd(d)


# B2: one token from a zero state: o = scale beta (k^.q^) v, final = beta k^ v^T
def test_b2_one_token_closed_form():
    rng = np.random.default_rng(21)
    K = V = 16
    d = rand_case(rng, 1, 1, 1, K, V, state=False)
    q, k, v = d["q"][0, 0, 0], d["k"][0, 0, 0], d["v"][0, 0, 0]
    b, s, do, dF = d["beta"][0, 0, 0], d["scale"], d["dout"][0, 0, 0], d["dfinal"][0, 0]
    nq, nk = np.sqrt(q @ q + 1e-6), np.sqrt(k @ k + 1e-6)
    qh, kh = q / nq, k / nk
    c = kh @ qh
    vdo = v @ do
    # L = s b c (v.do) + b kh^T dF v
    dv = s * b * c * do + b * (dF.T @ kh)
    dbeta = s * c * vdo + kh @ dF @ v
    dqh = s * b * vdo * kh
    dkh = s * b * vdo * qh + b * (dF @ v)
    dq = dqh / nq - q * (q @ dqh) / nq ** 3
    dk = dkh / nk - k * (k @ dkh) / nk ** 3
    gr = grads(d)
    np.testing.assert_allclose(gr["dv"][0, 0, 0], dv, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gr["dbeta"][0, 0, 0], dbeta, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gr["dq"][0, 0, 0], dq, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(gr["dk"][0, 0, 0], dk, rtol=1e-11, atol=1e-13)
    # a zero state makes the output independent of the decay
    assert np.all(gr["dg"] == 0) and np.all(gr["dA_log"] == 0) and np.all(gr["ddt_bias"] == 0)
    np.testing.assert_allclose(gr["dinitial_state"][0, 0],
                               np.exp(-np.exp(d["A_log"][0]) * np.logaddexp(0, d["g"][0, 0, 0] + d["dt_bias"][0]))[:, None]
                               * (dF - b * np.outer(kh, kh @ dF) + s * np.outer(qh, do) - s * b * np.outer(kh, c * do)),
                               rtol=1e-11, atol=1e-13)


# B3: beta = 0 freezes the state up to decay: S_t = Diag(P_t) S_0, P_t = prod_{s<=t} a_s
def test_b3_frozen_state_closed_form():
    rng = np.random.default_rng(31)
    K, V, T = 8, 6, 11
    d = rand_case(rng, 1, T, 1, K, V, lb=-0.7)
    d["beta"] = np.zeros_like(d["beta"])
    gr = grads(d)
    S0, dF, s = d["initial_state"][0, 0], d["dfinal"][0, 0], d["scale"]
    q = d["q"][0, :, 0]
    qh = q / np.sqrt(np.sum(q * q, -1, keepdims=True) + 1e-6)
    do = d["dout"][0, :, 0]
    x = d["g"][0, :, 0] + d["dt_bias"][0]
    rate = np.exp(d["A_log"][0])
    free = -rate * np.logaddexp(0, x)
    la = np.maximum(free, d["lower_bound"])
    P = np.exp(np.cumsum(la, axis=0))                       # [T, K]
    # dS_0 = sum_t s Diag(P_t) q^_t do_t^T + Diag(P_T) dF
    dS0 = s * np.einsum("tk,tk,tv->kv", P, qh, do) + P[-1][:, None] * dF
    np.testing.assert_allclose(gr["dinitial_state"][0, 0], dS0, rtol=1e-11, atol=1e-13)
    # dL/d la_{t,c} = sum_{r>=t} s q^_{r,c} P_{r,c} (S_0 do_r)_c + P_{T,c} (S_0 . dF)_c
    per_r = s * qh * P * (do @ S0.T)                        # [T, K]
    dla = np.cumsum(per_r[::-1], axis=0)[::-1] + (P[-1] * np.sum(S0 * dF, axis=1))[None, :]
    dla = np.where(free < d["lower_bound"], 0.0, dla)
    sig = 1.0 / (1.0 + np.exp(-x))
    np.testing.assert_allclose(gr["dg"][0, :, 0], dla * (-rate) * sig, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(gr["ddt_bias"][0], np.sum(dla * (-rate) * sig, 0), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(gr["dA_log"][0], np.sum(dla * free), rtol=1e-10, atol=1e-13)
    # beta = 0: the key and the value never reach the output
    assert np.abs(gr["dk"]).max() == 0 and np.abs(gr["dv"]).max() == 0
    # dbeta_t = k^_t^T dS_t u_t with u_t = v_t - (Diag(P_t) S_0)^T k^_t
    k = d["k"][0, :, 0]
    kh = k / np.sqrt(np.sum(k * k, -1, keepdims=True) + 1e-6)
    v = d["v"][0, :, 0]
    for t in range(T):
        dSt = sum(s * np.outer(qh[r] * P[r] / P[t], do[r]) for r in range(t, T)) + (P[-1] / P[t])[:, None] * dF
        u = v[t] - (P[t][:, None] * S0).T @ kh[t]
        np.testing.assert_allclose(gr["dbeta"][0, t, 0], kh[t] @ dSt @ u, rtol=1e-10, atol=1e-12)


# B4: an element whose rate term is below lower_bound passes no gate gradient
def test_b4_clamp_blocks_gate_gradient():
    rng = np.random.default_rng(41)
    d = rand_case(rng, 1, 10, 2, 8, 8, lb=-1.0)
    free = -np.exp(d["A_log"])[None, None, :, None] * np.logaddexp(0, d["g"] + d["dt_bias"][None, None])
    cl = free < d["lower_bound"]
    assert cl.any() and (~cl).any()
    gr = grads(d)
    assert np.all(gr["dg"][cl] == 0)
    assert np.abs(gr["dg"][~cl]).min() > 0
    # all elements clamped: no gradient reaches A_log or dt_bias
    d2 = dict(d, lower_bound=-1e-3)
    free2 = -np.exp(d2["A_log"])[None, None, :, None] * np.logaddexp(0, d2["g"] + d2["dt_bias"][None, None])
    assert np.all(free2 < d2["lower_bound"])
    gr2 = grads(d2)
    assert np.all(gr2["dg"] == 0) and np.all(gr2["dA_log"] == 0) and np.all(gr2["ddt_bias"] == 0)
    check_fd(d)
