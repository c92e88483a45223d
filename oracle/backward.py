"""fp64 CPU oracle for the gradients of the Kimi Delta Attention forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the CPU-baseline leg of
``bench.py``, never by the product package. It shares no code with the HIP
library.

The FlashKDA pages show only the forward call ("Core Kernel API / flash_kda.fwd",
ccm-staging page) and recommend inference mode ("Kernel API and Constraints",
trend.ondo.sh page); they define no backward. The gradients here are the plain
derivatives of the forward this project reads from those pages (the recurrence
documented in ``oracle/__init__.py``), taken in reverse mode through the
per-token recurrence:

    q^ = q / sqrt(|q|^2 + 1e-6),   k^ = k / sqrt(|k|^2 + 1e-6)
    log a = max(-exp(A_log[h]) * softplus(g + dt_bias[h]), lower_bound)
    X_t = Diag(a_t) S_{t-1},   u_t = v_t - X_t^T k^_t,   S_t = X_t + beta_t k^_t u_t^T
    o_t = scale * S_t^T q^_t

for the scalar L = <dout, out> + <dfinal, final_state>. The clamp takes the
unclamped branch on ties (gradient through the rate) and passes no gradient
where the rate lies strictly below lower_bound.

Pinned by tests/test_oracle_backward.py: central differences of the C
recurrence (an independent forward), and closed forms for one token and for
a frozen state.
"""
from __future__ import annotations

import numpy as np

from . import _as_f64, _sequences


def _norm_rows(x):
    """Row-wise q / sqrt(|q|^2 + 1e-6); returns (normalised rows, norms)."""
    n = np.sqrt(np.sum(x * x, axis=-1) + 1e-6)
    return x / n[:, None], n


def _norm_rows_grad(xn, n, dxn):
    """Gradient through x -> x / n(x), n = sqrt(|x|^2 + eps): (dxn - xn (xn . dxn)) / n."""
    return (dxn - xn * np.sum(xn * dxn, axis=-1, keepdims=True)) / n[:, None]


def bwd(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, dout,
        initial_state=None, dfinal=None, cu_seqlens=None):
    """Reverse-mode gradients of L = <dout, out> + <dfinal, final>.

    Inputs as for ``oracle.fwd`` (float64, or uint16 bf16 bit patterns) plus
    dout [B, T, H, V] and dfinal [N, H, K, V] (None = zero). Returns a dict
    with float64 arrays dq, dk, dg [B, T, H, K], dv [B, T, H, V],
    dbeta [B, T, H], dA_log [H], ddt_bias [H, K] and dinitial_state
    [N, H, K, V] (the gradient with respect to the initial state, zero
    initial state when None).
    """
    q, k, v, g, beta, dout = map(_as_f64, (q, k, v, g, beta, dout))
    B, T, H, K = q.shape
    V = v.shape[-1]
    BT = B * T
    qf, kf, gf = q.reshape(BT, H, K), k.reshape(BT, H, K), g.reshape(BT, H, K)
    vf, of, bf = v.reshape(BT, H, V), dout.reshape(BT, H, V), beta.reshape(BT, H)
    dtb = np.asarray(dt_bias, dtype=np.float64).reshape(H, K)
    alog = np.asarray(A_log, dtype=np.float64).reshape(H)
    lb = float(lower_bound)
    seqs = _sequences(B, T, cu_seqlens)
    N = len(seqs)
    init = _as_f64(initial_state)
    dfin = _as_f64(dfinal)

    dq = np.zeros((BT, H, K))
    dk = np.zeros((BT, H, K))
    dg = np.zeros((BT, H, K))
    dv = np.zeros((BT, H, V))
    dbeta = np.zeros((BT, H))
    dA_log = np.zeros(H)
    ddt = np.zeros((H, K))
    dinit = np.zeros((N, H, K, V))

    for n, bos, eos in seqs:
        L = eos - bos
        for h in range(H):
            qn, nq = _norm_rows(qf[bos:eos, h])
            kn, nk = _norm_rows(kf[bos:eos, h])
            x = gf[bos:eos, h] + dtb[h]
            rate = np.exp(alog[h])
            la_free = -rate * np.logaddexp(0.0, x)
            clamped = la_free < lb
            a = np.exp(np.where(clamped, lb, la_free))
            vv, bb, do = vf[bos:eos, h], bf[bos:eos, h], of[bos:eos, h]

            # forward, keeping every state
            states = np.empty((L + 1, K, V))
            states[0] = 0.0 if init is None else init[n, h]
            for t in range(L):
                X = a[t][:, None] * states[t]
                u = vv[t] - X.T @ kn[t]
                states[t + 1] = X + bb[t] * np.outer(kn[t], u)

            # reverse sweep
            dS = np.zeros((K, V)) if dfin is None else dfin[n, h].copy()
            dqn = np.zeros((L, K))
            dkn = np.zeros((L, K))
            dla = np.zeros((L, K))
            for t in range(L - 1, -1, -1):
                dS += scale * np.outer(qn[t], do[t])
                dqn[t] = scale * (states[t + 1] @ do[t])
                X = a[t][:, None] * states[t]
                u = vv[t] - X.T @ kn[t]
                dSu = dS @ u
                dbeta[bos + t, h] = kn[t] @ dSu
                du = bb[t] * (dS.T @ kn[t])
                dv[bos + t, h] = du
                dkn[t] = bb[t] * dSu - X @ du
                dX = dS - np.outer(kn[t], du)
                dla[t] = a[t] * np.sum(dX * states[t], axis=1)
                dS = a[t][:, None] * dX
            dinit[n, h] = dS

            # gate: d la / d x = -rate * sigmoid(x), d la / d A_log = la
            dla_free = np.where(clamped, 0.0, dla)
            sig = 0.5 * (1.0 + np.tanh(0.5 * x))
            dx = dla_free * (-rate) * sig
            dg[bos:eos, h] = dx
            ddt[h] += dx.sum(axis=0)
            dA_log[h] += np.sum(dla_free * la_free)

            dq[bos:eos, h] = _norm_rows_grad(qn, nq, dqn)
            dk[bos:eos, h] = _norm_rows_grad(kn, nk, dkn)

    return dict(dq=dq.reshape(B, T, H, K), dk=dk.reshape(B, T, H, K),
                dv=dv.reshape(B, T, H, V), dg=dg.reshape(B, T, H, K),
                dbeta=dbeta.reshape(B, T, H), dA_log=dA_log, ddt_bias=ddt,
                dinitial_state=dinit)


def clamp_margin(g, dt_bias, A_log, lower_bound):
    """Smallest |rate term - lower_bound| over all elements, in fp64.

    Where this is tiny, fp32 and fp64 evaluations of the clamp may take
    different branches; tests mask such elements.
    """
    g = _as_f64(g)
    H, K = g.shape[-2], g.shape[-1]
    x = g + np.asarray(dt_bias, dtype=np.float64).reshape(H, K)
    la = -np.exp(np.asarray(A_log, dtype=np.float64).reshape(H))[:, None] * np.logaddexp(0.0, x)
    return np.abs(la - float(lower_bound))
