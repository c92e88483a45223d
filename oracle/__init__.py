"""fp64 CPU oracle for the Kimi Delta Attention forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the product package. It shares
no code with the HIP library.

Contents
--------
``fwd``            ctypes wrapper of the C per-token recurrence (kda_oracle.c).
``brute_force``    numpy, literal K x K transition matrices, tiny inputs only.
``chunk_twin``     numpy fp64 chunkwise evaluation (WY/UT form) used to check the
                   chunk algebra the GPU kernels implement against the recurrence.
``gate_log_alpha`` numpy gate, written independently of the C code.

Pages: FlashKDA, "Kernel API and Constraints" (trend.ondo.sh page) and
"Core Kernel API / flash_kda.fwd" (ccm-staging page) give the call and its
constraints; the recurrence, the gate and the q/k normalisation are this
project's stated reading (the pages print no formula).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

F64, BF16, F32 = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2 -fopenmp, IEEE arithmetic)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.kda_oracle_fwd.restype = ctypes.c_int
        lib.kda_oracle_fwd.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_double, P,
                                       P, P, ctypes.c_double, P, ctypes.c_int, P,
                                       P, I64, I64, I64, I64, I64, I64, ctypes.c_int]
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def fwd(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound,
        initial_state=None, cu_seqlens=None, want_final=True, nthreads=0,
        state_is_bf16=None):
    """Run the fp64 per-token recurrence.

    q, k, g: [B, T, H, K]; v: [B, T, H, V]; beta: [B, T, H]. Either all float64,
    or all uint16 bf16 bit patterns. initial_state: [N, H, K, V] float64, float32
    or uint16 (bf16 bits) or None. Returns (out [B,T,H,V] f64, final [N,H,K,V]
    f64 or None).
    """
    lib = _load()
    q = np.ascontiguousarray(q)
    if q.dtype == np.uint16:
        dt = BF16
        conv = lambda a: np.ascontiguousarray(a, dtype=np.uint16)
    else:
        dt = F64
        conv = lambda a: np.ascontiguousarray(a, dtype=np.float64)
    q, k, v, g, beta = conv(q), conv(k), conv(v), conv(g), conv(beta)
    B, T, H, K = q.shape
    V = v.shape[-1]
    assert k.shape == (B, T, H, K) and g.shape == (B, T, H, K)
    assert v.shape == (B, T, H, V) and beta.shape == (B, T, H)
    A_log = np.ascontiguousarray(A_log, dtype=np.float64).reshape(H)
    dt_bias = np.ascontiguousarray(dt_bias, dtype=np.float64).reshape(H, K)
    cu = None
    N = B
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        N = len(cu) - 1
    sd = F64
    init = None
    if initial_state is not None:
        init = np.ascontiguousarray(initial_state)
        if init.dtype == np.uint16 or state_is_bf16:
            sd = BF16
            init = init.astype(np.uint16, copy=False)
        elif init.dtype == np.float32:
            sd = F32
        else:
            init = init.astype(np.float64, copy=False)
            sd = F64
        assert init.shape == (N, H, K, V)
    out = np.empty((B, T, H, V), dtype=np.float64)
    fin = np.empty((N, H, K, V), dtype=np.float64) if want_final else None
    rc = lib.kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), dt,
                            float(scale), _ptr(out), _ptr(A_log), _ptr(dt_bias),
                            float(lower_bound), _ptr(init), sd, _ptr(fin), _ptr(cu),
                            N if cu is not None else 0, B, T, H, K, V, int(nthreads))
    if rc != 0:
        raise ValueError("kda_oracle_fwd failed with code %d" % rc)
    return out, fin


def fwd_inputs(d: dict, nthreads: int = 0, want_final=None):
    """Oracle on a dict produced by ``kda_inputs`` (bf16 bit patterns)."""
    if want_final is None:
        want_final = d.get("final", False)
    return fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["A_log"],
               d["dt_bias"], d["lower_bound"], initial_state=d["initial_state"],
               cu_seqlens=d["cu_seqlens"], want_final=want_final, nthreads=nthreads,
               state_is_bf16=(d.get("state_dtype") == "bf16"))


# ---------------------------------------------------------------------------
# numpy references (independent of the C code)
# ---------------------------------------------------------------------------

def gate_log_alpha(g, dt_bias, A_log_h, lower_bound):
    """log alpha = max(-exp(A_log) * softplus(g + dt_bias), lower_bound).

    softplus via numpy's logaddexp(0, x) = ln(e^0 + e^x).
    """
    x = np.asarray(g, dtype=np.float64) + np.asarray(dt_bias, dtype=np.float64)
    return np.maximum(-np.exp(float(A_log_h)) * np.logaddexp(0.0, x), float(lower_bound))


def _l2n(x):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)


def _as_f64(a):
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _sequences(B, T, cu):
    if cu is None:
        return [(b, b * T, b * T + T) for b in range(B)]
    return [(n, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def brute_force(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound,
                initial_state=None, cu_seqlens=None):
    """Literal recurrence with explicit K x K matrices (tiny inputs only).

    S_t = (I - b k^ k^T) Diag(alpha_t) S_{t-1} + b k^ v^T ; o_t = scale S_t^T q^.
    """
    q, k, v, g, beta = map(_as_f64, (q, k, v, g, beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    qf = _l2n(q).reshape(B * T, H, K)
    kf = _l2n(k).reshape(B * T, H, K)
    vf = v.reshape(B * T, H, V)
    gf = g.reshape(B * T, H, K)
    bf = beta.reshape(B * T, H)
    seqs = _sequences(B, T, cu_seqlens)
    out = np.zeros((B * T, H, V))
    fin = np.zeros((len(seqs), H, K, V))
    init = _as_f64(initial_state)
    I = np.eye(K)
    for n, bos, eos in seqs:
        for h in range(H):
            S = np.zeros((K, V)) if init is None else init[n, h].copy()
            for t in range(bos, eos):
                la = gate_log_alpha(gf[t, h], np.asarray(dt_bias, dtype=np.float64).reshape(H, K)[h],
                                    np.asarray(A_log).reshape(H)[h], lower_bound)
                kk = kf[t, h]
                M = (I - bf[t, h] * np.outer(kk, kk)) @ np.diag(np.exp(la))
                S = M @ S + bf[t, h] * np.outer(kk, vf[t, h])
                out[t, h] = scale * S.T @ qf[t, h]
            fin[n, h] = S
    return out.reshape(B, T, H, V), fin


def chunk_twin(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound,
               initial_state=None, cu_seqlens=None, chunk=64, return_parts=False):
    """Chunkwise (WY/UT) evaluation of the same recurrence, fp64, numpy.

    Per chunk of L tokens with G = inclusive cumsum of log alpha inside the chunk:
      A_rj = b_r sum_c k_r k_j e^{G_r - G_j}  (j < r),  T = (I + A)^-1
      W = T diag(b) (K o e^G),  U = T diag(b) V,  D = U - W S
      P_rj = sum_c q_r k_j e^{G_r - G_j}  (j <= r)
      O = scale [(Q o e^G) S + P D]
      S <- diag(e^{G_L}) S + (K o e^{G_L - G})^T D
    Pairwise factors are formed directly as e^{G_r - G_j} (no factorisation).
    With return_parts, also returns a list of per-chunk dicts (sequence, head,
    start, W, U, P, Qt, Kt, gL) for inspection.
    """
    q, k, v, g, beta = map(_as_f64, (q, k, v, g, beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    qf = _l2n(q).reshape(B * T, H, K)
    kf = _l2n(k).reshape(B * T, H, K)
    vf = v.reshape(B * T, H, V)
    gf = g.reshape(B * T, H, K)
    bf = beta.reshape(B * T, H)
    dtb = np.asarray(dt_bias, dtype=np.float64).reshape(H, K)
    alog = np.asarray(A_log, dtype=np.float64).reshape(H)
    seqs = _sequences(B, T, cu_seqlens)
    out = np.zeros((B * T, H, V))
    fin = np.zeros((len(seqs), H, K, V))
    init = _as_f64(initial_state)
    parts = []
    for n, bos, eos in seqs:
        for h in range(H):
            S = np.zeros((K, V)) if init is None else init[n, h].copy()
            for c0 in range(bos, eos, chunk):
                c1 = min(c0 + chunk, eos)
                L = c1 - c0
                la = gate_log_alpha(gf[c0:c1, h], dtb[h], alog[h], lower_bound)
                G = np.cumsum(la, axis=0)
                Kc, Qc, Vc, bc = kf[c0:c1, h], qf[c0:c1, h], vf[c0:c1, h], bf[c0:c1, h]
                # pairwise decay e^{G_r - G_j} for j <= r only (the exponent is <= 0
                # there); pairs j > r get exponent -inf, i.e. factor 0
                causal = np.tril(np.ones((L, L), dtype=bool))
                E = np.exp(np.where(causal[:, :, None], G[:, None, :] - G[None, :, :], -np.inf))  # [L, L, K]
                strict = np.tril(np.ones((L, L), dtype=bool), -1)
                A = bc[:, None] * np.einsum("rc,jc,rjc->rj", Kc, Kc, np.where(strict[:, :, None], E, 0.0))
                Pm = np.einsum("rc,jc,rjc->rj", Qc, Kc, E)
                Tm = np.linalg.inv(np.eye(L) + A)
                W = Tm @ (bc[:, None] * Kc * np.exp(G))
                U = Tm @ (bc[:, None] * Vc)
                D = U - W @ S
                O = scale * ((Qc * np.exp(G)) @ S + Pm @ D)
                out[c0:c1, h] = O
                Kt = Kc * np.exp(G[-1][None, :] - G)
                if return_parts:
                    parts.append(dict(seq=n, head=h, start=c0, W=W, U=U, P=Pm,
                                      Qt=Qc * np.exp(G), Kt=Kt, gL=np.exp(G[-1]), S_in=S.copy()))
                S = np.exp(G[-1])[:, None] * S + Kt.T @ D
            fin[n, h] = S
    res = (out.reshape(B, T, H, V), fin)
    if return_parts:
        return res + (parts,)
    return res


# ---------------------------------------------------------------------------
# acceptance arithmetic (the tolerance bar: relative L2 and largest absolute
# error per tensor, plus a per-row relative error that no single wrong row of
# a large tensor can pass)
# ---------------------------------------------------------------------------

def rel_l2(x, ref):
    """||x - ref||_2 / ||ref||_2 over the whole tensor, in fp64 (||x||_2 if ref is 0)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    if den == 0.0:
        return float(np.linalg.norm(x.ravel()))
    return float(num / den)


def max_abs(x, ref):
    """max |x - ref| over the whole tensor, in fp64 (0 for empty tensors)."""
    return float(np.max(np.abs(np.asarray(x, dtype=np.float64) - np.asarray(ref, dtype=np.float64)))) if np.size(ref) else 0.0


def row_rel_l2(x, ref, row_ndim=1, floor=1.0):
    """Largest relative L2 error over rows, and the row where it occurs.

    A row is a slice over the trailing ``row_ndim`` axes (the 128 values of one
    token and head for ``out``; the K x V block of one sequence and head for a
    state). Row r's error is ||x_r - ref_r||_2 / max(||ref_r||_2, floor * R),
    where R is the root mean square of the reference row norms: a row is
    measured against its own norm, or against a typical row where cancellation
    has made its own norm small (the rounding error of a row follows the size of
    the operands that formed it, not the size of the result).
    Returns (error, flat row index); (0.0, -1) for empty tensors.
    """
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0, -1
    n = int(np.prod(ref.shape[ref.ndim - row_ndim:]))
    d = (x - ref).reshape(-1, n)
    r = ref.reshape(-1, n)
    dn = np.sqrt(np.sum(d * d, axis=1))
    rn = np.sqrt(np.sum(r * r, axis=1))
    rms = np.sqrt(np.mean(rn * rn))
    den = np.maximum(rn, floor * rms)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.where(den > 0, dn / np.where(den > 0, den, 1.0), np.where(dn > 0, np.inf, 0.0))
    i = int(np.argmax(e))
    return float(e[i]), i
