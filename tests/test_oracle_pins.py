"""Pins of the fp64 oracle against what mathematics fixes (CPU only).

The FlashKDA pages print no formula and no worked example, so each pin is a
closed form, an invariant, a special case that reduces to a textbook routine,
or a brute-force evaluation on tiny inputs. Together they fail on a dropped
term, a wrong sign, a wrong order of decay/erase/write/read, a transposed state
or an indexing slip (tests/test_oracle_mutants.py plants such mistakes).
"""
import csv
import math
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(rng, B, T, H, K=128, V=128, lb=-5.0, state=True, N=None):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    g = rng.standard_normal((B, T, H, K))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    A_log = np.log(rng.uniform(1, 16, H))
    dt_bias = 0.1 * rng.standard_normal((H, K))
    init = 0.05 * rng.standard_normal(((N or B), H, K, V)) if state else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, scale=K ** -0.5, A_log=A_log,
                dt_bias=dt_bias, lower_bound=lb, initial_state=init)


def run(d, **kw):
    args = dict(d)
    args.update(kw)
    return oracle.fwd(args["q"], args["k"], args["v"], args["g"], args["beta"], args["scale"],
                      args["A_log"], args["dt_bias"], args["lower_bound"],
                      initial_state=args.get("initial_state"), cu_seqlens=args.get("cu_seqlens"))


# P1: the rank-1 rewrite equals the literal matrix recurrence
@pytest.mark.parametrize("K,V,T,H", [(128, 128, 48, 2), (8, 5, 64, 3), (16, 16, 33, 1)])
def test_p1_brute_force(K, V, T, H):
    rng = np.random.default_rng(1)
    d = rand_inputs(rng, 1, T, H, K=K, V=V)
    o, f = run(d)
    ob, fb = oracle.brute_force(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["A_log"],
                                d["dt_bias"], d["lower_bound"], initial_state=d["initial_state"])
    assert oracle.rel_l2(o, ob) < 1e-12
    assert oracle.rel_l2(f, fb) < 1e-12


def test_p1_brute_force_varlen():
    rng = np.random.default_rng(2)
    lens = [5, 17, 1, 20]
    d = rand_inputs(rng, 1, sum(lens), 2, K=16, V=12, N=len(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, f = run(d, cu_seqlens=cu)
    ob, fb = oracle.brute_force(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["A_log"],
                                d["dt_bias"], d["lower_bound"], initial_state=d["initial_state"],
                                cu_seqlens=cu)
    assert oracle.rel_l2(o, ob) < 1e-12 and oracle.rel_l2(f, fb) < 1e-12


# P2: a beta = 1 write of a unit key is read back exactly: S_t^T k_t = v_t
def test_p2_exact_retrieval():
    rng = np.random.default_rng(3)
    d = rand_inputs(rng, 1, 80, 2)
    k = d["k"] / np.linalg.norm(d["k"], axis=-1, keepdims=True)
    d["k"] = k
    q = d["q"].copy()
    beta = d["beta"].copy()
    picks = [0, 7, 40, 63, 64, 79]
    for t in picks:
        beta[0, t, :] = 1.0
        q[0, t] = k[0, t]
    o, _ = run(d, q=q, beta=beta)
    for t in picks:
        want = d["scale"] * d["v"][0, t]
        err = np.abs(o[0, t] - want).max() / np.abs(want).max()
        assert err < 1e-5, (t, err)       # the 1e-6 eps of the L2 norm is the only deviation
    # without the beta = 1 / q = k construction the readout is far from v
    o2, _ = run(d)
    assert np.abs(o2[0, 40] - d["scale"] * d["v"][0, 40]).max() > 1e-2


# P3: beta = 0 and alpha -> 1 freeze the state: out = scale * q^ S0, final = S0
def test_p3_frozen_state():
    rng = np.random.default_rng(4)
    d = rand_inputs(rng, 2, 40, 3)
    d["beta"] = np.zeros_like(d["beta"])
    d["A_log"] = np.full(3, -30.0)
    o, f = run(d)
    qn = d["q"] / np.sqrt(np.sum(d["q"] ** 2, -1, keepdims=True) + 1e-6)
    want = d["scale"] * np.einsum("bthk,bhkv->bthv", qn, d["initial_state"])
    assert oracle.rel_l2(o, want) < 1e-10
    assert oracle.rel_l2(f, d["initial_state"]) < 1e-10
    # state orientation: S is indexed [key channel, value channel]
    wrong = d["scale"] * np.einsum("bthk,bhvk->bthv", qn, d["initial_state"])
    assert oracle.rel_l2(o, wrong) > 0.5


def basis_keys(rng, T, H, K=128):
    """Keys that are distinct standard basis vectors (exact in bf16)."""
    k = np.zeros((1, T, H, K))
    perm = np.stack([rng.permutation(K)[:T] for _ in range(H)], 1)   # [T, H]
    for t in range(T):
        for h in range(H):
            k[0, t, h, perm[t, h]] = 1.0
    return k, perm


# P4: orthogonal keys and no decay reduce the delta rule to causal linear attention
def test_p4_linear_attention():
    rng = np.random.default_rng(5)
    T, H = 100, 2
    d = rand_inputs(rng, 1, T, H, state=False)
    d["k"], _ = basis_keys(rng, T, H)
    d["lower_bound"] = 0.0                        # log alpha = 0 exactly
    o, f = run(d)
    qn = d["q"] / np.sqrt(np.sum(d["q"] ** 2, -1, keepdims=True) + 1e-6)
    kn = d["k"] / math.sqrt(1.0 + 1e-6)
    for h in range(H):
        scores = qn[0, :, h] @ kn[0, :, h].T                            # [T, T]
        mask = np.tril(np.ones((T, T)))
        want = d["scale"] * (scores * mask * d["beta"][0, None, :, h]) @ d["v"][0, :, h]
        assert oracle.rel_l2(o[0, :, h], want) < 1e-12
        want_S = (kn[0, :, h] * d["beta"][0, :, h, None]).T @ d["v"][0, :, h]
        assert oracle.rel_l2(f[0, h], want_S) < 1e-12


# P5: orthogonal keys with per-channel gates give the gated-linear-attention closed form
def test_p5_gated_closed_form():
    rng = np.random.default_rng(6)
    T, H = 90, 2
    d = rand_inputs(rng, 1, T, H, state=False, lb=-5.0)
    d["k"], perm = basis_keys(rng, T, H)
    o, _ = run(d)
    qn = d["q"] / np.sqrt(np.sum(d["q"] ** 2, -1, keepdims=True) + 1e-6)
    c = 1.0 / math.sqrt(1.0 + 1e-6)
    for h in range(H):
        x = d["g"][0, :, h] + d["dt_bias"][h]
        sp = np.log1p(np.exp(x))                          # softplus, moderate x here
        la = np.maximum(-np.exp(d["A_log"][h]) * sp, d["lower_bound"])  # [T, K]
        cum = np.cumsum(la, axis=0)
        want = np.zeros((T, 128))
        for t in range(T):
            for j in range(t + 1):
                ch = perm[j, h]
                decay = math.exp(cum[t, ch] - cum[j, ch])        # sum_{i=j+1..t} la_i[ch]
                want[t] += d["beta"][0, j, h] * qn[0, t, h, ch] * c * decay * d["v"][0, j, h]
        want *= d["scale"]
        assert oracle.rel_l2(o[0, :, h], want) < 1e-11


# P6: packed sequences behave as independent runs
def test_p6_varlen_equals_separate():
    rng = np.random.default_rng(7)
    lens = [70, 1, 64, 129, 3]
    d = rand_inputs(rng, 1, sum(lens), 2, N=len(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, f = run(d, cu_seqlens=cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        sl = lambda x: x[:, a:b]
        on, fn = run(d, q=sl(d["q"]), k=sl(d["k"]), v=sl(d["v"]), g=sl(d["g"]), beta=sl(d["beta"]),
                     initial_state=d["initial_state"][n:n + 1], cu_seqlens=None)
        assert np.array_equal(on, o[:, a:b])
        assert np.array_equal(fn[0], f[n])


# P7: running [0, t) then [t, T) from the handed-over state equals the whole run
@pytest.mark.parametrize("split", [64, 37, 1, 127])
def test_p7_state_chaining(split):
    rng = np.random.default_rng(8)
    d = rand_inputs(rng, 1, 128, 2)
    o, f = run(d)
    sl1 = lambda x: x[:, :split]
    sl2 = lambda x: x[:, split:]
    o1, f1 = run(d, q=sl1(d["q"]), k=sl1(d["k"]), v=sl1(d["v"]), g=sl1(d["g"]), beta=sl1(d["beta"]))
    o2, f2 = run(d, q=sl2(d["q"]), k=sl2(d["k"]), v=sl2(d["v"]), g=sl2(d["g"]), beta=sl2(d["beta"]),
                 initial_state=f1)
    assert oracle.rel_l2(np.concatenate([o1, o2], 1), o) < 1e-13
    assert oracle.rel_l2(f2, f) < 1e-13


# P8: a batch equals separate calls per batch row
def test_p8_batch_equals_separate():
    rng = np.random.default_rng(9)
    d = rand_inputs(rng, 3, 50, 2)
    o, f = run(d)
    for b in range(3):
        sl = lambda x: x[b:b + 1]
        ob, fb = run(d, q=sl(d["q"]), k=sl(d["k"]), v=sl(d["v"]), g=sl(d["g"]), beta=sl(d["beta"]),
                     initial_state=d["initial_state"][b:b + 1])
        assert np.array_equal(ob, o[b:b + 1]) and np.array_equal(fb, f[b:b + 1])


# P9: permuting heads (with their A_log and dt_bias) permutes the outputs
def test_p9_head_equivariance():
    rng = np.random.default_rng(10)
    d = rand_inputs(rng, 1, 40, 4)
    o, f = run(d)
    p = np.array([2, 0, 3, 1])
    op, fp = run(d, q=d["q"][:, :, p], k=d["k"][:, :, p], v=d["v"][:, :, p], g=d["g"][:, :, p],
                 beta=d["beta"][:, :, p], A_log=d["A_log"][p], dt_bias=d["dt_bias"][p],
                 initial_state=d["initial_state"][:, p])
    assert np.array_equal(op, o[:, :, p]) and np.array_equal(fp, f[:, p])


# P10: scale multiplies the output only
def test_p10_scale_linearity():
    rng = np.random.default_rng(11)
    d = rand_inputs(rng, 1, 40, 2)
    o, f = run(d)
    o3, f3 = run(d, scale=3.0 * d["scale"])
    assert oracle.rel_l2(o3, 3.0 * o) < 1e-15
    assert np.array_equal(f3, f)


def _gate_cases():
    rows = []
    with open(os.path.join(GOLD, "gate_closed_forms.csv")) as fh:
        for r in csv.reader(fh):
            if not r or r[0].startswith("#"):
                continue
            rows.append(r)
    return rows


# P11: the gate at closed-form points, read back through the full oracle
def test_p11_gate_closed_forms():
    cases = _gate_cases()
    assert len(cases) >= 8
    K = V = 128
    H = len(cases)
    # one token; S0 = identity; beta = 0; q = all ones => o[c] = scale * alpha_c * q^[c]
    q = np.ones((1, 1, H, K))
    k = np.ones((1, 1, H, K))
    v = np.zeros((1, 1, H, V))
    beta = np.zeros((1, 1, H))
    g = np.zeros((1, 1, H, K))
    dt = np.zeros((H, K))
    A_log = np.zeros(H)
    init = np.broadcast_to(np.eye(K), (1, H, K, V)).copy()
    for h, (name, alog, gv, dtv, lb, expr) in enumerate(cases):
        A_log[h] = eval(alog, {"math": math})
        g[0, 0, h, :] = float(gv)
        dt[h, :] = float(dtv)
    for lb_case in sorted(set(float(c[4]) for c in cases)):
        o, _ = oracle.fwd(q, k, v, g, beta, 1.0, A_log, dt, lb_case, initial_state=init)
        qn = 1.0 / math.sqrt(K + 1e-6)
        for h, (name, alog, gv, dtv, lb, expr) in enumerate(cases):
            if float(lb) != lb_case:
                continue
            want = eval(expr, {"math": math})
            got = math.log(o[0, 0, h, 0] / qn)
            assert abs(got - want) <= 1e-12 * max(1.0, abs(want)), (name, got, want)
            assert np.allclose(o[0, 0, h], o[0, 0, h, 0], rtol=0, atol=0)


# P11 (numpy side): the numpy gate agrees with the closed forms too
def test_p11_numpy_gate():
    for name, alog, gv, dtv, lb, expr in _gate_cases():
        got = oracle.gate_log_alpha(float(gv), float(dtv), eval(alog, {"math": math}), float(lb))
        want = eval(expr, {"math": math})
        assert abs(float(got) - want) <= 1e-12 * max(1.0, abs(want)), name


# P12: the L2 normalisation makes the result invariant to positive rescaling of q and k
def test_p12_normalisation_idempotence():
    rng = np.random.default_rng(12)
    d = rand_inputs(rng, 1, 50, 2)
    d["q"] /= np.linalg.norm(d["q"], axis=-1, keepdims=True)
    d["k"] /= np.linalg.norm(d["k"], axis=-1, keepdims=True)
    o, f = run(d)
    o2, f2 = run(d, q=3.0 * d["q"], k=5.0 * d["k"])
    assert oracle.rel_l2(o2, o) < 2e-6 and oracle.rel_l2(f2, f) < 2e-6   # eps 1e-6 only
    o3, _ = run(d, q=-d["q"])
    assert oracle.rel_l2(o3, -o) < 1e-14


# P13: the chunkwise WY/UT algebra equals the per-token recurrence
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("lb", [0.0, -3.0, -5.0, -20.0])
def test_p13_chunk_algebra(chunk, lb):
    rng = np.random.default_rng(13)
    lens = [150, 64, 1, 77]
    d = rand_inputs(rng, 1, sum(lens), 2, lb=lb, N=len(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, f = run(d, cu_seqlens=cu)
    oc, fc = oracle.chunk_twin(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["A_log"],
                               d["dt_bias"], lb, initial_state=d["initial_state"], cu_seqlens=cu,
                               chunk=chunk)
    assert oracle.rel_l2(oc, o) < 1e-12 and oracle.rel_l2(fc, f) < 1e-12


# R11: a zero-length sequence passes its state through unchanged
def test_zero_length_sequence():
    rng = np.random.default_rng(14)
    lens = [10, 0, 5]
    d = rand_inputs(rng, 1, 15, 2, N=3)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, f = run(d, cu_seqlens=cu)
    assert np.array_equal(f[1], d["initial_state"][1])
    _, f0 = run(d, cu_seqlens=cu, initial_state=None)
    assert np.all(f0[1] == 0.0)


def test_bf16_inputs_match_f64_path():
    """The bf16 entry upcasts exactly: same result as feeding the widened values."""
    import kda_inputs as ki
    d = ki.make_inputs(1, 70, 2, seed=3, state="bf16", initial=True)
    o, f = oracle.fwd_inputs(d, want_final=True)
    w = lambda a: ki.bf16_bits_to_f64(a)
    o2, f2 = oracle.fwd(w(d["q"]), w(d["k"]), w(d["v"]), w(d["g"]), w(d["beta"]), d["scale"],
                        d["A_log"], d["dt_bias"], d["lower_bound"],
                        initial_state=w(d["initial_state"]))
    assert np.array_equal(o, o2) and np.array_equal(f, f2)


# ---------------------------------------------------------------------------
# Acceptance arithmetic. The tolerance bar (relative L2 and largest absolute
# error per tensor) and the per-row bound are themselves pinned on vectors whose
# results are worked out by hand, so a missing abs(), a norm taken over the
# candidate instead of the reference, or a row slice along the wrong axis fails.
# ---------------------------------------------------------------------------
def test_rel_l2_hand_values():
    ref = np.array([3.0, 4.0])                      # ||ref|| = 5
    assert oracle.rel_l2(np.array([3.0, 4.0]), ref) == 0.0
    assert oracle.rel_l2(np.array([3.0, 5.0]), ref) == pytest.approx(1.0 / 5.0, rel=1e-15)
    assert oracle.rel_l2(np.array([3.0, 3.0]), ref) == pytest.approx(1.0 / 5.0, rel=1e-15)  # sign of the deviation
    # normalised by the reference, not the candidate: x = 2 ref gives ||ref|| / ||ref|| = 1
    assert oracle.rel_l2(2.0 * ref, ref) == pytest.approx(1.0, rel=1e-15)
    assert oracle.rel_l2(0.5 * ref, ref) == pytest.approx(0.5, rel=1e-15)
    # a zero reference falls back to ||x||
    assert oracle.rel_l2(np.array([0.0, 2.0]), np.zeros(2)) == pytest.approx(2.0, rel=1e-15)
    assert oracle.rel_l2(np.zeros(3), np.zeros(3)) == 0.0
    # whole-tensor norms: [[1, 0], [0, 1]] against [[1, 1], [1, 1]] -> sqrt(2) / 2
    assert oracle.rel_l2(np.eye(2), np.ones((2, 2))) == pytest.approx(math.sqrt(2.0) / 2.0, rel=1e-15)


def test_max_abs_hand_values():
    ref = np.array([1.0, -2.0, 0.5])
    assert oracle.max_abs(ref, ref) == 0.0
    assert oracle.max_abs(np.array([1.0, -2.5, 0.5]), ref) == pytest.approx(0.5)    # negative deviation
    assert oracle.max_abs(np.array([1.25, -2.0, 0.0]), ref) == pytest.approx(0.5)   # largest of 0.25 and 0.5
    assert oracle.max_abs(np.array([[0.0, 3.0]]), np.array([[0.0, -1.0]])) == pytest.approx(4.0)
    assert oracle.max_abs(np.zeros(0), np.zeros(0)) == 0.0


def test_row_rel_l2_hand_values():
    ref = np.array([[3.0, 4.0], [0.0, 5.0], [5.0, 0.0]])    # every row norm 5, rms 5
    e, i = oracle.row_rel_l2(ref, ref)
    assert e == 0.0
    x = ref.copy()
    x[1, 1] = 4.0                                            # row 1 off by 1 -> 1 / 5
    e, i = oracle.row_rel_l2(x, ref)
    assert i == 1 and e == pytest.approx(0.2, rel=1e-15)
    # the whole-tensor error of the same deviation is diluted: 1 / sqrt(75)
    assert oracle.rel_l2(x, ref) == pytest.approx(1.0 / math.sqrt(75.0), rel=1e-15)
    # one zero row among unit rows: measured against floor * rms
    ref2 = np.array([[1.0, 0.0], [0.0, 1.0], [0.0, 0.0], [1.0, 0.0]])   # rms of norms = sqrt(3/4)
    x2 = ref2.copy()
    x2[2] = [0.1, 0.0]
    e, i = oracle.row_rel_l2(x2, ref2, floor=0.25)
    assert i == 2 and e == pytest.approx(0.1 / (0.25 * math.sqrt(0.75)), rel=1e-12)
    # rows over two trailing axes (a state block per sequence and head)
    refs = np.ones((2, 3, 2, 2))
    xs = refs.copy()
    xs[1, 2, 0, 1] = 3.0                                    # block (1, 2): ||d|| = 2, ||ref|| = 2
    e, i = oracle.row_rel_l2(xs, refs, row_ndim=2)
    assert i == 1 * 3 + 2 and e == pytest.approx(1.0, rel=1e-15)
    assert oracle.row_rel_l2(np.zeros((0, 4)), np.zeros((0, 4))) == (0.0, -1)


def test_chunk_twin_no_overflow_at_strong_decay():
    """The twin forms the pairwise decay only for j <= r, where the exponent is <= 0,
    so a very negative lower_bound raises no floating-point overflow."""
    rng = np.random.default_rng(31)
    d = rand_inputs(rng, 1, 96, 1, K=16, V=8, lb=-200.0)
    d["A_log"] = np.array([math.log(16.0)])
    with np.errstate(over="raise", invalid="raise"):
        ot, ft = oracle.chunk_twin(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["A_log"],
                                   d["dt_bias"], d["lower_bound"], initial_state=d["initial_state"])
    o, f = run(d)
    assert oracle.rel_l2(ot, o) < 1e-12 and oracle.rel_l2(ft, f) < 1e-12
