"""GPU parity of libkda (through its C ABI) against the fp64 oracle.

Bar (fixed before measuring): per tensor, relative L2 error <= 1e-2 and max
absolute error <= 5e-2 for ``out`` and, where returned, ``final_state``; per
row (the 128 outputs of one token and head, or the 128 x 128 final state of one
sequence and head), relative L2 error <= 5e-2 against the larger of the row's
reference norm and the root-mean-square row norm; exact (bitwise) equality
where the chunking makes two computations identical (varlen vs separate calls,
batch vs separate calls, chained calls split at a multiple of 64 with an fp32
state, repeated calls).

The per-row bound: an element of ``out`` is a sum of bf16-rounded products
(relative rounding 2^-9 per operand), so the error of a correct row is a few
1e-3 of the size of the operands that formed it, as for the whole tensor. A
row's own norm can be far smaller than those operands (the reference row norms
of the dense batch spread over three decades: median 0.56, 1 % of rows below
0.03 of the root-mean-square row norm), so small rows are measured against a
typical row. 5e-2 leaves an order of magnitude for accumulation over chunks,
while a wrong, stale or unwritten row of typical size (relative error about 1)
fails it however large the tensor is.
"""
import math
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import kda_inputs as ki
import oracle

pytestmark = pytest.mark.gpu

REL_TOL = 1e-2
ABS_TOL = 5e-2
ROW_TOL = 5e-2


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


def check(name, got, ref, row_ndim=1):
    """The tensor bar and the per-row bound; rows span the trailing row_ndim axes."""
    rel = oracle.rel_l2(got, ref)
    mab = oracle.max_abs(got, ref)
    row, at = oracle.row_rel_l2(got, ref, row_ndim=row_ndim)
    print("%-28s rel_l2=%.3e max_abs=%.3e row_max=%.3e (row %d)" % (name, rel, mab, row, at), flush=True)
    assert np.all(np.isfinite(got)), name + ": non-finite values"
    assert rel <= REL_TOL and mab <= ABS_TOL, (name, rel, mab)
    assert row <= ROW_TOL, (name, "row", at, row)


def check_state(name, got, ref):
    """check() with one row per (sequence, head) state block."""
    check(name, got, ref, row_ndim=2)


# ---------------------------------------------------------------- workloads
# full-size workloads run on the GPU exactly as the bench launches them; the
# oracle recomputes every head, token and state
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_workload_parity(cfg):
    gu = _gpu()
    print("workload %d" % cfg, flush=True)
    d = ki.config_inputs(cfg)
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=d["final"])
    check("cfg%d out" % cfg, o, ro)
    if d["final"]:
        check_state("cfg%d final_state" % cfg, f, rf)


# ---------------------------------------------------------------- edge cases
@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 129, 200])
def test_ragged_lengths(T):
    gu = _gpu()
    d = ki.make_inputs(2, T, 3, seed=T, state="fp32", initial=True, sigma=0.05)
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    check("T=%d out" % T, o, ro)
    check_state("T=%d final" % T, f, rf)


@pytest.mark.parametrize("state", ["bf16", "fp32"])
def test_varlen_with_empty_and_single(state):
    gu = _gpu()
    lens = [1, 0, 64, 65, 130, 3, 0, 200]
    d = ki.make_inputs(1, sum(lens), 2, seed=5, lengths=lens, state=state, initial=True, sigma=0.05)
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    check("varlen %s out" % state, o, ro)
    check_state("varlen %s final" % state, f, rf)
    # empty sequences pass the state through (bf16 -> fp32 -> bf16 is exact)
    init = d["initial_state"]
    init64 = ki.bf16_bits_to_f64(init) if state == "bf16" else init.astype(np.float64)
    assert np.array_equal(f[1], init64[1]) and np.array_equal(f[6], init64[6])


def test_no_state_and_final_only():
    gu = _gpu()
    d = ki.make_inputs(1, 300, 2, seed=6, state="fp32", initial=False)
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    check("final-only out", o, ro)
    check_state("final-only final", f, rf)
    d2 = ki.make_inputs(1, 300, 2, seed=6)
    o2, f2 = gu.run_gpu(d2)
    assert f2 is None and np.array_equal(o2, o)


@pytest.mark.parametrize("lb", [0.0, -1.0, -10.0, -10.5, -20.0, -60.0, -1000.0])
def test_lower_bound_range(lb):
    """Below -10 the chunk preparation builds every decay factor from exponents
    <= 0 and sums the diagonal blocks element by element (any finite bound)."""
    gu = _gpu()
    d = ki.make_inputs(1, 256, 2, seed=7, lower_bound=lb, state="fp32", initial=True, sigma=0.05)
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    check("lb=%g out" % lb, o, ro)
    check_state("lb=%g final" % lb, f, rf)


def test_maximum_sizes():
    """A sequence of 2^20 + 3 tokens (16,385 chunks, segment-parallel scan) and a
    batch of 256 heads (64 KB token rows, many-chain scan), against the oracle."""
    gu = _gpu()
    T = (1 << 20) + 3
    d = ki.make_inputs(1, T, 2, seed=28, state="fp32", initial=True, sigma=0.05)
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    check("T=2^20+3 out", o, ro)
    check_state("T=2^20+3 final", f, rf)
    del d, o, ro
    d = ki.make_inputs(1, 300, 256, seed=29, state="bf16", initial=True, sigma=0.05)
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    check("H=256 out", o, ro)
    check_state("H=256 final", f, rf)


def test_unnormalised_inputs():
    """q and k that are not unit rows are normalised inside the kernel."""
    gu = _gpu()
    d = ki.make_inputs(1, 192, 2, seed=8, state="fp32", initial=True)
    rng = np.random.default_rng(0)
    for key in ("q", "k"):
        x = ki.bf16_bits_to_f32(d[key]) * rng.uniform(0.1, 30.0, d[key].shape[:-1] + (1,)).astype(np.float32)
        d[key] = ki.f32_to_bf16_bits(x)
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    check("unnormalised out", o, ro)
    check_state("unnormalised final", f, rf)


# ---------------------------------------------------------------- exact invariants
def test_varlen_equals_separate_bitwise():
    gu = _gpu()
    lens = [70, 1, 128, 129, 3]
    d = ki.make_inputs(1, sum(lens), 2, seed=9, lengths=lens, state="fp32", initial=True)
    o, f = gu.run_gpu(d)
    cu = d["cu_seqlens"]
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        e = dict(d)
        for key in ("q", "k", "v", "g", "beta"):
            e[key] = np.ascontiguousarray(d[key][:, a:b])
        e.update(T=b - a, N=1, cu_seqlens=None, initial_state=np.ascontiguousarray(d["initial_state"][n:n + 1]))
        on, fn = gu.run_gpu(e)
        assert np.array_equal(on, o[:, a:b]) and np.array_equal(fn[0], f[n]), n


# With 128 or more (sequence, head) chains the scan runs on its eight-wave
# kernel; in a packed batch, sequences of more than 128 chunks go to its
# three-wave kernel instead (listed by the chunk-table kernel). With fewer chains
# the three-wave kernel runs them all. The two use the same arithmetic in the
# same order, so a sequence gives the same bits either way.
@pytest.mark.parametrize("state", ["fp32", "bf16"])
def test_many_chain_scan(state):
    gu = _gpu()
    rng = np.random.default_rng(21)
    lens = [8300, 0, 1, 64, 65, 129, 8200] + [int(x) for x in rng.integers(1, 300, 57)]
    d = ki.make_inputs(1, sum(lens), 2, seed=21, lengths=lens, state=state, initial=True, sigma=0.05)
    assert len(lens) * 2 >= 128 and lens[0] > 128 * 64 and lens[6] > 128 * 64
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    check("many-chain %s out" % state, o, ro)
    check_state("many-chain %s final" % state, f, rf)
    cu = d["cu_seqlens"]
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        e = dict(d)
        for key in ("q", "k", "v", "g", "beta"):
            e[key] = np.ascontiguousarray(d[key][:, a:b])
        e.update(T=b - a, N=1, cu_seqlens=None, initial_state=np.ascontiguousarray(d["initial_state"][n:n + 1]))
        if b == a:
            continue
        on, fn = gu.run_gpu(e)
        assert np.array_equal(on, o[:, a:b]) and np.array_equal(fn[0], f[n]), n


def test_many_sequences_chunk_table():
    """3000 packed sequences: the chunk table's prefix sums (chunk offsets and the
    list of sequences of more than 128 chunks) carry across its 1024-thread
    passes; long sequences sit in the second and third passes."""
    gu = _gpu()
    rng = np.random.default_rng(25)
    lens = [int(x) for x in rng.integers(0, 40, 3000)]
    lens[1500], lens[2999], lens[700] = 8300, 9000, 130
    d = ki.make_inputs(1, sum(lens), 1, seed=25, lengths=lens, state="fp32", initial=True, sigma=0.05)
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    check("3000 seqs out", o, ro)
    check_state("3000 seqs final", f, rf)


def test_many_chain_fixed_batch():
    """A fixed-length batch of 128 chains (eight-wave kernel) against the oracle
    and, bit for bit, against single-sequence calls (three-wave kernel)."""
    gu = _gpu()
    d = ki.make_inputs(64, 200, 2, seed=22, state="fp32", initial=True, sigma=0.05)
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    check("fixed-batch out", o, ro)
    check_state("fixed-batch final", f, rf)
    for b in (0, 17, 63):
        e = dict(d)
        for key in ("q", "k", "v", "g", "beta"):
            e[key] = np.ascontiguousarray(d[key][b:b + 1])
        e.update(B=1, N=1, initial_state=np.ascontiguousarray(d["initial_state"][b:b + 1]))
        ob, fb = gu.run_gpu(e)
        assert np.array_equal(ob, o[b:b + 1]) and np.array_equal(fb, f[b:b + 1]), b


# Fixed-length batches of at most 10 long (sequence, head) chains take the
# segment-parallel scan (segment maps M, B; their fp32 chaining; a rescan of
# every segment). It agrees with the oracle to the same bar as the plain scan,
# and with the plain scan that the one-sequence varlen form of the same input
# runs, to rounding.
@pytest.mark.parametrize("B,T,H,state", [(1, 8192, 2, "fp32"), (1, 8192 - 37, 1, "bf16"), (2, 5000, 3, "fp32"),
                                         (1, 4096, 4, None)])
def test_segmented_scan(B, T, H, state):
    gu = _gpu()
    import kimi_delta_attention_fwd_amd as kda
    nchunk = (T + 63) // 64
    assert B * H <= 10 and nchunk >= 48  # the sizes that select three or more segments
    d = ki.make_inputs(B, T, H, seed=23 + T, state=state or "fp32", initial=state is not None, sigma=0.05)
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=d["final"])
    check("segmented B=%d T=%d H=%d out" % (B, T, H), o, ro)
    if d["final"]:
        check_state("segmented B=%d T=%d H=%d final" % (B, T, H), f, rf)
    # the same batch as packed sequences (cu_seqlens): the plain scan
    e = dict(d)
    for key in ("q", "k", "v", "g", "beta"):
        e[key] = np.ascontiguousarray(d[key].reshape((1, B * T) + d[key].shape[2:]))
    e.update(B=1, T=B * T, N=B, cu_seqlens=np.arange(B + 1, dtype=np.int64) * T)
    op, fp = gu.run_gpu(e)
    assert oracle.rel_l2(op.reshape(o.shape), o) < 2e-3
    if d["final"]:
        assert oracle.rel_l2(fp, f) < 2e-3


@pytest.mark.parametrize("lens,H,state", [([6000, 3000], 2, "fp32"), ([5000, 0, 30, 2000], 2, "bf16")])
def test_segmented_scan_packed(lens, H, state):
    """Packed batches of at most 10 chains: per-sequence segment counts (an empty
    and a one-chunk sequence have one segment). Checked against the oracle and
    against the plain scan, which the same sequences take when five one-token
    sequences push the batch past 10 chains."""
    gu = _gpu()
    d = ki.make_inputs(1, sum(lens), H, seed=26, lengths=lens, state=state, initial=True, sigma=0.05)
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    check("segmented packed %s out" % lens, o, ro)
    check_state("segmented packed %s final" % lens, f, rf)
    n, t = len(lens), sum(lens)
    e = ki.make_inputs(1, t + 5, H, seed=27, lengths=lens + [1] * 5, state=state, initial=True, sigma=0.05)
    for key in ("q", "k", "v", "g", "beta"):
        e[key][:, :t] = d[key]
    for key in ("A_log", "dt_bias"):
        e[key] = d[key]
    e["initial_state"][:n] = d["initial_state"]
    o2, f2 = gu.run_gpu(e)
    assert oracle.rel_l2(o2[:, :t], o) < 2e-3 and oracle.rel_l2(f2[:n], f) < 2e-3


def test_segmented_exact_invariants():
    """On the segment-parallel path (T = 8192, H = 2): with beta = 0 and no decay
    every segment map is exactly [0 | I], so the final state equals the initial
    one bit for bit; and a beta = 1 write of a unit key is read back."""
    gu = _gpu()
    d = ki.make_inputs(1, 8192, 2, seed=30, state="fp32", initial=True, lower_bound=0.0)
    d["beta"][:] = 0
    o, f = gu.run_gpu(d)
    assert np.array_equal(f, d["initial_state"].astype(np.float64))
    ro, _ = oracle.fwd_inputs(d, want_final=False)
    check("segmented frozen out", o, ro)
    d = ki.make_inputs(1, 8192, 2, seed=31, state="fp32", initial=True)
    picks = [5, 2047, 2048, 6000, 8191]
    for t in picks:
        d["beta"][0, t] = ki.f32_to_bf16_bits(np.ones(2, np.float32))
        d["q"][0, t] = d["k"][0, t]
    o, _ = gu.run_gpu(d)
    v = ki.bf16_bits_to_f64(d["v"])
    for t in picks:
        want = d["scale"] * v[0, t]
        err = np.abs(o[0, t] - want).max() / np.abs(want).max()
        assert err < 2e-2, (t, err)


@pytest.mark.parametrize("packed", [False, True])
def test_segmented_long_memory(packed):
    """Weak decay (A_log = -12, a per-token decay of about e^-4e-6) and small beta
    (at most 0.02): the state keeps its memory across all segments, so the
    segment maps M are far from zero and their chaining is exercised (with the
    default inputs the state forgets its start within a segment and M underflows
    to 0). Against the oracle, and against the plain scan of the same sequences."""
    gu = _gpu()
    lens = [8192, 3000]
    d = ki.make_inputs(1, sum(lens), 2, seed=32, lengths=lens if packed else None, state="fp32", initial=True,
                       sigma=0.5) if packed else \
        ki.make_inputs(1, 8192, 2, seed=32, state="fp32", initial=True, sigma=0.5)
    d["A_log"][:] = -12.0
    d["beta"] = ki.f32_to_bf16_bits(ki.bf16_bits_to_f32(d["beta"]) * np.float32(0.02))
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    check("long-memory %s out" % ("packed" if packed else "batch"), o, ro)
    check_state("long-memory %s final" % ("packed" if packed else "batch"), f, rf)
    # the plain scan: the same sequences plus 5 one-token sequences (more than 10 chains)
    ls = lens if packed else [8192]
    n, t = len(ls), sum(ls)
    e = ki.make_inputs(1, t + 5, 2, seed=33, lengths=ls + [1] * 5, state="fp32", initial=True, sigma=0.5)
    for key in ("q", "k", "v", "g", "beta"):
        e[key][:, :t] = d[key].reshape(e[key][:, :t].shape)
    for key in ("A_log", "dt_bias"):
        e[key] = d[key]
    e["initial_state"][:n] = d["initial_state"]
    o2, f2 = gu.run_gpu(e)
    assert oracle.rel_l2(o2[:, :t].reshape(o.shape), o) < 2e-3 and oracle.rel_l2(f2[:n], f) < 2e-3
    # the first chunk's state really persists: the final state still depends on it
    d0 = dict(d)
    d0["initial_state"] = np.zeros_like(d["initial_state"])
    _, f0 = gu.run_gpu(d0)
    assert oracle.rel_l2(f0, f) > 1e-2


def test_segmented_in_place_state():
    gu = _gpu()
    d = ki.make_inputs(1, 6000, 2, seed=24, state="fp32", initial=True, sigma=0.05)
    o, f = gu.run_gpu(d)
    o2, f2 = gu.run_gpu(d, in_place=True)
    assert np.array_equal(o, o2) and np.array_equal(f, f2)


def test_batch_equals_separate_bitwise():
    gu = _gpu()
    d = ki.make_inputs(3, 150, 2, seed=10, state="bf16", initial=True)
    o, f = gu.run_gpu(d)
    for b in range(3):
        e = dict(d)
        for key in ("q", "k", "v", "g", "beta"):
            e[key] = np.ascontiguousarray(d[key][b:b + 1])
        e.update(B=1, N=1, initial_state=np.ascontiguousarray(d["initial_state"][b:b + 1]))
        ob, fb = gu.run_gpu(e)
        assert np.array_equal(ob, o[b:b + 1]) and np.array_equal(fb, f[b:b + 1])


@pytest.mark.parametrize("split", [128, 100])
def test_state_chaining(split):
    gu = _gpu()
    d = ki.make_inputs(1, 320, 2, seed=11, state="fp32", initial=True)
    o, f = gu.run_gpu(d)
    first, second = dict(d), dict(d)
    for key in ("q", "k", "v", "g", "beta"):
        first[key] = np.ascontiguousarray(d[key][:, :split])
        second[key] = np.ascontiguousarray(d[key][:, split:])
    first["T"], second["T"] = split, 320 - split
    o1, f1 = gu.run_gpu(first)
    second["initial_state"] = f1.astype(np.float32)
    o2, f2 = gu.run_gpu(second)
    oc = np.concatenate([o1, o2], axis=1)
    if split % 64 == 0:
        assert np.array_equal(oc, o) and np.array_equal(f2, f)
    else:
        check("chain out", oc, o)
        check_state("chain final", f2, f)


def test_in_place_state():
    gu = _gpu()
    d = ki.make_inputs(2, 100, 2, seed=12, state="fp32", initial=True)
    o, f = gu.run_gpu(d)
    o2, f2 = gu.run_gpu(d, in_place=True)
    assert np.array_equal(o, o2) and np.array_equal(f, f2)


def test_deterministic_and_full_coverage():
    gu = _gpu()
    d = ki.make_inputs(1, 333, 3, seed=13, state="fp32", initial=True)
    t = gu.dev_inputs(d)
    out = torch.full((1, 333, 3, 128), float("nan"), dtype=torch.bfloat16, device=gu.DEV)
    o1, f1 = gu.run_gpu(d, t=t, out=out)
    assert np.all(np.isfinite(o1))
    out2 = torch.full((1, 333, 3, 128), float("nan"), dtype=torch.bfloat16, device=gu.DEV)
    o2, f2 = gu.run_gpu(d, t=t, out=out2)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_guard_bands_untouched():
    """Writes stay inside out and final_state (canaries around both)."""
    gu = _gpu()
    import kimi_delta_attention_fwd_amd as kda
    d = ki.make_inputs(1, 130, 2, seed=14, state="fp32", initial=True)
    t = gu.dev_inputs(d)
    n_out = 130 * 2 * 128
    big = torch.full((n_out + 2048,), 7.0, dtype=torch.bfloat16, device=gu.DEV)
    out = big[1024:1024 + n_out].view(1, 130, 2, 128)
    n_st = 2 * 128 * 128
    bigs = torch.full((n_st + 2048,), 3.0, dtype=torch.float32, device=gu.DEV)
    fin = bigs[1024:1024 + n_st].view(1, 2, 128, 128)
    kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], out, t["A_log"], t["dt_bias"],
            d["lower_bound"], initial_state=t["initial_state"], final_state=fin)
    torch.cuda.synchronize()
    assert torch.all(big[:1024] == 7.0) and torch.all(big[1024 + n_out:] == 7.0)
    assert torch.all(bigs[:1024] == 3.0) and torch.all(bigs[1024 + n_st:] == 3.0)


# ---------------------------------------------------------------- pins on the GPU
def test_retrieval_on_gpu():
    """A beta = 1 write of a unit key is read back: out_t = scale * v_t."""
    gu = _gpu()
    d = ki.make_inputs(1, 128, 2, seed=15, state="fp32", initial=True)
    picks = [5, 63, 64, 100]
    for t in picks:
        d["beta"][0, t] = ki.f32_to_bf16_bits(np.ones(2, np.float32))
        d["q"][0, t] = d["k"][0, t]
    o, _ = gu.run_gpu(d)
    v = ki.bf16_bits_to_f64(d["v"])
    for t in picks:
        want = d["scale"] * v[0, t]
        err = np.abs(o[0, t] - want).max() / np.abs(want).max()
        assert err < 2e-2, (t, err)


def test_frozen_state_on_gpu():
    """beta = 0 and alpha = 1 (lower_bound 0 and A_log -30): final == initial exactly."""
    gu = _gpu()
    d = ki.make_inputs(1, 200, 2, seed=16, state="fp32", initial=True, lower_bound=0.0)
    d["beta"][:] = 0
    o, f = gu.run_gpu(d)
    assert np.array_equal(f, d["initial_state"].astype(np.float64))
    ro, _ = oracle.fwd_inputs(d, want_final=False)
    check("frozen out", o, ro)


# ---------------------------------------------------------------- argument errors
def test_errors_raise():
    gu = _gpu()
    import kimi_delta_attention_fwd_amd as kda
    d = ki.make_inputs(1, 64, 1, seed=17)
    t = gu.dev_inputs(d)
    out = torch.empty((1, 64, 1, 128), dtype=torch.bfloat16, device=gu.DEV)
    with pytest.raises(ValueError, match="KDA_ERR_ARG"):
        kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], out, t["A_log"], t["dt_bias"], 0.5)
    with pytest.raises(ValueError, match="KDA_ERR_ARG"):
        kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], out, t["A_log"], t["dt_bias"], float("nan"))
    with pytest.raises(ValueError, match="KDA_ERR_ALIAS"):
        kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], t["v"], t["A_log"], t["dt_bias"], -5.0)
    s32 = torch.zeros((1, 1, 128, 128), dtype=torch.float32, device=gu.DEV)
    s16 = torch.zeros((1, 1, 128, 128), dtype=torch.bfloat16, device=gu.DEV)
    with pytest.raises(ValueError):
        kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], out, t["A_log"], t["dt_bias"], -5.0,
                initial_state=s32, final_state=s16)
    cu = torch.tensor([0, 32, 64], dtype=torch.int32, device=gu.DEV)
    q2 = torch.zeros((2, 32, 1, 128), dtype=torch.bfloat16, device=gu.DEV)
    b2 = torch.zeros((2, 32, 1), dtype=torch.bfloat16, device=gu.DEV)
    o2 = torch.empty_like(q2)
    with pytest.raises(ValueError, match="KDA_ERR_SHAPE"):
        kda.fwd(q2, q2, q2, q2, b2, d["scale"], o2, t["A_log"], t["dt_bias"], -5.0, cu_seqlens=cu)


def test_library_loaded_before_torch():
    """A fresh process that loads libkda before importing torch runs kda.fwd
    correctly (regression: libkda used to bind the system HIP runtime next to
    torch's own, and every launch failed with KDA_ERR_HIP)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = """
import sys
sys.path.insert(0, %r)
import kimi_delta_attention_fwd_amd as kda
kda.load_library()
import numpy as np, torch
import kda_inputs as ki, oracle
d = ki.make_inputs(1, 100, 2, seed=3, state="fp32", initial=True, sigma=0.02)
bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")
out = torch.empty((1, 100, 2, 128), dtype=torch.bfloat16, device="cuda:0")
kda.fwd(bf(d["q"]), bf(d["k"]), bf(d["v"]), bf(d["g"]), bf(d["beta"]), d["scale"], out,
        torch.from_numpy(d["A_log"]).to("cuda:0"), torch.from_numpy(d["dt_bias"]).to("cuda:0"), d["lower_bound"],
        initial_state=torch.from_numpy(d["initial_state"]).to("cuda:0"))
torch.cuda.synchronize()
ro, _ = oracle.fwd_inputs(d)
e = oracle.rel_l2(out.float().cpu().numpy(), ro)
assert e <= 1e-2, e
print("ok", e)
""" % root
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout[-1000:] + r.stderr[-2000:]


# From 33 to 127 (sequence, head) chains the scan runs as pairs of value tiles
# (six waves per workgroup, four CUs per chain); 32 chains or fewer take the
# three-wave kernel. Both evaluate the same chunk update in the same order, so a
# head gives the same bits on either.
@pytest.mark.parametrize("B,T,H,state", [(1, 1000, 33, "fp32"), (3, 333, 16, "bf16"), (2, 129, 50, None),
                                         (1, 70, 127, "fp32")])
def test_pair_scan(B, T, H, state):
    gu = _gpu()
    assert 33 <= B * H < 128
    d = ki.make_inputs(B, T, H, seed=40 + H, state=state or "fp32", initial=state is not None, sigma=0.05)
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=d["final"])
    check("pair B=%d T=%d H=%d out" % (B, T, H), o, ro)
    if d["final"]:
        check_state("pair B=%d T=%d H=%d final" % (B, T, H), f, rf)
    # the first head alone (B chains, the three-wave kernel): the same bits
    e = gu.subset_heads(d, [0])
    oe, fe = gu.run_gpu(e)
    assert np.array_equal(oe[:, :, 0], o[:, :, 0])
    if d["final"]:
        assert np.array_equal(fe[:, 0], f[:, 0])


def test_pair_scan_packed_and_in_place():
    """40 packed sequences (with empty and one-token ones) on one head: the pair
    scan over cu_seqlens, against the oracle and, for an in-place state, against
    itself."""
    gu = _gpu()
    rng = np.random.default_rng(45)
    lens = [0, 1, 64, 65, 700] + [int(x) for x in rng.integers(1, 400, 35)]
    d = ki.make_inputs(1, sum(lens), 1, seed=45, lengths=lens, state="bf16", initial=True, sigma=0.05)
    o, f = gu.run_gpu(d)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    check("pair packed out", o, ro)
    check_state("pair packed final", f, rf)
    init = ki.bf16_bits_to_f64(d["initial_state"])
    assert np.array_equal(f[0], init[0])
    o2, f2 = gu.run_gpu(d, in_place=True)
    assert np.array_equal(o, o2) and np.array_equal(f, f2)
