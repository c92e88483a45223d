"""GPU parity of kda_bwd against the fp64 backward oracle (oracle/backward.py).

Every case draws seeded bf16 inputs (kda_inputs), a bf16 output gradient and
an fp32 final-state gradient, runs the HIP backward through the C ABI, and
compares every gradient with the oracle's on the same bf16 values.

Tolerance: the kernels compute in fp32 (unit roundoff 6e-8). The largest
error source is the reverse state recurrence, whose rounding grows with the
number of chunks, and the cancellation in the decay gradient dg between the
row-side and column-side pairwise terms. The bar is a relative L2 error of
1e-3 per gradient tensor and a largest element error of 1e-2 of the tensor's
largest magnitude. Elements whose rate term lies within 1e-5 of lower_bound
are left out of the dg comparison: there fp32 and fp64 may take different
clamp branches, and the gradient jumps between branches.
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import kimi_delta_attention_fwd_amd as kda
import oracle
from oracle import backward as obwd
from tests.gpu_util import DEV, dev_inputs, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

REL_L2 = 1e-3
MAX_FRAC = 1e-2
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dA_log", "ddt_bias", "dinitial_state")


def case(B, T, H, seed, lengths=None, lb=-5.0, state="fp32", initial=True, dfinal=True, sigma=0.05):
    d = ki.make_inputs(B, T, H, seed, lengths=lengths, lower_bound=lb, state=state, initial=initial,
                       sigma=sigma, dt_sigma=0.1)
    rng = np.random.default_rng(seed + 1000)
    d["dout"] = ki.f32_to_bf16_bits(rng.standard_normal((B, T, H, 128), dtype=np.float32))
    d["dfinal"] = (rng.standard_normal((d["N"], H, 128, 128), dtype=np.float32) * np.float32(0.1)
                   if dfinal else None)
    return d


def run_bwd(d):
    t = dev_inputs(d)
    dout = to_dev_bf16(d["dout"])
    dfin = None if d["dfinal"] is None else to_dev(d["dfinal"])
    print("kda_bwd case B=%d T=%d H=%d N=%d lb=%g" % (d["B"], d["T"], d["H"], d["N"], d["lower_bound"]),
          flush=True)
    gr = kda.bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], dout, t["A_log"], t["dt_bias"],
                 d["lower_bound"], initial_state=t["initial_state"], dfinal_state=dfin,
                 cu_seqlens=t["cu_seqlens"])
    torch.cuda.synchronize()
    return {n: gr[n].cpu().numpy().astype(np.float64) for n in NAMES}


def run_oracle(d):
    init = d["initial_state"]
    return obwd.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["A_log"], d["dt_bias"],
                    d["lower_bound"], d["dout"], initial_state=init, dfinal=d["dfinal"],
                    cu_seqlens=d["cu_seqlens"])


def compare(d, got, ref):
    margin = obwd.clamp_margin(d["g"], d["dt_bias"], d["A_log"], d["lower_bound"])
    report = {}
    for n in NAMES:
        x, r = got[n], ref[n]
        if n == "dg":
            keep = margin >= 1e-5
            x, r = x[keep], r[keep]
        rel = oracle.rel_l2(x, r)
        mx = oracle.max_abs(x, r)
        scale = float(np.abs(r).max()) if r.size else 0.0
        report[n] = (rel, mx / scale if scale > 0 else mx)
        assert np.all(np.isfinite(x)), n
        if scale == 0.0:
            assert mx == 0.0, (n, mx)
            continue
        assert rel <= REL_L2, (n, rel)
        assert mx <= MAX_FRAC * scale, (n, mx, scale)
    print({n: "%.2e / %.2e" % v for n, v in report.items()}, flush=True)


def test_bwd_fixed_length_ragged():
    d = case(2, 200, 2, 1)          # 3 full chunks and an 8-token tail per sequence
    compare(d, run_bwd(d), run_oracle(d))


def test_bwd_packed_with_empty_sequence():
    lens = [37, 130, 0, 64, 5, 1]
    d = case(1, sum(lens), 2, 2, lengths=lens)
    compare(d, run_bwd(d), run_oracle(d))


def test_bwd_no_states():
    d = case(1, 150, 1, 3, state=None, initial=False, dfinal=False)
    compare(d, run_bwd(d), run_oracle(d))


def test_bwd_bf16_initial_state():
    d = case(1, 100, 2, 4, state="bf16", sigma=0.1)
    compare(d, run_bwd(d), run_oracle(d))


@pytest.mark.parametrize("lb", [0.0, -1.0, -30.0])
def test_bwd_lower_bounds(lb):
    d = case(1, 130, 1, 5, lb=lb)
    got, ref = run_bwd(d), run_oracle(d)
    compare(d, got, ref)
    if lb == 0.0:   # every rate term is clamped: no gate gradient at all
        assert np.all(got["dg"] == 0) and np.all(got["dA_log"] == 0) and np.all(got["ddt_bias"] == 0)


def test_bwd_long_chain():
    d = case(1, 1100, 1, 6)         # 18 chunks, 12-token tail
    compare(d, run_bwd(d), run_oracle(d))


def test_bwd_repeatable():
    d = case(1, 200, 2, 7)
    a, b = run_bwd(d), run_bwd(d)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("cfg,h0", [(3, 5), (2, 17)])
def test_bwd_full_size_sampled_head(cfg, h0):
    """Backward workloads at full size, run whole on the GPU in the launch
    configuration of `bench.py --backward --config cfg` (the bench's seeded bf16
    output gradient and fp32 final-state gradient): the long prefill (B=1,
    T=65536, H=32, lower_bound -3, no initial state) and the varlen batch (16
    packed sequences, 66,399 tokens, H=32, bf16 initial state). Head h0 is checked
    against the oracle run on that head alone (heads are independent)."""
    d = ki.config_inputs(cfg)
    B, T, H, N = d["B"], d["T"], d["H"], d["N"]
    rng = np.random.default_rng(1234)
    dout = ki.f32_to_bf16_bits(rng.standard_normal((B, T, H, 128), dtype=np.float32))
    dfin = rng.standard_normal((N, H, 128, 128), dtype=np.float32) * np.float32(0.1)
    if not d["final"]:
        dfin = None
    t = dev_inputs(d)
    print("kda_bwd %s B=%d T=%d H=%d N=%d" % (d["name"], B, T, H, N), flush=True)
    gr = kda.bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], to_dev_bf16(dout), t["A_log"],
                 t["dt_bias"], d["lower_bound"], initial_state=t["initial_state"],
                 dfinal_state=None if dfin is None else to_dev(dfin), cu_seqlens=t["cu_seqlens"])
    torch.cuda.synchronize()
    got = {n: gr[n][:, :, h0:h0 + 1].cpu().numpy().astype(np.float64) for n in ("dq", "dk", "dv", "dg", "dbeta")}
    got["dA_log"] = gr["dA_log"][h0:h0 + 1].cpu().numpy().astype(np.float64)
    got["ddt_bias"] = gr["ddt_bias"][h0:h0 + 1].cpu().numpy().astype(np.float64)
    got["dinitial_state"] = gr["dinitial_state"][:, h0:h0 + 1].cpu().numpy().astype(np.float64)
    del gr, t
    d1 = dict(d)
    for key in ("q", "k", "v", "g", "beta"):
        d1[key] = np.ascontiguousarray(d[key][:, :, h0:h0 + 1])
    d1["A_log"] = np.ascontiguousarray(d["A_log"][h0:h0 + 1])
    d1["dt_bias"] = np.ascontiguousarray(d["dt_bias"][h0:h0 + 1])
    d1["H"] = 1
    if d["initial_state"] is not None:
        d1["initial_state"] = np.ascontiguousarray(d["initial_state"][:, h0:h0 + 1])
    d1["dout"] = np.ascontiguousarray(dout[:, :, h0:h0 + 1])
    d1["dfinal"] = None if dfin is None else np.ascontiguousarray(dfin[:, h0:h0 + 1])
    compare(d1, got, run_oracle(d1))
