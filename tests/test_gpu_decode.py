"""GPU parity of kda_decode (one token per sequence, state in place) against
the fp64 oracle: the decode step is the per-token recurrence of the FlashKDA
pages' fwd call ("Core Kernel API / flash_kda.fwd", ccm-staging page) with one
token per sequence, so the oracle runs it as a varlen batch of length-1
sequences with initial_state = the decode state."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import kda_inputs as ki
import kimi_delta_attention_fwd_amd as kda
import oracle
from tests.gpu_util import DEV, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

# the decode path computes in fp32 end to end; only out (bf16) and a bf16 state
# are rounded, so the bounds are tighter than the chunked path's 1e-2 / 5e-2
OUT_REL, OUT_ABS = 5e-3, 2e-2


def decode_inputs(N, H, state, lower_bound=-5.0, seed=0, sigma=0.05):
    return ki.make_inputs(1, N, H, seed=seed, lengths=[1] * N, lower_bound=lower_bound, state=state,
                          initial=True, sigma=sigma)


def run_decode(d, state_t):
    q = to_dev_bf16(d["q"][0])
    k = to_dev_bf16(d["k"][0])
    v = to_dev_bf16(d["v"][0])
    g = to_dev_bf16(d["g"][0])
    beta = to_dev_bf16(d["beta"][0])
    out = torch.empty_like(q)
    kda.decode(q, k, v, g, beta, d["scale"], out, to_dev(d["A_log"]), to_dev(d["dt_bias"]), d["lower_bound"],
               state_t)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def state_dev(d):
    return to_dev_bf16(d["initial_state"]) if d["state_dtype"] == "bf16" else to_dev(d["initial_state"])


@pytest.mark.parametrize("state", ["fp32", "bf16"])
@pytest.mark.parametrize("N,H", [(1, 1), (37, 4), (256, 8)])
def test_decode_matches_oracle(state, N, H):
    d = decode_inputs(N, H, state)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    st = state_dev(d)
    go = run_decode(d, st)
    gf = st.float().cpu().numpy().astype(np.float64)
    assert oracle.rel_l2(go, ro[0]) < OUT_REL and oracle.max_abs(go, ro[0]) < OUT_ABS
    if state == "fp32":
        assert oracle.rel_l2(gf, rf) < 1e-5
    else:  # one bf16 rounding of the new state
        assert oracle.rel_l2(gf, rf) < 4e-3


@pytest.mark.parametrize("lb", [0.0, -1.0, -20.0])
def test_decode_lower_bounds(lb):
    """No chunk anchoring is involved, so bounds below the chunked path's -10 are exact too."""
    d = decode_inputs(64, 4, "fp32", lower_bound=lb, seed=3)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    st = state_dev(d)
    go = run_decode(d, st)
    assert oracle.rel_l2(go, ro[0]) < OUT_REL
    assert oracle.rel_l2(st.float().cpu().numpy().astype(np.float64), rf) < 1e-5


def test_decode_steps_equal_the_sequence():
    """T decode steps on one state equal the recurrence over a T-token sequence."""
    T, H = 24, 3
    d = ki.make_inputs(1, T, H, seed=11, lower_bound=-5.0, state="fp32", initial=True, sigma=0.05)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    st = to_dev(d["initial_state"])        # [1, H, 128, 128], updated in place step by step
    outs = []
    for t in range(T):
        e = dict(d)
        for key in ("q", "k", "v", "g", "beta"):
            e[key] = np.ascontiguousarray(d[key][:, t:t + 1])   # [1, 1, H, ...] -> N = 1 sequence
        outs.append(run_decode(e, st)[0])
    go = np.stack(outs)                     # [T, H, 128]
    assert oracle.rel_l2(go, ro[0]) < OUT_REL
    assert oracle.rel_l2(st.float().cpu().numpy().astype(np.float64), rf) < 1e-5


def test_decode_agrees_with_chunked_fwd():
    """The decode step and kda_fwd on the same length-1 varlen batch agree."""
    N, H = 96, 4
    d = decode_inputs(N, H, "fp32", seed=5)
    st = state_dev(d)
    go = run_decode(d, st)
    gf = st.float().cpu().numpy()
    q, k, v, g, beta = (to_dev_bf16(d[x]) for x in ("q", "k", "v", "g", "beta"))
    out = torch.empty_like(q)
    fin = torch.empty((N, H, 128, 128), dtype=torch.float32, device=DEV)
    kda.fwd(q, k, v, g, beta, d["scale"], out, to_dev(d["A_log"]), to_dev(d["dt_bias"]), d["lower_bound"],
            initial_state=to_dev(d["initial_state"]), final_state=fin,
            cu_seqlens=to_dev(d["cu_seqlens"].astype(np.int32)))
    torch.cuda.synchronize()
    fo = out.float().cpu().numpy()[0]
    assert oracle.rel_l2(go, fo) < 1e-2
    assert oracle.rel_l2(gf, fin.cpu().numpy()) < 1e-2


def test_decode_bench_shape():
    """The bench's decode workload (512 sequences x 64 heads, fp32 state) against
    the oracle on every sequence and head, with the per-row bound of the forward
    tests (one row per (sequence, head) output and state block)."""
    N, H = 512, 64
    d = decode_inputs(N, H, "fp32", seed=0)
    st = state_dev(d)
    go = run_decode(d, st)
    gf = st.cpu().numpy().astype(np.float64)
    ro, rf = oracle.fwd_inputs(d, want_final=True)
    assert oracle.rel_l2(go, ro[0]) < OUT_REL and oracle.max_abs(go, ro[0]) < OUT_ABS
    assert oracle.rel_l2(gf, rf) < 1e-5
    assert oracle.row_rel_l2(go, ro[0])[0] < 5e-2
    assert oracle.row_rel_l2(gf, rf, row_ndim=2)[0] < 1e-4
