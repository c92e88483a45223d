"""kda_fwd_noalloc (the forward with the library's built-in scratch instead of a
caller workspace) against kda_fwd through the C ABI: the same kernels on the
same inputs give the same bits, and both meet the oracle's tolerance bar.
Calls in a row reuse one scratch array per GPU, so the second call of each pair
runs on a smaller input over what the first one left there."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import kda_inputs as ki
import kimi_delta_attention_fwd_amd as kda
import oracle

pytestmark = pytest.mark.gpu

REL_TOL, ABS_TOL = 1e-2, 5e-2


def _gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


def _run(gu, d, noalloc):
    t = gu.dev_inputs(d)
    out = torch.full((d["B"], d["T"], d["H"], 128), float("nan"), dtype=torch.bfloat16, device=gu.DEV)
    fin = None
    if d["final"]:
        dt = torch.bfloat16 if d["state_dtype"] == "bf16" else torch.float32
        fin = torch.full((d["N"], d["H"], 128, 128), float("nan"), dtype=dt, device=gu.DEV)
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], out, t["A_log"], t["dt_bias"], d["lower_bound"])
    kw = dict(initial_state=t["initial_state"], final_state=fin, cu_seqlens=t["cu_seqlens"])
    if noalloc:
        kda.fwd_noalloc(*args, **kw)
    else:
        kda.fwd(*args, **kw)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    f = None if fin is None else fin.float().cpu().numpy().astype(np.float64)
    return o, f


def _compare(gu, d, name):
    print("noalloc case %s: B=%d T=%d H=%d" % (name, d["B"], d["T"], d["H"]), flush=True)
    o_n, f_n = _run(gu, d, noalloc=True)
    o_w, f_w = _run(gu, d, noalloc=False)
    assert np.array_equal(o_n, o_w), name
    if f_w is not None:
        assert np.array_equal(f_n, f_w), name
    ro, rf = oracle.fwd_inputs(d, want_final=d["final"])
    assert oracle.rel_l2(o_n, ro) <= REL_TOL and oracle.max_abs(o_n, ro) <= ABS_TOL, name
    assert oracle.row_rel_l2(o_n, ro)[0] <= 5e-2, name
    if f_n is not None:
        assert oracle.rel_l2(f_n, rf) <= REL_TOL and oracle.max_abs(f_n, rf) <= ABS_TOL, name
        assert oracle.row_rel_l2(f_n, rf, row_ndim=2)[0] <= 5e-2, name


def test_noalloc_matches_fwd_two_calls():
    """A packed batch (many-chain and three-wave scans, fp32 states), then a
    smaller fixed-length batch with a bf16 state, on the same scratch."""
    gu = _gu()
    lens = [1500, 0, 1, 64, 65, 300] + [37] * 60
    d1 = ki.make_inputs(1, sum(lens), 3, seed=51, lengths=lens, state="fp32", initial=True, sigma=0.05)
    assert kda.workspace_size(1, d1["T"], 3, d1["N"]) <= kda.KDA_NOALLOC_SCRATCH_BYTES
    _compare(gu, d1, "packed")
    d2 = ki.make_inputs(2, 130, 2, seed=52, state="bf16", initial=True, sigma=0.05)
    assert kda.workspace_size(2, 130, 2) < kda.workspace_size(1, d1["T"], 3, d1["N"])
    _compare(gu, d2, "small")


def test_noalloc_segmented_two_calls():
    """The segment-parallel scan keeps its segment maps and entering states in
    the workspace too: a long two-head sequence, then a shorter one."""
    gu = _gu()
    d1 = ki.make_inputs(1, 8192, 2, seed=53, state="fp32", initial=True, sigma=0.05)
    _compare(gu, d1, "segmented 8192")
    d2 = ki.make_inputs(1, 4000, 1, seed=54, state="fp32", initial=False)
    assert kda.workspace_size(1, 4000, 1) < kda.workspace_size(1, 8192, 2)
    _compare(gu, d2, "segmented 4000")


def test_noalloc_rejects_too_large():
    gu = _gu()
    d = ki.make_inputs(1, 64, 1, seed=55)
    t = gu.dev_inputs(d)
    # the long prefill's sizes need 2.4 GB of workspace: rejected before any launch
    q = torch.zeros((1, 65536, 32, 128), dtype=torch.bfloat16, device=gu.DEV)
    beta = torch.zeros((1, 65536, 32), dtype=torch.bfloat16, device=gu.DEV)
    out = torch.empty_like(q)
    A_log = torch.zeros(32, dtype=torch.float32, device=gu.DEV)
    dt_bias = torch.zeros((32, 128), dtype=torch.float32, device=gu.DEV)
    with pytest.raises(ValueError, match="KDA_ERR_SCRATCH"):
        kda.fwd_noalloc(q, q, q, q, beta, d["scale"], out, A_log, dt_bias, -5.0)
    del t
