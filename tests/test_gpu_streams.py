"""libkda on torch streams and inside captured HIP graphs.

Every entry point enqueues its kernels on the caller's stream only, with no
host round trip, memset or allocation inside the library, so:
* calls on two streams that overlap in time give the results of the same calls
  made one after the other (each stream has its own workspace);
* a call captured into a graph and replayed gives, bit for bit, what the eager
  call gives on the same inputs (the kernels are deterministic); the replays
  here run on fresh inputs copied into the captured tensors, with eager calls
  and synchronisations between them, and the first replay is also checked
  against the fp64 oracle.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import kda_inputs as ki
import kimi_delta_attention_fwd_amd as kda
import oracle

pytestmark = pytest.mark.gpu

REL_TOL = 1e-2
ABS_TOL = 5e-2


def _gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


def _to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _outputs(gu, d):
    out = torch.empty((d["B"], d["T"], d["H"], 128), dtype=torch.bfloat16, device=gu.DEV)
    fin = None
    if d["final"]:
        dt = torch.bfloat16 if d["state_dtype"] == "bf16" else torch.float32
        fin = torch.empty((d["N"], d["H"], 128, 128), dtype=dt, device=gu.DEV)
    return out, fin


def _fwd(d, t, out, fin):
    kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], out, t["A_log"], t["dt_bias"],
            d["lower_bound"], initial_state=t["initial_state"], final_state=fin, cu_seqlens=t["cu_seqlens"])


def _refill(gu, t, d):
    """Copy a new draw of the same shapes into the captured input tensors."""
    e = gu.dev_inputs(d)
    for key in ("q", "k", "v", "g", "beta", "A_log", "dt_bias", "initial_state"):
        if t[key] is not None:
            t[key].copy_(e[key])


def test_overlapping_streams():
    """Two side streams, each with two calls in flight, no synchronisation between
    the streams: the results equal the calls made one by one on the default stream."""
    gu = _gu()
    cases = [ki.make_inputs(1, 8192, 4, seed=40, state="fp32", initial=True),
             ki.make_inputs(1, 877, 4, seed=41, lengths=[300, 77, 500], state="bf16", initial=True)]
    ref = []
    for d in cases:
        ref.append(gu.run_gpu(d))
    dev_in = [gu.dev_inputs(d) for d in cases]
    outs = [[_outputs(gu, d) for _ in range(2)] for d in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    main = torch.cuda.current_stream()
    for s in streams:
        s.wait_stream(main)
    print("two streams: T=8192 H=4 fp32 / packed [300, 77, 500] H=4 bf16", flush=True)
    for rep in range(2):
        for i, d in enumerate(cases):
            with torch.cuda.stream(streams[i]):
                _fwd(d, dev_in[i], *outs[i][rep])
    torch.cuda.synchronize()
    for i in range(2):
        for rep in range(2):
            o, f = outs[i][rep]
            assert np.array_equal(_to_np(o), ref[i][0]), (i, rep)
            assert np.array_equal(_to_np(f), ref[i][1]), (i, rep)


@pytest.mark.parametrize("packed", [False, True])
def test_fwd_graph_replays(packed):
    gu = _gu()
    if packed:
        mk = lambda seed: ki.make_inputs(1, 1000, 3, seed=seed, lengths=[1, 400, 0, 599], state="bf16",
                                         initial=True, dt_sigma=0.1)
    else:
        mk = lambda seed: ki.make_inputs(2, 333, 3, seed=seed, state="fp32", initial=True, dt_sigma=0.1)
    d0 = mk(50)
    t = gu.dev_inputs(d0)
    out, fin = _outputs(gu, d0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _fwd(d0, t, out, fin)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    print("capture kda.fwd (packed=%s)" % packed, flush=True)
    with torch.cuda.graph(graph):
        _fwd(d0, t, out, fin)
    torch.cuda.synchronize()
    for rep in range(3):
        d = mk(60 + rep)
        _refill(gu, t, d)
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        og, fg = _to_np(out), _to_np(fin)
        oe, fe = gu.run_gpu(d)  # eager, between the replays
        assert np.array_equal(og, oe) and np.array_equal(fg, fe), rep
        if rep == 0:
            ro, rf = oracle.fwd_inputs(d, want_final=True)
            for name, got, r in (("out", og, ro), ("final", fg, rf)):
                rel, mab = oracle.rel_l2(got, r), oracle.max_abs(got, r)
                print("graph %-6s rel_l2=%.3e max_abs=%.3e" % (name, rel, mab), flush=True)
                assert rel <= REL_TOL and mab <= ABS_TOL, (name, rel, mab)


def test_decode_graph_replays():
    """A captured decode step advances the captured state once per replay, like
    the same steps made eagerly on a copy of the state."""
    gu = _gu()
    N, H = 40, 4
    mk = lambda seed: ki.make_inputs(1, N, H, seed=seed, lengths=[1] * N, state="fp32", initial=True,
                                     sigma=0.05)
    d0 = mk(70)
    tok = {key: gu.to_dev_bf16(d0[key][0]) for key in ("q", "k", "v", "g", "beta")}
    A_log, dt_bias = gu.to_dev(d0["A_log"]), gu.to_dev(d0["dt_bias"])
    state = gu.to_dev(d0["initial_state"])
    out = torch.empty_like(tok["q"])

    def step(tk, o, st):
        kda.decode(tk["q"], tk["k"], tk["v"], tk["g"], tk["beta"], d0["scale"], o, A_log, dt_bias,
                   d0["lower_bound"], st)

    eager_state = state.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    warm_state = state.clone()
    with torch.cuda.stream(side):
        step(tok, torch.empty_like(out), warm_state)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    print("capture kda.decode N=%d H=%d" % (N, H), flush=True)
    with torch.cuda.graph(graph):
        step(tok, out, state)
    torch.cuda.synchronize()
    assert torch.equal(state, eager_state)  # capture ran nothing
    for rep in range(3):
        d = mk(80 + rep)
        for key in tok:
            tok[key].copy_(gu.to_dev_bf16(d[key][0]))
        graph.replay()
        torch.cuda.synchronize()
        eo = torch.empty_like(out)
        step({key: v.clone() for key, v in tok.items()}, eo, eager_state)
        torch.cuda.synchronize()
        assert torch.equal(out, eo), rep
        assert torch.equal(state, eager_state), rep


def test_bwd_graph_replays():
    gu = _gu()
    from tests.test_gpu_backward import NAMES, case
    mk = lambda seed: case(1, 300, 2, seed, lengths=[170, 130])
    d0 = mk(90)
    t = gu.dev_inputs(d0)
    dout = gu.to_dev_bf16(d0["dout"])
    dfin = gu.to_dev(d0["dfinal"])
    grads = kda.bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], d0["scale"], dout, t["A_log"], t["dt_bias"],
                    d0["lower_bound"], initial_state=t["initial_state"], dfinal_state=dfin,
                    cu_seqlens=t["cu_seqlens"])
    torch.cuda.synchronize()

    def call(gr):
        return kda.bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], d0["scale"], dout, t["A_log"], t["dt_bias"],
                       d0["lower_bound"], initial_state=t["initial_state"], dfinal_state=dfin,
                       cu_seqlens=t["cu_seqlens"], grads=gr)

    graph = torch.cuda.CUDAGraph()
    print("capture kda.bwd packed [170, 130] H=2", flush=True)
    with torch.cuda.graph(graph):
        call(grads)
    torch.cuda.synchronize()
    for rep in range(3):
        d = mk(100 + rep)
        _refill(gu, t, d)
        dout.copy_(gu.to_dev_bf16(d["dout"]))
        dfin.copy_(gu.to_dev(d["dfinal"]))
        for n in NAMES:
            grads[n].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = {n: grads[n].clone() for n in NAMES}
        eager = call(None)
        torch.cuda.synchronize()
        for n in NAMES:
            assert torch.equal(got[n], eager[n]), (rep, n)


def test_workspace_cache_release():
    """The binding caches one forward and one backward workspace per (device,
    stream); a backward workspace above BWD_CACHE_MAX_BYTES is not kept, and
    release_workspaces() drops every cached buffer. Results do not depend on it."""
    gu = _gu()
    kda.release_workspaces()
    d = ki.make_inputs(1, 200, 2, seed=41, state="fp32", initial=True, sigma=0.05)
    o1, f1 = gu.run_gpu(d)
    keys = list(kda._ws_cache)
    assert len(keys) == 1 and keys[0][0] == "fwd"
    n = kda.release_workspaces()
    assert n >= kda.workspace_size(1, 200, 2) and not kda._ws_cache
    o2, f2 = gu.run_gpu(d)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)
    old = kda.BWD_CACHE_MAX_BYTES
    try:
        kda.BWD_CACHE_MAX_BYTES = 0  # every backward workspace counts as large
        t = gu.dev_inputs(d)
        dout = torch.ones((1, 200, 2, 128), dtype=torch.bfloat16, device=gu.DEV)
        kda.bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], dout, t["A_log"], t["dt_bias"],
                d["lower_bound"], initial_state=t["initial_state"])
        torch.cuda.synchronize()
        assert all(key[0] == "fwd" for key in kda._ws_cache)
    finally:
        kda.BWD_CACHE_MAX_BYTES = old
    kda.release_workspaces()
