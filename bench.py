#!/usr/bin/env python3
"""Throughput of the chunked Kimi Delta Attention forward (libkda) on one MI355X.

A step is one kda_fwd call (chunk map if varlen, prep kernel, scan kernel) over
one batch of seeded synthetic inputs already resident in HBM. The default
workload is the long prefill: B = 1, T = 65536, H = 32, K = V = 128, bf16
activations, lower_bound = -3, fp32 final state, no initial state.

Prints one JSON line with the throughput (token*heads/s) of K uninstrumented
steps, the HBM roofline of the step (its algorithmic bytes, 1,282 per token-head
plus the state tensors, over the step's mean duration between hipEvents on the
launch stream; the counter-measured HBM bytes of all its kernels beside them),
per-kernel figures from a second, instrumented pass, and the fp64 oracle timed on
this host's cores on the same workload; the oracle's output is also compared
with the GPU's. Workloads small enough for the 256 MB Infinity Cache to keep
between steps are timed one step at a time after a 512 MiB write (--warm skips
that).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 0..4]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA fwd tokens*heads/s + % of binding MFMA/HBM roofline, T=64K H=32"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
# algorithmic HBM bytes per token-head at K = V = D: q, k, g, v reads (4 x 2 D),
# out write (2 D), beta (2)
def prep_bytes_per_th(D=128):
    return 4 * 2 * D + 2


def scan_bytes_per_th(D=128):
    return 2 * D


PREP_BYTES_PER_TH = prep_bytes_per_th()
SCAN_BYTES_PER_TH = scan_bytes_per_th()
# HBM bytes per launch read from rocprofv3 FETCH_SIZE / WRITE_SIZE counters,
# scaled by the same counters' reading for a device copy of known size; valid
# only while the kernel's sources hash to the recorded value
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
CSRC = os.path.join(ROOT, "kimi_delta_attention_fwd_amd", "csrc")
KERNEL_SOURCES = {"kda_prep": ("kda_prep.hip", "kda_device.h", "kda_internal.h", "../../include/kda.h", "../build.py"),
                  "kda_scan": ("kda_scan.hip", "kda_scan_pair.hip", "kda_device.h", "kda_internal.h", "../build.py"),
                  "kda_decode": ("kda_decode.hip", "kda_device.h", "kda_internal.h"),
                  "kda_bwd_chunk": ("kda_bwd.hip", "kda_device.h", "kda_internal.h"),
                  "kda_bwd_scan": ("kda_bwd.hip", "kda_device.h", "kda_internal.h"),
                  "kda_bwd_grad": ("kda_bwd.hip", "kda_device.h", "kda_internal.h"),
                  "kda_bwd_reduce": ("kda_bwd.hip", "kda_device.h", "kda_internal.h")}
# algorithmic MFMA flops per token-head with 16x16 blocks and 64-token chunks:
# state-side 6*K*V + intra-chunk 2*C*(3K + 2V)
def flops_per_th(D=128):
    return 6 * D * D + 2 * 64 * (3 * D + 2 * D)


FLOPS_PER_TH = flops_per_th()


# backward: published fp32 vector peak of MI355X, and algorithmic flops per
# token-head of the gradient kernel (64-token chunks, K = V = 128):
# its products per (chunk, head) are 5 of 64x128x128 and 8 of 64x64x128 (or
# 64x128x64), T^T dT (64^3) and the lower triangle of X1 T^T (64^3 / 2), 2 flops
# per multiply-add; the two pairwise passes take 17 flops per (i, j <= i, channel)
PEAK_FP32_TFLOPS = 157.3
# algorithmic HBM bytes per token-head of the backward: q, k, g, v, dout read in
# bf16 (5 x 256), beta 2; dq, dk, dg, dv written in fp32 (4 x 512), dbeta 4
BWD_BYTES_PER_TH = 5 * 256 + 2 + 4 * 512 + 4
BWD_GRAD_FLOPS_PER_TH = (2 * (5 * 64 * 128 * 128 + 8 * 64 * 64 * 128 + 64 ** 3 + 64 ** 3 // 2)
                         + 17 * (64 * 65 // 2) * 128) / 64.0


# Infinity Cache (MALL) of the MI355X
MALL_BYTES = 256 << 20
# the long-prefill scan's kernel time in the committed kernel-stats profile; the
# bench flags a run where it is more than 3 % slower (its warming loop's place
# relative to instruction-fetch blocks moved it by up to 6 %)
SCAN_REF_MS = {"long_prefill": 0.996}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def state_bytes(d):
    if d["state_dtype"] is None:
        return 0
    D = d.get("K", 128)
    per = D * D * (4 if d["state_dtype"] == "fp32" else 2)
    n = (1 if d["initial_state"] is not None else 0) + (1 if d["final"] else 0)
    return n * d["N"] * d["H"] * per


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, ()):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, counter=None):
    """HBM bytes per launch of ``kernel`` on ``workload`` from the counter
    summary (or, with ``counter``, that counter line's value), or None if there
    is none for the current sources."""
    if kernel not in KERNEL_SOURCES or not os.path.exists(TRAFFIC_FILE):
        return None
    want = kernel_source_hash(kernel)
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if line.startswith("#"):
                continue
            f = dict(kv.split("=", 1) for kv in line.split() if "=" in kv)
            if f.get("kernel") == kernel and f.get("workload") == workload and f.get("src") == want \
                    and f.get("counter") == counter:
                return float(f["value" if counter else "hbm_bytes"])
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload 0..4 (default: 3, the long prefill)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="prefix length on which the oracle is timed, all heads (0: the whole workload)")
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0,
                    help="repeat the oracle over the sample until this much time has passed")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle leg")
    ap.add_argument("--decode", action="store_true",
                    help="time the single-token decode step instead (512 sequences x 64 heads, fp32 state)")
    ap.add_argument("--backward", action="store_true",
                    help="time kda_bwd (gradients) on the workload instead of the forward")
    ap.add_argument("--lower-bound", type=float, default=None,
                    help="override the workload's lower_bound (below -10 selects the wide-range chunk preparation)")
    ap.add_argument("--heads", type=int, default=0,
                    help="keep only the first N heads of the workload (one GPU's share when heads are sharded)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after timing, run 3 device copies of this many MiB (counter calibration)")
    ap.add_argument("--head-dim", type=int, default=128, choices=(128, 64),
                    help="K = V of the workload (the forward also takes 64)")
    ap.add_argument("--warm", action="store_true",
                    help="never flush the Infinity Cache between steps (small workloads are flushed by default)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: libkda has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kda_inputs as ki
    import kimi_delta_attention_fwd_amd as kda

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    kda.load_library()
    if args.head_dim != 128 and (args.decode or args.backward):
        print("bench.py: --decode and --backward run at K = V = 128 only", file=sys.stderr)
        sys.exit(2)
    if args.decode:
        return run_decode(args)
    if args.backward:
        return run_backward(args)
    dev = "cuda:0"
    t_gen = time.time()
    d = ki.config_inputs(args.config, head_dim=args.head_dim)
    HD = args.head_dim
    if HD != 128:
        d["name"] = "%s_k%d" % (d["name"], HD)
    if 0 < args.heads < d["H"]:
        nh = args.heads
        for key in ("q", "k", "v", "g", "beta"):
            d[key] = np.ascontiguousarray(d[key][:, :, :nh])
        for key in ("A_log", "dt_bias"):
            d[key] = np.ascontiguousarray(d[key][:nh])
        if d["initial_state"] is not None:
            d["initial_state"] = np.ascontiguousarray(d["initial_state"][:, :nh])
        d["H"] = nh
        d["name"] = "%s_h%d" % (d["name"], nh)
    if args.lower_bound is not None:
        d["lower_bound"] = float(args.lower_bound)
        d["name"] = "%s_lb%g" % (d["name"], args.lower_bound)
    print("[bench] inputs for workload %d (%s) drawn in %.1f s" % (args.config, d["name"], time.time() - t_gen),
          file=sys.stderr, flush=True)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v, g, beta = bf(d["q"]), bf(d["k"]), bf(d["v"]), bf(d["g"]), bf(d["beta"])
    A_log = torch.from_numpy(d["A_log"]).to(dev)
    dt_bias = torch.from_numpy(d["dt_bias"]).to(dev)
    sdt = torch.float32 if d["state_dtype"] == "fp32" else torch.bfloat16
    init = None
    if d["initial_state"] is not None:
        init = torch.from_numpy(d["initial_state"]).to(dev) if sdt == torch.float32 else bf(d["initial_state"])
    fin = torch.empty((d["N"], d["H"], HD, HD), dtype=sdt, device=dev) if d["final"] else None
    cu = None if d["cu_seqlens"] is None else torch.from_numpy(d["cu_seqlens"]).to(dev)
    B, T, H = d["B"], d["T"], d["H"]
    out = torch.empty((B, T, H, HD), dtype=torch.bfloat16, device=dev)
    nseq = 0 if cu is None else d["N"]
    ws = torch.empty(kda.workspace_size(B, T, H, nseq), dtype=torch.uint8, device=dev)

    def step():
        kda.fwd(q, k, v, g, beta, d["scale"], out, A_log, dt_bias, d["lower_bound"],
                initial_state=init, final_state=fin, cu_seqlens=cu, workspace=ws)

    th = ki.token_heads(d)
    path_bytes = th * (prep_bytes_per_th(HD) + scan_bytes_per_th(HD)) + state_bytes(d)
    # The 256 MB Infinity Cache (MALL) keeps a small workload's inputs between
    # steps. Working sets below twice its size are timed one step at a time with
    # a 512 MiB write between steps (outside the timed events), unless --warm.
    flush = (not args.warm) and (path_bytes + ws.numel() < 2 * MALL_BYTES)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if not flush:
        # the timed region: K uninstrumented steps, synchronised on both sides
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record()
        for _ in range(args.steps):
            step()
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        event_ms = ev0.elapsed_time(ev1) / args.steps
        ms_per_step = wall / args.steps * 1e3
        ws_bytes = path_bytes + ws.numel()
        mall = ("cold: the step moves %.2f GB, more than twice the 256 MB Infinity Cache" % (ws_bytes / 1e9)
                if ws_bytes >= 2 * MALL_BYTES else
                "warm: the step's %.0f MB may stay in the 256 MB Infinity Cache between steps" % (ws_bytes / 1e6))
    else:
        sink = torch.empty(MALL_BYTES * 2, dtype=torch.uint8, device=dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for a, b in evs:
            sink.fill_(1)
            a.record()
            step()
            b.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        event_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
        ms_per_step = event_ms
        mall = "flushed: a 512 MiB write before each step, steps timed one by one with events"
        del sink
    value = th / (ms_per_step * 1e-3)

    # per-kernel times: a second pass of K steps with the library's own events
    # around each kernel (not part of the timed region above)
    kda.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kda.profile_enable(False)
    prof = kda.profile_read()

    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    kernels = {name: tot / cnt for name, (tot, cnt) in prof.items()}
    alg_bytes = {"kda_prep": th * prep_bytes_per_th(HD),
                 "kda_scan": th * scan_bytes_per_th(HD) + state_bytes(d),
                 "kda_chunk_map": 0}
    per_kernel = {}
    for name, ms in kernels.items():
        per_kernel[name] = {"ms": ms, "alg_bytes": alg_bytes.get(name, 0),
                            "frac_hbm": alg_bytes.get(name, 0) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                            "traffic": measured_traffic(name, d["name"])}
    dom = max(kernels, key=kernels.get)
    # counter-measured HBM bytes of the whole step: every kernel of the call must
    # have a figure for the current sources (the chunk map moves a few KB)
    traffic = 0.0
    for name in kernels:
        t = per_kernel[name]["traffic"]
        if t is None and name != "kda_chunk_map":
            traffic = None
            break
        traffic += t or 0.0
    achieved = path_bytes / (event_ms * 1e-3) / 1e9
    path_tflops = th * flops_per_th(HD) / (event_ms * 1e-3) / 1e12
    # bf16 MFMA flops the counters saw per launch (prep selector MFMAs included)
    mfma_counted = 0.0
    for name in kernels:
        if name == "kda_chunk_map":
            continue
        c = measured_traffic(name, d["name"], counter="mfma_bf16_flops")
        if c is None:
            mfma_counted = None
            break
        mfma_counted += c

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "token*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy draws, recipe in kda_inputs)",
        "config": {"workload": "%s: B=%d T=%d H=%d K=V=%d chunk=64 lower_bound=%g state=%s%s" % (
            d["name"], B, T, H, HD, d["lower_bound"], d["state_dtype"],
            " varlen N=%d" % d["N"] if cu is not None else ""),
            "global_batch": B, "seq_len": T, "heads": H, "parallelism": "single GPU"},
        # the unit of the roofline is one whole kda_fwd call (all of its kernels):
        # the algorithmic bytes of the step (1,282 B per token-head plus the state
        # tensors) over the step's mean duration between hipEvents on the launch
        # stream in the timed region
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "traffic_ratio": None if traffic is None else traffic / path_bytes,
                     "kernel": "kda_fwd step (%s)" % ", ".join(sorted(kernels)),
                     "launch_ms": event_ms, "alg_bytes_per_launch": path_bytes,
                     "mfma_frac": path_tflops / PEAK_BF16_TFLOPS,
                     "mfma_frac_counter": None if mfma_counted is None else
                     mfma_counted / (event_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
        "kernels": per_kernel,
        "dominant_kernel": dom,
        "mall": mall,
        "event_ms_per_step": event_ms,
    }
    ref = SCAN_REF_MS.get(d["name"])
    if ref is not None and "kda_scan" in kernels:
        res["scan_placement_check"] = {"ref_ms": ref, "ms": kernels["kda_scan"],
                                       "ok": kernels["kda_scan"] <= 1.03 * ref}
        if kernels["kda_scan"] > 1.03 * ref:
            print("[bench] warning: kda_scan took %.3f ms, more than 3%% over its reference %.3f ms (instruction "
                  "placement of its warming loop?)" % (kernels["kda_scan"], ref), file=sys.stderr, flush=True)

    if not args.no_cpu:
        import oracle
        ts = T if (cu is not None or args.cpu_sample_tokens <= 0) else min(args.cpu_sample_tokens, T)
        if cu is None:
            sub = dict(d)
            for key in ("q", "k", "v", "g", "beta"):
                sub[key] = np.ascontiguousarray(d[key][:, :ts])
            sub["T"] = ts
        else:
            sub = d
        threads = oracle.max_threads()
        tc, reps = 0.0, 0
        while reps == 0 or tc < args.cpu_min_seconds:
            tc0 = time.perf_counter()
            ro, _ = oracle.fwd_inputs(sub, want_final=False)
            tc += time.perf_counter() - tc0
            reps += 1
        sample_th = ki.token_heads(sub)
        got = out[:, :sub["T"]].float().cpu().numpy()
        res["cpu_baseline"] = {"value": reps * sample_th / tc, "unit": "token*heads/s", "cores": threads,
                               "kind": "oracle", "cpu": cpu_model(),
                               "sample": "fp64 per-token recurrence on %s (%d tokens x %d heads = %d token-heads), "
                                         "%d passes in %.1f s" % (
                                             "the whole workload" if sub["T"] == T else
                                             "the first %d tokens of the workload" % sub["T"],
                                             sub["T"], H, sample_th, reps, tc)}
        res["parity_sample"] = {"rel_l2": oracle.rel_l2(got, ro), "max_abs": oracle.max_abs(got, ro),
                                "tokens": sub["T"]}
    print(json.dumps(res), flush=True)


DECODE_N, DECODE_H = 512, 64


def run_decode(args):
    """One kda_decode call per step on 512 sequences x 64 heads with an fp32
    state updated in place (the decode neighbour of the continuation workload).
    Algorithmic bytes per (sequence, head): the fp32 state read and written
    (2 x 64 KiB), q, k, v, g read and out written (5 x 256 B), beta (2 B)."""
    import numpy as np
    import torch

    import kda_inputs as ki
    import kimi_delta_attention_fwd_amd as kda

    dev = "cuda:0"
    N, H = DECODE_N, DECODE_H
    d = ki.make_inputs(1, N, H, seed=0, lengths=[1] * N, lower_bound=-5.0, state="fp32", initial=True,
                       sigma=0.05)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v, g, beta = (bf(d[x][0]) for x in ("q", "k", "v", "g", "beta"))
    A_log = torch.from_numpy(d["A_log"]).to(dev)
    dt_bias = torch.from_numpy(d["dt_bias"]).to(dev)
    state = torch.from_numpy(d["initial_state"]).to(dev)
    out = torch.empty_like(q)
    state0 = state.clone()

    def step():
        kda.decode(q, k, v, g, beta, d["scale"], out, A_log, dt_bias, d["lower_bound"], state)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: K uninstrumented calls; the kernel time from a second,
    # instrumented pass
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kda.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kda.profile_enable(False)
    prof = kda.profile_read()
    kern_ms = prof["kda_decode"][0] / prof["kda_decode"][1]
    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    units = N * H
    alg = units * (2 * 128 * 128 * 4 + 5 * 256 + 2) + H * 4 + H * 128 * 4
    achieved = alg / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": "KDA decode step tokens*heads/s (one token per sequence, state in place)",
        "value": units * args.steps / wall, "unit": "token*heads/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded numpy draws)",
        "config": {"workload": "decode: N=%d sequences x H=%d heads, one token each, fp32 state" % (N, H),
                   "global_batch": N, "seq_len": 1, "heads": H, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic("kda_decode", "decode"),
                     "kernel": "kda_decode",
                     "kernel_ms": kern_ms, "alg_bytes_per_launch": alg},
    }
    if not args.no_cpu:
        import oracle
        tc, reps = 0.0, 0
        while reps == 0 or tc < args.cpu_min_seconds:
            tc0 = time.perf_counter()
            ro, rf = oracle.fwd_inputs(d, want_final=True)
            tc += time.perf_counter() - tc0
            reps += 1
        res["cpu_baseline"] = {"value": reps * units / tc, "unit": "token*heads/s", "cores": oracle.max_threads(),
                               "kind": "oracle", "cpu": cpu_model(), "sample": "fp64 recurrence on the whole workload (%d "
                               "token-heads), %d passes in %.1f s" % (units, reps, tc)}
        # parity of one step from the initial state
        state.copy_(state0)
        step()
        torch.cuda.synchronize()
        res["parity_sample"] = {"rel_l2": oracle.rel_l2(out.float().cpu().numpy(), ro[0]),
                                "state_rel_l2": oracle.rel_l2(state.cpu().numpy(), rf)}
    print(json.dumps(res), flush=True)


def run_backward(args):
    """One kda_bwd call per step on a workload of the forward (default: the long
    prefill), with a seeded bf16 output gradient and an fp32 final-state gradient
    where the workload returns a final state."""
    import numpy as np
    import torch

    import kda_inputs as ki
    import kimi_delta_attention_fwd_amd as kda

    dev = "cuda:0"
    d = ki.config_inputs(args.config)
    if 0 < args.heads < d["H"]:
        nh = args.heads
        for key in ("q", "k", "v", "g", "beta"):
            d[key] = np.ascontiguousarray(d[key][:, :, :nh])
        for key in ("A_log", "dt_bias"):
            d[key] = np.ascontiguousarray(d[key][:nh])
        if d["initial_state"] is not None:
            d["initial_state"] = np.ascontiguousarray(d["initial_state"][:, :nh])
        d["H"] = nh
        d["name"] = "%s_h%d" % (d["name"], nh)
    B, T, H, N = d["B"], d["T"], d["H"], d["N"]
    rng = np.random.default_rng(1234)
    dout_np = ki.f32_to_bf16_bits(rng.standard_normal((B, T, H, 128), dtype=np.float32))
    dfin_np = (rng.standard_normal((N, H, 128, 128), dtype=np.float32) * np.float32(0.1)) if d["final"] else None
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v, g, beta, dout = bf(d["q"]), bf(d["k"]), bf(d["v"]), bf(d["g"]), bf(d["beta"]), bf(dout_np)
    A_log = torch.from_numpy(d["A_log"]).to(dev)
    dt_bias = torch.from_numpy(d["dt_bias"]).to(dev)
    init = None
    if d["initial_state"] is not None:
        init = torch.from_numpy(d["initial_state"]).to(dev) if d["state_dtype"] == "fp32" else bf(d["initial_state"])
    dfin = None if dfin_np is None else torch.from_numpy(dfin_np).to(dev)
    cu = None if d["cu_seqlens"] is None else torch.from_numpy(d["cu_seqlens"]).to(dev)
    nseq = 0 if cu is None else N
    ws = torch.empty(kda.bwd_workspace_size(B, T, H, nseq), dtype=torch.uint8, device=dev)
    f32 = torch.float32
    grads = dict(dq=torch.empty((B, T, H, 128), dtype=f32, device=dev),
                 dk=torch.empty((B, T, H, 128), dtype=f32, device=dev),
                 dv=torch.empty((B, T, H, 128), dtype=f32, device=dev),
                 dg=torch.empty((B, T, H, 128), dtype=f32, device=dev),
                 dbeta=torch.empty((B, T, H), dtype=f32, device=dev),
                 dA_log=torch.empty((H,), dtype=f32, device=dev),
                 ddt_bias=torch.empty((H, 128), dtype=f32, device=dev),
                 dinitial_state=torch.empty((N, H, 128, 128), dtype=f32, device=dev))

    def step():
        kda.bwd(q, k, v, g, beta, d["scale"], dout, A_log, dt_bias, d["lower_bound"], initial_state=init,
                dfinal_state=dfin, cu_seqlens=cu, grads=grads, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: K uninstrumented calls, synchronised on both sides
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    event_ms = ev0.elapsed_time(ev1) / args.steps
    # per-kernel times from a second, instrumented pass
    kda.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kda.profile_enable(False)
    prof = kda.profile_read()
    kern = {name: ms / n for name, (ms, n) in prof.items()}
    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    units = ki.token_heads(d)
    grad_ms = kern["kda_bwd_grad"]
    grad_tflops = units * BWD_GRAD_FLOPS_PER_TH / (grad_ms * 1e-3) / 1e12
    # the step's algorithmic bytes: activations, output gradient and gradients,
    # plus the initial state read, the final-state gradient read and the
    # initial-state gradient written
    sb = 128 * 128
    state_b = N * H * sb * ((4 if d["state_dtype"] == "fp32" else 2) if init is not None else 0)
    state_b += N * H * sb * 4 * ((1 if dfin is not None else 0) + 1)
    step_bytes = units * BWD_BYTES_PER_TH + state_b
    traffic = 0.0
    per_kernel = {}
    for name, ms in kern.items():
        t = measured_traffic(name, d["name"] + "_backward")
        per_kernel[name] = {"ms": ms, "traffic": t,
                            "traffic_frac_hbm": None if t is None else t / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
        traffic = None if (traffic is None or t is None) else traffic + t
    achieved = step_bytes / (event_ms * 1e-3) / 1e9
    res = {
        "metric": "KDA bwd tokens*heads/s (gradients of q, k, v, g, beta, A_log, dt_bias, initial state)",
        "value": units * args.steps / wall, "unit": "token*heads/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded numpy draws)",
        "config": {"workload": "%s backward: B=%d T=%d H=%d, bf16 inputs, fp32 gradients" % (d["name"], B, T, H),
                   "global_batch": B, "seq_len": T, "heads": H, "parallelism": "single GPU"},
        # the whole kda_bwd call against the HBM roofline with its algorithmic
        # bytes; the counters show what the kernels actually move (the gradient
        # kernel's product operands go through HBM: traffic_ratio), and the
        # gradient kernel's algorithmic flops against the fp32 vector peak
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "traffic_ratio": None if traffic is None else traffic / step_bytes,
                     "kernel": "kda_bwd step (%s)" % ", ".join(sorted(kern)), "launch_ms": event_ms,
                     "alg_bytes_per_launch": step_bytes,
                     "grad_kernel_fp32": {"achieved": grad_tflops, "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                                          "frac": grad_tflops / PEAK_FP32_TFLOPS, "kernel_ms": grad_ms,
                                          "alg_flops_per_launch": units * BWD_GRAD_FLOPS_PER_TH}},
        "kernels": per_kernel,
        "kernels_ms": kern,
    }
    if not args.no_cpu:
        from threadpoolctl import threadpool_limits

        from oracle import backward as obwd
        # the numpy reverse pass is single-threaded (per-token steps on small
        # matrices; threads over heads measured slower, the interpreter lock)
        ts = min(T, 256)
        sub = lambda a: None if a is None else np.ascontiguousarray(a[:, :ts])
        tc, reps = 0.0, 0
        with threadpool_limits(1):
            while reps == 0 or tc < args.cpu_min_seconds:
                tc0 = time.perf_counter()
                obwd.bwd(sub(d["q"][:1]), sub(d["k"][:1]), sub(d["v"][:1]), sub(d["g"][:1]), sub(d["beta"][:1]),
                         d["scale"], d["A_log"], d["dt_bias"], d["lower_bound"], sub(dout_np[:1]))
                tc += time.perf_counter() - tc0
                reps += 1
        res["cpu_baseline"] = {"value": reps * ts * H / tc, "unit": "token*heads/s", "cores": 1, "kind": "oracle",
                               "cpu": cpu_model(),
                               "sample": "fp64 per-token reverse pass on the first %d tokens of sequence 0, all %d "
                               "heads, %d passes in %.1f s" % (ts, H, reps, tc)}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
