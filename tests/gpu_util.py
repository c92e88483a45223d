"""Helpers shared by the GPU tests: move seeded numpy inputs to the device,
call the libkda binding, bring results back as float64."""
import numpy as np
import torch

import kda_inputs as ki
import kimi_delta_attention_fwd_amd as kda

DEV = "cuda:0"


def to_dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_inputs(d):
    """Device tensors for a kda_inputs dict."""
    t = dict(q=to_dev_bf16(d["q"]), k=to_dev_bf16(d["k"]), v=to_dev_bf16(d["v"]),
             g=to_dev_bf16(d["g"]), beta=to_dev_bf16(d["beta"]), A_log=to_dev(d["A_log"]),
             dt_bias=to_dev(d["dt_bias"]))
    init = d.get("initial_state")
    sd = d.get("state_dtype")
    if init is not None:
        t["initial_state"] = to_dev_bf16(init) if sd == "bf16" else to_dev(init)
    else:
        t["initial_state"] = None
    t["cu_seqlens"] = None if d.get("cu_seqlens") is None else to_dev(d["cu_seqlens"].astype(np.int32))
    return t


def run_gpu(d, t=None, final=None, out=None, workspace=None, in_place=False):
    """Run kda.fwd on a kda_inputs dict; returns (out f64, final f64 or None)."""
    if t is None:
        t = dev_inputs(d)
    B, T, H = d["B"], d["T"], d["H"]
    K, V = d.get("K", 128), d.get("V", 128)
    if out is None:
        out = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=DEV)
    if final is None:
        final = d.get("final", False)
    fin = None
    if final:
        N = d["N"]
        dt = torch.bfloat16 if d.get("state_dtype") == "bf16" else torch.float32
        if in_place and t["initial_state"] is not None:
            fin = t["initial_state"]
        else:
            fin = torch.empty((N, H, K, V), dtype=dt, device=DEV)
    kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], d["scale"], out, t["A_log"], t["dt_bias"],
            d["lower_bound"], initial_state=t["initial_state"], final_state=fin,
            cu_seqlens=t["cu_seqlens"], workspace=workspace)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    f = None if fin is None else fin.float().cpu().numpy().astype(np.float64)
    return o, f


def subset_heads(d, heads):
    """Inputs restricted to a subset of heads (the chains are independent)."""
    heads = np.asarray(heads)
    e = dict(d)
    for key in ("q", "k", "v", "g"):
        e[key] = np.ascontiguousarray(d[key][:, :, heads])
    e["beta"] = np.ascontiguousarray(d["beta"][:, :, heads])
    e["A_log"] = np.ascontiguousarray(d["A_log"][heads])
    e["dt_bias"] = np.ascontiguousarray(d["dt_bias"][heads])
    if d.get("initial_state") is not None:
        e["initial_state"] = np.ascontiguousarray(d["initial_state"][:, heads])
    e["H"] = len(heads)
    return e
