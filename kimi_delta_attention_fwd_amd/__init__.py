"""MI355X-native chunked forward of Kimi Delta Attention (libkda).

``fwd`` mirrors the ``flash_kda.fwd`` call named on the FlashKDA pages
("Core Kernel API / flash_kda.fwd", ccm-staging page; constraints in
"Kernel API and Constraints", trend.ondo.sh page): q, k, v, g, beta, scale, out,
A_log, dt_bias, lower_bound, initial_state, final_state, cu_seqlens. It writes
``out`` (and ``final_state``) in place.

This module only marshals arguments: torch supplies device memory and the
current stream, and every step of the computation runs in the HIP kernels of
``libkda.so`` (built in-tree by ``build.py``). There is no fallback: if the
library is missing, or no GPU is present, calls raise.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["fwd", "fwd_noalloc", "decode", "bwd", "workspace_size", "bwd_workspace_size", "status_string", "library_path", "load_library",
           "profile_enable", "profile_read", "release_workspaces", "KDA_LOWER_BOUND_NARROW", "KDA_MAX_HEADS",
           "KdaError"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkda.so")
_lib = None

KDA_STATE_NONE, KDA_STATE_BF16, KDA_STATE_FP32 = 0, 1, 2
KDA_LOWER_BOUND_NARROW = -10.0  # below it kda_fwd takes its wide-range chunk preparation
KDA_MAX_HEADS = 65536  # H limit of kda_fwd and kda_decode (KDA_ERR_SHAPE above it)
EXPORTED = ("kda_fwd", "kda_fwd_noalloc", "kda_decode", "kda_fwd_workspace_size", "kda_status_string",
            "kda_profile_enable", "kda_profile_read", "kda_bwd", "kda_bwd_workspace_size")
KDA_ERR_HIP = 8
KDA_NOALLOC_SCRATCH_BYTES = 256 << 20  # built-in scratch of kda_fwd_noalloc, per GPU


class KdaError(RuntimeError):
    """A HIP launch/runtime error reported by libkda (status KDA_ERR_HIP)."""


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch ships its own HIP runtime; it must be the one in the process before
    # libkda binds to a HIP runtime, or libkda would load a second copy and its
    # launches on torch's memory and streams fail (KDA_ERR_HIP)
    import torch  # noqa: F401
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libkda.so is not built: run `python -c \"import __graft_entry__ as e; e.build()\"` "
                           "or `python kimi_delta_attention_fwd_amd/build.py`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.kda_fwd.restype = ctypes.c_int
    lib.kda_fwd.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, P, ctypes.c_float, P, P,
                            ctypes.c_int, P, I64, I64, I64, I64, I64, I64, P, ctypes.c_size_t, P]
    lib.kda_fwd_noalloc.restype = ctypes.c_int
    lib.kda_fwd_noalloc.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, P, ctypes.c_float, P, P,
                                    ctypes.c_int, P, I64, I64, I64, I64, I64, I64, P]
    lib.kda_decode.restype = ctypes.c_int
    lib.kda_decode.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, P, ctypes.c_float, P, ctypes.c_int,
                               I64, I64, I64, I64, P]
    lib.kda_bwd.restype = ctypes.c_int
    lib.kda_bwd.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, P, ctypes.c_float, P, ctypes.c_int, P,
                            P, I64, I64, I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.kda_bwd_workspace_size.restype = ctypes.c_size_t
    lib.kda_bwd_workspace_size.argtypes = [I64, I64, I64, I64]
    lib.kda_fwd_workspace_size.restype = ctypes.c_size_t
    lib.kda_fwd_workspace_size.argtypes = [I64, I64, I64, I64]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_profile_enable.restype = ctypes.c_int
    lib.kda_profile_enable.argtypes = [ctypes.c_int]
    lib.kda_profile_read.restype = ctypes.c_int
    lib.kda_profile_read.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float),
                                     ctypes.POINTER(ctypes.c_int), ctypes.c_int]
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().kda_status_string(int(code)).decode()


def workspace_size(B: int, T: int, H: int, num_seqs: int = 0) -> int:
    """Bytes of device workspace ``fwd`` needs (num_seqs = 0: no cu_seqlens)."""
    return int(load_library().kda_fwd_workspace_size(int(B), int(T), int(H), int(num_seqs)))


def bwd_workspace_size(B: int, T: int, H: int, num_seqs: int = 0) -> int:
    """Bytes of device workspace ``bwd`` needs (num_seqs = 0: no cu_seqlens)."""
    return int(load_library().kda_bwd_workspace_size(int(B), int(T), int(H), int(num_seqs)))


def profile_enable(on: bool = True) -> None:
    """Start (clearing earlier records) or stop per-kernel event timing."""
    rc = load_library().kda_profile_enable(1 if on else 0)
    if rc != 0:
        raise KdaError(status_string(rc))


def profile_read(cap: int = 8):
    """{kernel name: (total ms, launches)} over the profiled calls (synchronises)."""
    lib = load_library()
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_float * cap)()
    counts = (ctypes.c_int * cap)()
    n = lib.kda_profile_read(names, ms, counts, cap)
    if n < 0:
        raise KdaError("kda_profile_read failed")
    return {names[i].decode(): (float(ms[i]), int(counts[i])) for i in range(n)}


_ws_cache = {}
# backward workspaces larger than this are allocated per call and not kept
# (the long prefill's is 13.5 GB)
BWD_CACHE_MAX_BYTES = 1 << 30


def _workspace(nbytes, device, kind="fwd"):
    """Workspace for a call on the current stream of ``device``.

    One cached buffer per (kind, device, stream), kind "fwd" or "bwd": calls on
    one stream run in order and may share it, calls on different streams may
    overlap and must not (the caching allocator also ties a buffer to the stream
    it was allocated on, so a buffer outgrown on one stream is only recycled after
    that stream's work). Forward and backward keep separate buffers, and a
    backward workspace above BWD_CACHE_MAX_BYTES is not cached at all, so one
    large backward call does not pin its workspace for the later forward calls.
    During graph capture the buffer is allocated per call from the graph's
    memory pool, which keeps it reserved for every replay.
    ``release_workspaces`` drops the cached buffers.
    """
    import torch
    stream = torch.cuda.current_stream(device)
    n = max(nbytes, 256)
    if torch.cuda.is_current_stream_capturing():
        return torch.empty(n, dtype=torch.uint8, device=device)
    if kind == "bwd" and n > BWD_CACHE_MAX_BYTES:
        return torch.empty(n, dtype=torch.uint8, device=device)
    key = (kind, str(device), stream.cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < n:
        _ws_cache.pop(key, None)
        buf = torch.empty(n, dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def release_workspaces() -> int:
    """Drop every cached workspace buffer (their memory returns to torch's
    caching allocator once the streams that used them are done with it).
    Returns the number of bytes released."""
    n = sum(int(b.numel()) for b in _ws_cache.values())
    _ws_cache.clear()
    return n


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _fwd_args(q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state, cu_seqlens, workspace):
    """Check dtypes, devices, contiguity and shapes on the host; returns
    (state_dtype, num_seqs, B, T, H, K, V)."""
    import torch
    bf16 = torch.bfloat16
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("out", out)):
        if t.dtype != bf16:
            raise ValueError("%s must be bfloat16 (got %s)" % (name, t.dtype))
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        if t.dtype != torch.float32:
            raise ValueError("%s must be float32 (got %s)" % (name, t.dtype))
    tensors = [q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state, cu_seqlens, workspace]
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, K]")
    B, T, H, K = q.shape
    V = v.shape[-1]
    for name, t in (("k", k), ("g", g)):
        if tuple(t.shape) != (B, T, H, K):
            raise ValueError("%s must have the shape of q" % name)
    if tuple(v.shape) != (B, T, H, V) or tuple(out.shape) != (B, T, H, V):
        raise ValueError("v and out must be [B, T, H, V]")
    if tuple(beta.shape) != (B, T, H):
        raise ValueError("beta must be [B, T, H]")
    if A_log.numel() != H or dt_bias.numel() != H * K:
        raise ValueError("A_log must have H elements and dt_bias H*K")
    num_seqs = 0
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32:
            raise ValueError("cu_seqlens must be int32")
        num_seqs = cu_seqlens.numel() - 1
        if num_seqs <= 0:
            raise ValueError("cu_seqlens must have at least 2 entries")
    sd = KDA_STATE_NONE
    states = [s for s in (initial_state, final_state) if s is not None]
    if states:
        dts = {s.dtype for s in states}
        if len(dts) != 1:
            raise ValueError("initial_state and final_state must have the same dtype")
        dt = dts.pop()
        if dt == torch.float32:
            sd = KDA_STATE_FP32
        elif dt == bf16:
            sd = KDA_STATE_BF16
        else:
            raise ValueError("states must be bfloat16 or float32")
        N = num_seqs if cu_seqlens is not None else B
        for s in states:
            if tuple(s.shape) != (N, H, K, V):
                raise ValueError("states must be [N, H, K, V] = %s" % ((N, H, K, V),))
    return sd, num_seqs, B, T, H, K, V


def _check(lib, rc):
    if rc == 0:
        return
    msg = lib.kda_status_string(rc).decode()
    if rc == KDA_ERR_HIP:
        raise KdaError(msg)
    raise ValueError(msg)


def fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
        initial_state=None, final_state=None, cu_seqlens=None, workspace=None):
    """Chunked KDA forward on the current torch (ROCm) stream; fills ``out``.

    q, k, g: bf16 [B, T, H, 128]; v, out: bf16 [B, T, H, 128]; beta: bf16
    [B, T, H]; A_log: fp32 [H]; dt_bias: fp32 [H, 128]; lower_bound: finite,
    <= 0; initial_state / final_state: None or
    [N, H, 128, 128] of one dtype (bf16 or fp32), final_state may be the same
    tensor as initial_state; cu_seqlens: None or int32 [N + 1] on the device
    (B must be 1). ``workspace`` (optional) is a uint8 device tensor of at least
    ``workspace_size`` bytes; by default a cached buffer is used.
    Raises ValueError for invalid arguments and KdaError for HIP failures.
    """
    import torch
    lib = load_library()
    sd, num_seqs, B, T, H, K, V = _fwd_args(q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state,
                                            cu_seqlens, workspace)
    need = lib.kda_fwd_workspace_size(B, T, H, num_seqs)
    if workspace is None:
        ws = _workspace(need, q.device)
    else:
        ws = workspace
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib.kda_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(out),
                     _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state),
                     _ptr(final_state), sd, _ptr(cu_seqlens), num_seqs, B, T, H, K, V,
                     _ptr(ws), ws.numel(), ctypes.c_void_p(stream))
    _check(lib, rc)
    return out


def fwd_noalloc(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
                initial_state=None, final_state=None, cu_seqlens=None):
    """``fwd`` through kda_fwd_noalloc: the workspace is the library's built-in
    scratch array of the GPU (KDA_NOALLOC_SCRATCH_BYTES), so the call allocates
    nothing, neither in libkda nor here. Same arguments and results as ``fwd``;
    sizes whose workspace exceeds the scratch raise ValueError
    (KDA_ERR_SCRATCH). Calls that may overlap in time on one GPU share the
    scratch and must be serialised by the caller.
    """
    import torch
    lib = load_library()
    sd, num_seqs, B, T, H, K, V = _fwd_args(q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state,
                                            cu_seqlens, None)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib.kda_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(out),
                             _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state),
                             _ptr(final_state), sd, _ptr(cu_seqlens), num_seqs, B, T, H, K, V,
                             ctypes.c_void_p(stream))
    _check(lib, rc)
    return out


def decode(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, state):
    """One token per sequence, state updated in place, on the current torch stream.

    q, k, v, g, out: bf16 [N, H, 128]; beta: bf16 [N, H]; A_log: fp32 [H];
    dt_bias: fp32 [H, 128]; lower_bound: finite, <= 0; state: [N, H, 128, 128]
    bf16 or fp32 (read, then overwritten with the state after the token).
    The same step as ``fwd`` with one token per sequence and
    initial_state = final_state = state. Raises ValueError for invalid
    arguments and KdaError for HIP failures.
    """
    import torch
    lib = load_library()
    bf16 = torch.bfloat16
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("out", out)):
        if t.dtype != bf16:
            raise ValueError("%s must be bfloat16 (got %s)" % (name, t.dtype))
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        if t.dtype != torch.float32:
            raise ValueError("%s must be float32 (got %s)" % (name, t.dtype))
    for t in (q, k, v, g, beta, out, A_log, dt_bias, state):
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if q.dim() != 3:
        raise ValueError("q must be [N, H, K]")
    N, H, K = q.shape
    V = v.shape[-1]
    for name, t in (("k", k), ("g", g)):
        if tuple(t.shape) != (N, H, K):
            raise ValueError("%s must have the shape of q" % name)
    if tuple(v.shape) != (N, H, V) or tuple(out.shape) != (N, H, V):
        raise ValueError("v and out must be [N, H, V]")
    if tuple(beta.shape) != (N, H):
        raise ValueError("beta must be [N, H]")
    if A_log.numel() != H or dt_bias.numel() != H * K:
        raise ValueError("A_log must have H elements and dt_bias H*K")
    if tuple(state.shape) != (N, H, K, V):
        raise ValueError("state must be [N, H, K, V] = %s" % ((N, H, K, V),))
    if state.dtype == torch.float32:
        sd = KDA_STATE_FP32
    elif state.dtype == bf16:
        sd = KDA_STATE_BF16
    else:
        raise ValueError("state must be bfloat16 or float32")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib.kda_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(out),
                        _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(state), sd, N, H, K, V,
                        ctypes.c_void_p(stream))
    if rc == 0:
        return out
    msg = lib.kda_status_string(rc).decode()
    if rc == 8:
        raise KdaError(msg)
    raise ValueError(msg)


def bwd(q, k, v, g, beta, scale, dout, A_log, dt_bias, lower_bound, initial_state=None,
        dfinal_state=None, cu_seqlens=None, grads=None, workspace=None):
    """Gradients of sum(dout * out) + sum(dfinal_state * final_state) for the forward.

    Inputs as for ``fwd``; dout: bf16 [B, T, H, 128]; dfinal_state: None or fp32
    [N, H, 128, 128]. Returns a dict of fp32 tensors dq, dk, dv, dg [B, T, H, 128],
    dbeta [B, T, H], dA_log [H], ddt_bias [H, 128] and dinitial_state
    [N, H, 128, 128]. ``grads`` (optional) is a dict of preallocated outputs with
    those names. Raises ValueError for invalid arguments and KdaError for HIP
    failures.
    """
    import torch
    lib = load_library()
    bf16 = torch.bfloat16
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("dout", dout)):
        if t.dtype != bf16:
            raise ValueError("%s must be bfloat16 (got %s)" % (name, t.dtype))
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        if t.dtype != torch.float32:
            raise ValueError("%s must be float32 (got %s)" % (name, t.dtype))
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, K]")
    B, T, H, K = q.shape
    V = v.shape[-1]
    for name, t in (("k", k), ("g", g)):
        if tuple(t.shape) != (B, T, H, K):
            raise ValueError("%s must have the shape of q" % name)
    if tuple(v.shape) != (B, T, H, V) or tuple(dout.shape) != (B, T, H, V):
        raise ValueError("v and dout must be [B, T, H, V]")
    if tuple(beta.shape) != (B, T, H):
        raise ValueError("beta must be [B, T, H]")
    if A_log.numel() != H or dt_bias.numel() != H * K:
        raise ValueError("A_log must have H elements and dt_bias H*K")
    num_seqs = 0
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32:
            raise ValueError("cu_seqlens must be int32")
        num_seqs = cu_seqlens.numel() - 1
        if num_seqs <= 0:
            raise ValueError("cu_seqlens must have at least 2 entries")
    N = num_seqs if cu_seqlens is not None else B
    sd = KDA_STATE_NONE
    if initial_state is not None:
        if initial_state.dtype == torch.float32:
            sd = KDA_STATE_FP32
        elif initial_state.dtype == bf16:
            sd = KDA_STATE_BF16
        else:
            raise ValueError("initial_state must be bfloat16 or float32")
        if tuple(initial_state.shape) != (N, H, K, V):
            raise ValueError("initial_state must be [N, H, K, V] = %s" % ((N, H, K, V),))
    if dfinal_state is not None:
        if dfinal_state.dtype != torch.float32 or tuple(dfinal_state.shape) != (N, H, K, V):
            raise ValueError("dfinal_state must be float32 [N, H, K, V] = %s" % ((N, H, K, V),))
    dev = q.device
    f32 = torch.float32
    shapes = dict(dq=(B, T, H, K), dk=(B, T, H, K), dv=(B, T, H, V), dg=(B, T, H, K), dbeta=(B, T, H),
                  dA_log=(H,), ddt_bias=(H, K), dinitial_state=(N, H, K, V))
    if grads is None:
        grads = {n: torch.empty(shp, dtype=f32, device=dev) for n, shp in shapes.items()}
    else:
        for n, shp in shapes.items():
            t = grads.get(n)
            if t is None or t.dtype != f32 or tuple(t.shape) != shp:
                raise ValueError("grads[%r] must be float32 %s" % (n, shp))
    tensors = [q, k, v, g, beta, dout, A_log, dt_bias, initial_state, dfinal_state, cu_seqlens, workspace,
               *grads.values()]
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    need = lib.kda_bwd_workspace_size(B, T, H, num_seqs)
    ws = _workspace(need, dev, "bwd") if workspace is None else workspace
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.kda_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(dout),
                     _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state), sd,
                     _ptr(dfinal_state), _ptr(cu_seqlens), num_seqs, B, T, H, K, V,
                     _ptr(grads["dq"]), _ptr(grads["dk"]), _ptr(grads["dv"]), _ptr(grads["dg"]),
                     _ptr(grads["dbeta"]), _ptr(grads["dA_log"]), _ptr(grads["ddt_bias"]),
                     _ptr(grads["dinitial_state"]), _ptr(ws), ws.numel(), ctypes.c_void_p(stream))
    if rc == 0:
        return grads
    msg = lib.kda_status_string(rc).decode()
    if rc == 8:
        raise KdaError(msg)
    raise ValueError(msg)
