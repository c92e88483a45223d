"""Seeded synthetic inputs for the Kimi Delta Attention chunked forward.

This module only draws random numbers and converts dtypes; it holds none of the
method's arithmetic. It is shared by the fp64 oracle (tests, bench CPU leg) and
by the GPU path (tests, bench, smoke) so that both consume identical bf16 bits.

Workload recipe (the five benchmark workloads of the KDA forward; the pages
about FlashKDA give only the argument list of ``flash_kda.fwd`` and its
constraints -- K = V = 128, bf16 activations, ``cu_seqlens`` with B = 1, bf16 or
fp32 states of matching dtype -- so the value distributions are this project's
stated recipe):

* q, k ~ N(0, 1) per element, divided by their L2 norm per (token, head), then
  cast to bf16 (round to nearest even).
* v, g ~ N(0, 1), bf16.
* beta = sigmoid(N(0, 1)), bf16, shape [B, T, H].
* A_log[h] = log(U[1, 16]) (natural log), fp32 [H].
* dt_bias = 0 (fp32 [H, 128]) except the dense-batch workload, N(0, 0.1).
* states ~ N(0, sigma) in fp32, or cast to bf16.
* scale = 128 ** -0.5.

Draw order from a fresh ``numpy.random.default_rng(seed)``: sequence lengths
(varlen workloads), q, k, v, g, beta pre-activation, A_log, dt_bias (when
random), initial_state.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128

# name, B, T, H, lower_bound, state dtype (None/'fp32'/'bf16'), initial state
# present, state sigma, varlen spec, dt_bias sigma
CONFIGS = {
    0: dict(name="tiny", B=1, T=256, H=1, lower_bound=-5.0, state=None,
            initial=False, sigma=0.0, varlen=None, dt_sigma=0.0),
    1: dict(name="dense_batch", B=4, T=2048, H=16, lower_bound=-5.0,
            state="fp32", initial=True, sigma=0.02, varlen=None, dt_sigma=0.1),
    2: dict(name="varlen_packed", B=1, T=None, H=32, lower_bound=-5.0,
            state="bf16", initial=True, sigma=0.02,
            varlen=dict(n=16, lo=37, hi=8192, avoid_multiple_of=64),
            dt_sigma=0.0),
    3: dict(name="long_prefill", B=1, T=65536, H=32, lower_bound=-3.0,
            state="fp32", initial=False, sigma=0.0, varlen=None, dt_sigma=0.0),
    4: dict(name="chunked_prefill_continuation", B=1, T=None, H=64,
            lower_bound=-5.0, state="fp32", initial=True, sigma=0.05,
            varlen=dict(n=512, lo=1, hi=129, avoid_multiple_of=None),
            dt_sigma=0.0),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the bf16 bit patterns as uint16. Inputs are finite by construction.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs only: u + 0x8000 cannot wrap below 0xFF800000 (the NaN range)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def draw_lengths(rng: np.random.Generator, n: int, lo: int, hi: int,
                 avoid_multiple_of: int | None) -> np.ndarray:
    """Sequence lengths iid uniform integers in [lo, hi); lengths that are a
    multiple of ``avoid_multiple_of`` are redrawn, in index order."""
    lens = rng.integers(lo, hi, n)
    if avoid_multiple_of:
        for i in range(n):
            while lens[i] % avoid_multiple_of == 0:
                lens[i] = rng.integers(lo, hi)
    return lens.astype(np.int64)


def _unit_rows_bf16(rng, shape):
    x = rng.standard_normal(shape, dtype=np.float32)
    nrm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    x /= nrm
    return f32_to_bf16_bits(x)


def make_inputs(B: int, T: int, H: int, seed: int = 0, *, lengths=None,
                lower_bound: float = -5.0, state: str | None = None,
                initial: bool = False, sigma: float = 0.02,
                dt_sigma: float = 0.0, rng: np.random.Generator | None = None,
                head_dim: int = HEAD_DIM):
    """Draw one batch of inputs.

    ``lengths`` (optional) packs sequences of these lengths into B = 1 with
    ``cu_seqlens``; then T must equal their sum. ``head_dim`` sets K = V (128
    for every benchmark workload). Returns a dict of numpy arrays (bf16 tensors
    as uint16 bit patterns) plus scalar arguments.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    K = V = int(head_dim)
    cu = None
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        assert B == 1 and T == int(lengths.sum())
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        N = len(lengths)
    else:
        N = B
    q = _unit_rows_bf16(rng, (B, T, H, K))
    k = _unit_rows_bf16(rng, (B, T, H, K))
    v = f32_to_bf16_bits(rng.standard_normal((B, T, H, V), dtype=np.float32))
    g = f32_to_bf16_bits(rng.standard_normal((B, T, H, K), dtype=np.float32))
    bpre = rng.standard_normal((B, T, H), dtype=np.float32)
    beta = f32_to_bf16_bits((1.0 / (1.0 + np.exp(-bpre))).astype(np.float32))
    A_log = np.log(rng.uniform(1.0, 16.0, H)).astype(np.float32)
    if dt_sigma > 0:
        dt_bias = (rng.standard_normal((H, K), dtype=np.float32) * np.float32(dt_sigma)).astype(np.float32)
    else:
        dt_bias = np.zeros((H, K), dtype=np.float32)
    init = None
    if state is not None and initial:
        s = (rng.standard_normal((N, H, K, V), dtype=np.float32) * np.float32(sigma)).astype(np.float32)
        init = s if state == "fp32" else f32_to_bf16_bits(s)
    return dict(q=q, k=k, v=v, g=g, beta=beta, A_log=A_log, dt_bias=dt_bias,
                scale=float(K) ** -0.5, lower_bound=float(lower_bound),
                initial_state=init, state_dtype=state, final=state is not None,
                cu_seqlens=cu, B=B, T=T, H=H, N=N, K=K, V=V)


def config_inputs(i: int, seed: int = 0, head_dim: int = HEAD_DIM) -> dict:
    """Inputs of benchmark workload ``i`` (0..4), drawn from default_rng(seed)
    (at head dims K = V = ``head_dim``)."""
    c = CONFIGS[i]
    rng = np.random.default_rng(seed)
    lengths = None
    T = c["T"]
    if c["varlen"] is not None:
        vl = c["varlen"]
        lengths = draw_lengths(rng, vl["n"], vl["lo"], vl["hi"], vl["avoid_multiple_of"])
        T = int(lengths.sum())
    d = make_inputs(c["B"], T, c["H"], lengths=lengths,
                    lower_bound=c["lower_bound"], state=c["state"],
                    initial=c["initial"], sigma=c["sigma"],
                    dt_sigma=c["dt_sigma"], rng=rng, head_dim=head_dim)
    d["config"] = i
    d["name"] = c["name"]
    return d


def token_heads(d: dict) -> int:
    """Total tokens x heads of one batch (the throughput unit)."""
    return int(d["B"]) * int(d["T"]) * int(d["H"])


def config_shape(i: int, seed: int = 0) -> dict:
    """Sizes of workload ``i`` without drawing the tensors (lengths only)."""
    c = CONFIGS[i]
    if c["varlen"] is None:
        return dict(B=c["B"], T=c["T"], H=c["H"], N=c["B"], lengths=None)
    rng = np.random.default_rng(seed)
    vl = c["varlen"]
    lengths = draw_lengths(rng, vl["n"], vl["lo"], vl["hi"], vl["avoid_multiple_of"])
    return dict(B=1, T=int(lengths.sum()), H=c["H"], N=len(lengths), lengths=lengths)
