"""The C ABI library loads, exports what include/kda.h declares, and rejects
invalid arguments before touching the GPU (CPU only: every call below fails
validation, so nothing is enqueued)."""
import ctypes
import os
import re

import pytest

import kimi_delta_attention_fwd_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    return sorted(set(re.findall(r"KDA_API\s+[\w\s\*]*?\b(kda_\w+)\s*\(", src)))


def test_exports_match_header():
    lib = kda.load_library()
    names = _declared()
    assert set(names) == set(kda.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code, tag in enumerate(["KDA_OK", "KDA_ERR_NULL", "KDA_ERR_HEAD_DIM", "KDA_ERR_SHAPE",
                                "KDA_ERR_STATE_DTYPE", "KDA_ERR_ARG", "KDA_ERR_WORKSPACE",
                                "KDA_ERR_ALIAS", "KDA_ERR_HIP", "KDA_ERR_SCRATCH"]):
        assert kda.status_string(code).startswith(tag)
    assert "unknown" in kda.status_string(99)


def test_workspace_size():
    rec, sink = 72192, 0
    assert kda.workspace_size(1, 65536, 32) == sink + 1024 * 32 * rec
    assert kda.workspace_size(4, 2048, 16) == sink + 4 * 32 * 16 * rec
    assert kda.workspace_size(1, 100, 2) == sink + 2 * 2 * rec
    assert kda.workspace_size(1, 66399, 32, 16) == sink + 256 + (66399 // 64 + 16) * 32 * rec
    assert kda.workspace_size(2, 100, 2, 3) == 0      # cu_seqlens requires B = 1
    assert kda.workspace_size(0, 100, 2) == 0


class FakeBufs:
    """Distinct, non-overlapping fake device addresses (never dereferenced)."""

    def __init__(self, B=1, T=64, H=2):
        self.B, self.T, self.H = B, T, H
        act = B * T * H * 128 * 2
        base = 1 << 40
        step = 1 << 32
        self.addr = {name: base + i * step for i, name in enumerate(
            ["q", "k", "v", "g", "beta", "out", "A_log", "dt_bias", "init", "fin", "cu", "ws"])}
        self.act = act

    def call(self, lib, **over):
        a = dict(self.addr)
        kw = dict(scale=0.088, lb=-5.0, sd=0, cu=None, nseq=0, B=self.B, T=self.T, H=self.H,
                  K=128, V=128, wsb=kda.workspace_size(self.B, self.T, self.H), init=None, fin=None)
        kw.update(over)
        p = lambda name: ctypes.c_void_p(a[name]) if a.get(name) else None
        ptr = {}
        for name in ["q", "k", "v", "g", "beta", "out", "A_log", "dt_bias", "ws"]:
            v = over.get("p_" + name, "default")
            ptr[name] = p(name) if v == "default" else (None if v is None else ctypes.c_void_p(v))
        init = ctypes.c_void_p(kw["init"]) if kw["init"] else None
        fin = ctypes.c_void_p(kw["fin"]) if kw["fin"] else None
        cu = ctypes.c_void_p(kw["cu"]) if kw["cu"] else None
        return lib.kda_fwd(ptr["q"], ptr["k"], ptr["v"], ptr["g"], ptr["beta"], kw["scale"], ptr["out"],
                           ptr["A_log"], ptr["dt_bias"], kw["lb"], init, fin, kw["sd"], cu, kw["nseq"],
                           kw["B"], kw["T"], kw["H"], kw["K"], kw["V"], ptr["ws"], kw["wsb"], None)


@pytest.fixture
def fb():
    return FakeBufs()


def test_rejects_head_dims(fb):
    """kda_fwd takes K = V = 128 and K = V = 64; every other pair is rejected."""
    lib = kda.load_library()
    for K, V in ((64, 128), (128, 64), (128, 256), (256, 256), (32, 32), (96, 96), (0, 0)):
        assert fb.call(lib, K=K, V=V) == 2, (K, V)
    # K = V = 64 passes the head-dim check: the fake buffers then fail on the
    # too-small workspace argument (a later check), not on the head dims
    assert fb.call(lib, K=64, V=64, wsb=0) == 6


def test_rejects_shapes(fb):
    lib = kda.load_library()
    assert fb.call(lib, B=0) == 3
    assert fb.call(lib, T=0) == 3
    assert fb.call(lib, H=-1) == 3
    cu = fb.addr["cu"]
    assert fb.call(lib, B=2, cu=cu, nseq=2) == 3          # cu_seqlens needs B = 1
    assert fb.call(lib, cu=cu, nseq=0) == 3
    # size limits: heads, 32-bit grids, int32 token offsets with cu_seqlens
    assert fb.call(lib, H=kda.KDA_MAX_HEADS + 1) == 3
    assert fb.call(lib, T=1 << 31, H=64) == 3                # chunk slots x H past INT32_MAX
    assert fb.call(lib, B=1 << 20, T=64, H=512) == 3          # 8 N H past INT32_MAX
    assert fb.call(lib, T=1 << 31, cu=cu, nseq=2) == 3        # int32 offsets
    assert fb.call(lib, B=1 << 40, T=1 << 40) == 3            # no overflow in the checks
    assert kda.workspace_size(1, 1 << 31, 64) == 0
    assert kda.workspace_size(1, 100, kda.KDA_MAX_HEADS + 1) == 0


def test_rejects_null(fb):
    lib = kda.load_library()
    for name in ["q", "k", "v", "g", "beta", "out", "A_log", "dt_bias"]:
        assert fb.call(lib, **{"p_" + name: None}) == 1, name


def test_rejects_state_dtype(fb):
    lib = kda.load_library()
    assert fb.call(lib, sd=0, init=fb.addr["init"]) == 4   # state given with NONE
    assert fb.call(lib, sd=1) == 4                         # BF16 without states
    assert fb.call(lib, sd=7, init=fb.addr["init"]) == 4


def test_rejects_args(fb):
    lib = kda.load_library()
    assert fb.call(lib, lb=0.5) == 5
    assert fb.call(lib, lb=float("-inf")) == 5
    assert fb.call(lib, lb=float("nan")) == 5
    assert fb.call(lib, scale=float("inf")) == 5


def test_rejects_misaligned(fb):
    """Tensors moved in 16-byte pieces must be 16-byte aligned (KDA_ERR_ARG)."""
    lib = kda.load_library()
    for name in ["q", "k", "v", "g", "out", "dt_bias"]:
        assert fb.call(lib, **{"p_" + name: fb.addr[name] + 2}) == 5, name
    assert fb.call(lib, sd=2, init=fb.addr["init"] + 8) == 5
    assert fb.call(lib, sd=2, fin=fb.addr["fin"] + 4) == 5
    # element alignment is enough for beta and A_log
    assert fb.call(lib, p_beta=fb.addr["beta"] + 2, wsb=0) == 6
    assert fb.call(lib, p_A_log=fb.addr["A_log"] + 4, wsb=0) == 6


def test_rejects_workspace(fb):
    lib = kda.load_library()
    assert fb.call(lib, p_ws=None) == 6
    assert fb.call(lib, wsb=100) == 6
    assert fb.call(lib, p_ws=fb.addr["ws"] + 8) == 6       # not 256-byte aligned


def test_rejects_aliasing(fb):
    lib = kda.load_library()
    assert fb.call(lib, p_out=fb.addr["v"] + 64) == 7      # out overlaps v
    assert fb.call(lib, p_ws=fb.addr["q"]) == 7            # workspace overlaps q
    st = fb.addr["init"]
    assert fb.call(lib, sd=2, init=st, fin=st + 1024) == 7  # partial state overlap
    assert fb.call(lib, sd=2, init=st, fin=fb.addr["k"]) == 7


def _decode_call(lib, over=None):
    """kda_decode on fake, non-overlapping addresses (never dereferenced)."""
    base, step = 1 << 40, 1 << 32
    names = ["q", "k", "v", "g", "beta", "out", "A_log", "dt_bias", "state"]
    a = {n: base + i * step for i, n in enumerate(names)}
    kw = dict(scale=0.088, lb=-5.0, sd=2, N=4, H=2, K=128, V=128)
    over = dict(over or {})
    for n in names:
        if "p_" + n in over:
            a[n] = over.pop("p_" + n)
    kw.update(over)
    p = lambda n: None if a[n] is None else ctypes.c_void_p(a[n])
    return lib.kda_decode(p("q"), p("k"), p("v"), p("g"), p("beta"), kw["scale"], p("out"), p("A_log"),
                          p("dt_bias"), kw["lb"], p("state"), kw["sd"], kw["N"], kw["H"], kw["K"], kw["V"], None)


def test_decode_rejects_bad_arguments():
    """kda_decode validates on the host and enqueues nothing on error."""
    lib = kda.load_library()
    assert _decode_call(lib, {"K": 64}) == 2
    assert _decode_call(lib, {"N": 0}) == 3
    assert _decode_call(lib, {"H": -2}) == 3
    assert _decode_call(lib, {"H": kda.KDA_MAX_HEADS + 1}) == 3
    assert _decode_call(lib, {"N": 1 << 31}) == 3
    for n in ["q", "k", "v", "g", "beta", "out", "A_log", "dt_bias", "state"]:
        assert _decode_call(lib, {"p_" + n: None}) == 1, n
    assert _decode_call(lib, {"sd": 0}) == 4                 # a state is required
    assert _decode_call(lib, {"sd": 9}) == 4
    assert _decode_call(lib, {"lb": 0.25}) == 5
    assert _decode_call(lib, {"lb": float("-inf")}) == 5
    assert _decode_call(lib, {"scale": float("nan")}) == 5
    base0, step0 = 1 << 40, 1 << 32
    assert _decode_call(lib, {"p_q": base0 + 2}) == 5                      # q not 16-byte aligned
    assert _decode_call(lib, {"p_state": base0 + 8 * step0 + 4}) == 5      # state not 16-byte aligned
    base, step = 1 << 40, 1 << 32
    assert _decode_call(lib, {"p_out": base + 2 * step + 16}) == 7         # out overlaps v
    assert _decode_call(lib, {"p_state": base + 0 * step + 256}) == 7      # state overlaps q
    assert _decode_call(lib, {"p_out": base + 8 * step + 512}) == 7        # out inside the state


def test_load_library_brings_torch_first():
    """torch ships its own HIP runtime: load_library() imports torch before binding
    libkda, so a program that loads the library before importing torch still runs
    libkda on torch's runtime (a second runtime would make every launch fail)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); import kimi_delta_attention_fwd_amd as kda; "
            "assert 'torch' not in sys.modules; kda.load_library(); assert 'torch' in sys.modules" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]


def test_noalloc_rejects_before_any_hip_call():
    """kda_fwd_noalloc validates like kda_fwd and rejects sizes whose workspace
    exceeds its built-in scratch (KDA_ERR_SCRATCH) before it touches HIP."""
    lib = kda.load_library()
    assert kda.KDA_NOALLOC_SCRATCH_BYTES == 256 << 20
    fbuf = FakeBufs()
    a = {n: ctypes.c_void_p(v) for n, v in fbuf.addr.items()}

    def call(B, T, H, K=128, lb=-5.0, q=a["q"]):
        return lib.kda_fwd_noalloc(q, a["k"], a["v"], a["g"], a["beta"], 0.088, a["out"], a["A_log"],
                                   a["dt_bias"], lb, None, None, 0, None, 0, B, T, H, K, 128, None)
    # 1024 chunks x 32 heads x 72 KB records: far beyond 256 MiB
    assert kda.workspace_size(1, 65536, 32) > kda.KDA_NOALLOC_SCRATCH_BYTES
    assert call(1, 65536, 32) == 9
    # 11 heads (more than 10 chains: no segment-parallel area): 338 chunks per head
    # are 3,718 records of 72,192 bytes and fit, 339 do not
    assert kda.workspace_size(1, 338 * 64, 11) <= kda.KDA_NOALLOC_SCRATCH_BYTES
    assert kda.workspace_size(1, 339 * 64, 11) > kda.KDA_NOALLOC_SCRATCH_BYTES
    assert call(1, 339 * 64, 11) == 9
    # kda_fwd's own checks come first
    assert call(1, 64, 2, K=64) == 2
    assert call(1, 64, 2, lb=1.0) == 5
    assert call(1, 64, 2, q=None) == 1
    assert call(0, 64, 2) == 3
