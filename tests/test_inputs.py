"""Seeded input generator: determinism, bf16 rounding, workload sizes (CPU)."""
import numpy as np
import torch

import kda_inputs as ki


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000)).astype(np.float32)
    ours = ki.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    back = ki.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_deterministic():
    a = ki.config_inputs(0)
    b = ki.config_inputs(0)
    for key in ("q", "k", "v", "g", "beta", "A_log", "dt_bias"):
        assert np.array_equal(a[key], b[key])
    c = ki.make_inputs(1, 256, 1, seed=1)
    assert not np.array_equal(a["q"], c["q"])


def test_workload_sizes():
    s2 = ki.config_shape(2)
    assert s2["N"] == 16 and s2["T"] == 66399
    assert np.all(s2["lengths"] % 64 != 0) and s2["lengths"].min() >= 37 and s2["lengths"].max() <= 8191
    s4 = ki.config_shape(4)
    assert s4["N"] == 512 and s4["T"] == 34408
    assert s4["lengths"].min() >= 1 and s4["lengths"].max() <= 128
    assert ki.config_shape(3)["T"] == 65536 and ki.config_shape(3)["H"] == 32


def test_distributions_tiny():
    d = ki.config_inputs(0)
    q = ki.bf16_bits_to_f64(d["q"])
    n = np.linalg.norm(q, axis=-1)
    assert np.all(np.abs(n - 1.0) < 1e-2)          # unit rows up to bf16 rounding
    b = ki.bf16_bits_to_f64(d["beta"])
    assert np.all((b > 0) & (b < 1))
    assert np.all((d["A_log"] >= 0) & (d["A_log"] <= np.log(16.0) + 1e-6))
    assert d["initial_state"] is None and d["cu_seqlens"] is None
    d1 = ki.config_inputs(1)
    assert d1["initial_state"].dtype == np.float32 and d1["initial_state"].shape == (4, 16, 128, 128)
    assert abs(d1["initial_state"].std() - 0.02) < 1e-3
    assert abs(d1["dt_bias"].std() - 0.1) < 1e-2
