"""Seeded input generators: determinism, distributions, shapes (CPU only)."""
import torch

from gated_delta_rule_13_amd.workloads import (WORKLOADS, algorithmic_bytes,
                                               algorithmic_flops, make_inputs, make_random)


def test_deterministic():
    w = WORKLOADS["deltanet"].with_shape(B=1, H=2, T=100)
    a, b = make_inputs(w, seed=0), make_inputs(w, seed=0)
    for key in ("q", "k", "v", "beta", "S0"):
        assert torch.equal(a[key], b[key])
    c = make_inputs(w, seed=1)
    assert not torch.equal(a["q"], c["q"])


def test_shapes_dtypes_and_ranges():
    for name, w in WORKLOADS.items():
        small = w.with_shape(B=min(w.B, 2), H=min(w.H, 2), T=min(w.T, 256))
        x = make_inputs(small)
        B, H, T = small.B, small.H, small.T
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        assert x["q"].shape == (B, H, T, w.dk) and x["q"].dtype == dt
        assert x["v"].shape == (B, H, T, w.dv) and x["v"].dtype == dt
        assert x["beta"].dtype == torch.float32 and x["beta"].shape == (B, H, T)
        kn = x["k"].float().norm(dim=-1)
        assert torch.allclose(kn, torch.ones_like(kn), atol=1e-2)
        if x["alpha"] is not None:
            assert bool((x["alpha"] > 0).all()) and bool((x["alpha"] <= 1).all())
        assert (x["S0"] is None) == (w.s0_std == 0)


def test_reflection_tokens():
    w = WORKLOADS["many_short"].with_shape(B=8, H=8, T=512)
    x = make_inputs(w)
    m = x["reflection_mask"]
    rate = m.float().mean().item()
    assert 0.005 < rate < 0.015
    kk = (x["k"].float() ** 2).sum(-1)
    assert torch.allclose(x["beta"][m] * kk[m], torch.full_like(kk[m], 2.0), rtol=1e-6)
    assert bool((x["alpha"][m] == 1).all())
    assert bool((x["beta"][~m] < 1).all())


def test_algorithmic_counts_main_workload():
    w = WORKLOADS["main"]
    assert algorithmic_bytes(w) == 341_835_776
    assert abs(algorithmic_flops(w) / 1e9 - 47.60) < 0.01


def test_make_random_custom_shape():
    x = make_random(1, 3, 70, 32, 48, dtype="f32", chunk=16, s0_std=0.02)
    assert x["q"].shape == (1, 3, 70, 32) and x["S0"].shape == (1, 3, 48, 32)
