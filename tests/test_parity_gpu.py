"""GPU path vs the fp64 oracle, element by element, through the C ABI.

Every (b, h) sequence of every case is compared, the full-size workloads
included.  Outputs are pre-filled with NaN, so an element the kernel never
writes fails the check.  The gate is the normwise max relative error per
tensor; an elementwise relative error is printed beside it as a diagnostic.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_13_amd.workloads import WORKLOADS, make_inputs, make_random
from oracle import chunked_ref as cr
from tests.gpu_helpers import TOL, elem_err, gpu_heads, rel_err, run_gpu, run_oracle, say

import gated_delta_rule_13_amd as gdn

pytestmark = pytest.mark.gpu


def check(x, O, S, heads=None, tol=None, label=""):
    w = x["workload"]
    tol = tol or TOL[w.dtype]
    Or, Sr = run_oracle(x, heads)
    if heads is None:
        Og, Sg = O.float().cpu().numpy(), S.cpu().numpy()
    else:
        Og, Sg = gpu_heads(O, heads), gpu_heads(S, heads)
    eo, es = rel_err(Og, Or), rel_err(Sg, Sr)
    say(f"{label or w.name}: O rel err {eo:.3e}  S rel err {es:.3e}  (tol {tol:.0e}); "
        f"elementwise O {elem_err(Og, Or):.3e}  S {elem_err(Sg, Sr):.3e}")
    assert np.isfinite(Og).all() and np.isfinite(Sg).all()
    assert eo < tol, f"O rel err {eo}"
    assert es < tol, f"S rel err {es}"
    return eo, es


# ---------------------------------------------------------------- workloads

def test_workload_tiny_fp32():
    x = make_inputs(WORKLOADS["tiny"])
    say("case: tiny B1 H1 T64 d16 C16 f32")
    O, S = run_gpu(x, 16)
    check(x, O, S)


def test_workload_deltanet_bf16():
    x = make_inputs(WORKLOADS["deltanet"])
    say("case: deltanet B2 H4 T1024 d64 C64 bf16, alpha=1, S0 random")
    O, S = run_gpu(x, 64)
    check(x, O, S)


def test_workload_main_full_size():
    x = make_inputs(WORKLOADS["main"])
    say("case: main B4 H16 T4096 d128 C64 bf16 (all 64 heads)")
    O, S = run_gpu(x, 64)
    check(x, O, S)


def test_workload_long_full_size():
    x = make_inputs(WORKLOADS["long"])
    say("case: long B1 H32 T32768 dk128 dv256 C64 bf16 (all 32 heads)")
    O, S = run_gpu(x, 64)
    check(x, O, S)


def test_workload_many_short_full_size():
    x = make_inputs(WORKLOADS["many_short"])
    say(f"case: many_short B64 H8 T512 d128 C32 bf16 (all 512 heads, "
        f"{int(x['reflection_mask'].sum())} reflection tokens)")
    O, S = run_gpu(x, 32)
    check(x, O, S)


def test_workload_olmo_hybrid_full_size():
    """"从电路复杂性理论的角度分析大模型的可并行性和表达能力--Olmo Hybrid 系列",
    Olmo Hybrid architecture: 30 heads, q/k dimension 96, v dimension 192,
    erase strength 2 beta.  B * H = 60 is not a multiple of 8 (no XCD
    grouping of a head's workgroups)."""
    x = make_inputs(WORKLOADS["olmo_hybrid"])
    say("case: olmo_hybrid B2 H30 T4096 dk96 dv192 C64 bf16, beta in (0, 2) (all 60 heads)")
    O, S = run_gpu(x, 64)
    check(x, O, S)


# ---------------------------------------------------- shapes, tiles, tails

BF16_SHAPES = [
    # (B, H, T, dk, dv, C)
    (1, 1, 1, 128, 128, 64),
    (1, 2, 63, 128, 64, 64),
    (1, 1, 64, 64, 64, 64),
    (2, 1, 65, 128, 128, 64),
    (1, 3, 200, 32, 48, 32),
    (1, 2, 333, 64, 256, 32),
    (2, 2, 257, 128, 16, 64),
    (1, 1, 130, 128, 512, 64),
]


@pytest.mark.parametrize("B,H,T,dk,dv,C", BF16_SHAPES)
def test_bf16_shapes(B, H, T, dk, dv, C):
    x = make_random(B, H, T, dk, dv, dtype="bf16", chunk=C, seed=T + dk, s0_std=0.02)
    say(f"case: bf16 B{B} H{H} T{T} dk{dk} dv{dv} C{C}")
    O, S = run_gpu(x, C)
    check(x, O, S, label=f"bf16 {B}x{H}x{T} dk{dk} dv{dv} C{C}")


F32_SHAPES = [
    (1, 1, 16, 16, 16, 16),
    (1, 2, 37, 16, 32, 16),
    (2, 1, 100, 32, 32, 32),
    (1, 1, 129, 64, 64, 64),
    (1, 2, 77, 64, 48, 16),
]


# Head counts large enough that the kernel runs two, three or four scan
# waves per workgroup (the launch weighs a round of four-wave workgroups as
# 1.4 rounds and of three-wave ones as 1.2, three needing d_v / 16 divisible
# by 3); with up to three the values are staged through LDS by a prep wave,
# with four the scan waves load them.  Ragged T in every case; every head is
# compared.
WAVE_SHAPES = [
    # (B, H, T, dk, dv, C)
    (4, 16, 333, 128, 128, 64),   # two scan waves
    (4, 16, 97, 64, 128, 32),     # two scan waves, d_k 64, 32-token chunks
    (8, 32, 150, 64, 64, 64),     # four scan waves
    (16, 16, 97, 128, 128, 32),   # four scan waves, 32-token chunks
    (8, 32, 100, 64, 256, 64),    # four scan waves, d_v 256 (non-temporal fp32 stores)
    (2, 30, 300, 96, 192, 64),    # three scan waves (five prep waves), the Olmo head shape
    (6, 16, 150, 128, 96, 32),    # three scan waves, 32-token chunks
    (8, 16, 77, 64, 48, 16),      # three scan waves, 16-token chunks
    (16, 16, 77, 64, 64, 16),     # four scan waves beside six prep waves, 16-token chunks
    (8, 32, 70, 256, 64, 32),     # four scan waves beside four prep waves at d_k 256
]


@pytest.mark.parametrize("B,H,T,dk,dv,C", WAVE_SHAPES)
def test_scan_wave_counts_ragged(B, H, T, dk, dv, C):
    x = make_random(B, H, T, dk, dv, dtype="bf16", chunk=C, seed=T + B, s0_std=0.02)
    say(f"case: bf16 B{B} H{H} T{T} dk{dk} dv{dv} C{C} (all heads)")
    O, S = run_gpu(x, C)
    check(x, O, S, label=f"B{B} H{H} T{T} dk{dk} dv{dv} C{C}")


@pytest.mark.parametrize("B,H,T,dk,dv,C", F32_SHAPES)
def test_f32_shapes(B, H, T, dk, dv, C):
    x = make_random(B, H, T, dk, dv, dtype="f32", chunk=C, seed=3 * T + dv, s0_std=0.05,
                    alpha_scale=0.1)
    say(f"case: f32 B{B} H{H} T{T} dk{dk} dv{dv} C{C}")
    O, S = run_gpu(x, C)
    check(x, O, S, label=f"f32 {B}x{H}x{T} dk{dk} dv{dv} C{C}")


# ---------------------------------------------------------- API semantics

def test_null_alpha_and_null_state_match_explicit():
    x = make_random(1, 2, 150, 64, 64, dtype="bf16", chunk=64, seed=5)
    say("case: alpha None vs ones, S0 None vs zeros")
    x["alpha"] = None
    O1, S1 = run_gpu(x, 64)
    d = {**x, "alpha": torch.ones(1, 2, 150), "S0": torch.zeros(1, 2, 64, 64)}
    O2, S2 = run_gpu(d, 64)
    assert torch.equal(O1, O2) and torch.equal(S1, S2)
    check(x, O1, S1)


def test_in_place_state_and_chaining():
    """S_final may alias S0; splitting the sequence and feeding S_final back
    as S0 reproduces the one-call result (chunks chain)."""
    x = make_random(2, 2, 300, 128, 128, dtype="bf16", chunk=64, seed=9, s0_std=0.02)
    say("case: chaining 300 = 100 + 200 with in-place state")
    O_full, S_full = run_gpu(x, 64)
    cut = 100
    part = lambda t, a, b: None if t is None else t[:, :, a:b].contiguous()
    x1 = {**x, **{k: part(x[k], 0, cut) for k in ("q", "k", "v", "alpha", "beta")}}
    x2 = {**x, **{k: part(x[k], cut, 300) for k in ("q", "k", "v", "alpha", "beta")}}
    state = x["S0"].cuda().clone()
    O1, _ = run_gpu(x1, 64, S0=state, S_final=state)
    O2, _ = run_gpu(x2, 64, S0=state, S_final=state)
    O_cat = torch.cat([O1, O2], dim=2)
    # the split moves chunk boundaries (different rounding): both results lie
    # within the tolerance of the exact one
    Or, Sr = run_oracle(x)
    assert rel_err(O_cat.cpu().numpy(), Or) < TOL["bf16"]
    assert rel_err(state.cpu().numpy(), Sr) < TOL["bf16"]
    check(x, O_full, S_full)


def test_bf16_output_dtype():
    x = make_random(1, 2, 200, 128, 128, dtype="bf16", chunk=64, seed=11)
    say("case: bf16 O")
    O, S = run_gpu(x, 64, o_dtype=torch.bfloat16)
    assert O.dtype == torch.bfloat16
    # rounding O to bf16 adds at most 2^-9 relative per element
    check(x, O, S, tol=2e-3 + 2 ** -9)


def test_deterministic():
    x = make_random(1, 4, 500, 128, 128, dtype="bf16", chunk=64, seed=13)
    say("case: determinism")
    O1, S1 = run_gpu(x, 64)
    O2, S2 = run_gpu(x, 64)
    assert torch.equal(O1, O2) and torch.equal(S1, S2)


def test_nan_stays_in_its_sequence():
    x = make_random(1, 3, 100, 64, 64, dtype="bf16", chunk=32, seed=17)
    x["beta"] = x["beta"].clone()
    x["beta"][0, 1, 50] = float("nan")
    say("case: NaN beta in head 1")
    O, S = run_gpu(x, 32)
    O, S = O.cpu(), S.cpu()
    assert torch.isfinite(O[0, 0]).all() and torch.isfinite(O[0, 2]).all()
    assert torch.isfinite(S[0, 0]).all() and torch.isfinite(S[0, 2]).all()
    assert torch.isnan(O[0, 1, 50:]).any() and torch.isfinite(O[0, 1, :32]).all()


def test_reflection_tokens_beta_two():
    """Every token a Householder reflection (beta = 2 / k^T k, alpha = 1)."""
    x = make_random(1, 2, 256, 128, 128, dtype="bf16", chunk=64, seed=19, s0_std=0.5)
    kk = (x["k"].float() ** 2).sum(-1)
    x["beta"] = (2.0 / kk).float()
    x["alpha"] = None
    say("case: all reflections")
    O, S = run_gpu(x, 64)
    check(x, O, S)


# ------------------------------------------------------ stage parity (T, W, U)

@pytest.mark.parametrize("dtype,B,H,T,dk,dv,C", [
    ("bf16", 1, 2, 150, 128, 64, 64),
    ("bf16", 1, 1, 70, 64, 32, 32),
    ("f32", 1, 2, 45, 32, 32, 16),
    ("f32", 1, 1, 64, 64, 16, 64),
])
def test_chunk_prep_matches_chunked_reference(dtype, B, H, T, dk, dv, C):
    x = make_random(B, H, T, dk, dv, dtype=dtype, chunk=C, seed=T)
    say(f"case: prep {dtype} T{T} dk{dk} dv{dv} C{C}")
    d = {k_: (None if x[k_] is None else x[k_].cuda()) for k_ in ("k", "v", "alpha", "beta")}
    out = gdn.gdn_chunk_prep(d["k"], d["v"], d["alpha"], d["beta"], chunk_size=C)
    torch.cuda.synchronize()
    tol = 1e-4 if dtype == "bf16" else 1e-5
    k64 = x["k"].double().numpy()
    v64 = x["v"].double().numpy()
    a64 = x["alpha"].double().numpy()
    b64 = x["beta"].double().numpy()
    for b in range(B):
        for h in range(H):
            for c, t0 in enumerate(range(0, T, C)):
                t1 = min(T, t0 + C)
                m = cr.gated_chunk_matrices(k64[b, h, t0:t1], v64[b, h, t0:t1],
                                            a64[b, h, t0:t1], b64[b, h, t0:t1])
                L = t1 - t0
                Tg = out["T"][b, h, c].cpu().double().numpy()
                assert rel_err(Tg[:L, :L], m["T"]) < tol
                assert np.all(Tg[L:, :L] == 0) or L == C
                assert rel_err(out["W"][b, h, t0:t1].cpu().numpy(), m["W"]) < tol
                assert rel_err(out["U"][b, h, t0:t1].cpu().numpy(), m["U"]) < tol
