"""The default bf16 path (fp16-operand fused kernel) beyond the workloads:
its own intermediates against the pages' chunk matrices, the wider shape
matrix (16-token chunks, d_k 16 / 32 / 96 / 256, the Olmo-Hybrid head shape), and
the split-bf16 alternative, gdn_chunk_fwd_precise, where the fast path's
error grows (ungated reflections over long sequences).

Every case compares all (b, h) sequences against the fp64 oracle, with
NaN-prefilled outputs.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import chunked_ref as cr
import gated_delta_rule_13_amd as gdn
from gated_delta_rule_13_amd.workloads import make_random
from tests.gpu_helpers import TOL, elem_err, nan_outputs, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


def oracle_all(x, eta=None):
    return oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"], eta=eta)


def check_all(x, O, S, tol, label, eta=None):
    Or, Sr = oracle_all(x, eta)
    Og, Sg = O.float().cpu().numpy(), S.cpu().numpy()
    assert np.isfinite(Og).all() and np.isfinite(Sg).all(), "unwritten or non-finite output"
    eo, es = rel_err(Og, Or), rel_err(Sg, Sr)
    say(f"{label}: O rel err {eo:.3e}  S rel err {es:.3e}  (tol {tol:.0e}); "
        f"elementwise O {elem_err(Og, Or):.3e}  S {elem_err(Sg, Sr):.3e}")
    assert eo < tol and es < tol
    return eo, es


# ----------------------------------------------------- stage parity (T, V')

# T and V' of the fast kernel against "从零开始的 GDN 推导"'s chunk matrices
# (UT transform: T = (I + L)^{-1}; S update: V' = U - W S^T), evaluated in
# fp64 from the same rounded inputs, with the chunk input state S taken from
# the fp64 recurrence over the tokens before the chunk.  The kernel holds T in
# fp16 (relative rounding 2^-11 per entry, plus the roundings of the block
# products that form the entries below the diagonal blocks) and forms V'
# from fp16 copies of S, of Y and of T: the stage tolerance is 4e-3
# normwise per chunk, eight fp16 unit roundings.
STAGE_TOL = 4e-3


@pytest.mark.parametrize("B,H,T,dk,dv,C", [
    (1, 2, 150, 128, 64, 64),
    (1, 2, 333, 128, 128, 64),   # ragged tail
    (1, 1, 70, 64, 32, 32),
    (1, 2, 45, 64, 48, 16),
    (4, 16, 130, 128, 128, 64),  # two scan waves per workgroup
    (2, 30, 130, 96, 192, 64),   # three scan waves, five prep waves
    (16, 16, 64, 128, 128, 32),  # four scan waves, six prep waves
    (8, 32, 100, 64, 64, 64),    # four scan waves, four prep waves
    (1, 2, 100, 16, 32, 32),     # d_k 16, zero-padded
])
def test_stages_match_chunk_matrices(B, H, T, dk, dv, C):
    x = make_random(B, H, T, dk, dv, dtype="bf16", chunk=C, seed=T + C, s0_std=0.02,
                    alpha_scale=0.1)
    say(f"case: stages B{B} H{H} T{T} dk{dk} dv{dv} C{C}")
    d = to_dev(x)
    O, S, Tg, Vg = gdn.gdn_chunk_fwd_stages(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                            chunk_size=C)
    torch.cuda.synchronize()
    Tg, Vg = Tg.cpu().double().numpy(), Vg.cpu().double().numpy()
    q64, k64, v64 = (x[n].double().numpy() for n in ("q", "k", "v"))
    a64, b64 = x["alpha"].double().numpy(), x["beta"].double().numpy()
    worst_t = worst_v = 0.0
    for b in range(B):
        for h in range(min(H, 3)):
            for c, t0 in enumerate(range(0, T, C)):
                t1 = min(T, t0 + C)
                L = t1 - t0
                m = cr.gated_chunk_matrices(k64[b, h, t0:t1], v64[b, h, t0:t1],
                                            a64[b, h, t0:t1], b64[b, h, t0:t1])
                et = rel_err(Tg[b, h, c, :L, :L], m["T"])
                # past a ragged end the kernel's T is the identity
                if L < C:
                    assert np.allclose(Tg[b, h, c, L:, L:], np.eye(C - L))
                    assert np.all(Tg[b, h, c, L:, :L] == 0)
                assert np.all(np.triu(Tg[b, h, c], 1) == 0)
                # chunk input state from the recurrence over tokens [0, t0)
                if t0 == 0:
                    S_in = x["S0"][b, h].double().numpy()
                else:
                    pick = lambda t: None if t is None else t[b:b + 1, h:h + 1, :t0]
                    _, Sr = oracle.recurrent(pick(x["q"]), pick(x["k"]), pick(x["v"]),
                                             pick(x["alpha"]), pick(x["beta"]),
                                             S0=x["S0"][b:b + 1, h:h + 1])
                    S_in = Sr[0, 0]
                Vp_ref = m["U"] - m["W"] @ S_in.T
                ev = rel_err(Vg[b, h, t0:t1], Vp_ref)
                worst_t, worst_v = max(worst_t, et), max(worst_v, ev)
                assert et < STAGE_TOL, f"T of chunk {c} (b {b}, h {h}): {et}"
                assert ev < STAGE_TOL, f"V' of chunk {c} (b {b}, h {h}): {ev}"
    say(f"  worst chunk: T {worst_t:.3e}  V' {worst_v:.3e}")
    check_all(x, O, S, TOL["bf16"], f"stages run B{B} H{H} T{T}")


def test_stages_entry_matches_plain_entry():
    """The stage entry runs the same kernel: identical O and S_final."""
    x = make_random(2, 4, 200, 128, 128, dtype="bf16", chunk=64, seed=41, s0_std=0.02)
    d = to_dev(x)
    O1, S1 = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], chunk_size=64)
    O2, S2, _, _ = gdn.gdn_chunk_fwd_stages(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                            chunk_size=64)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(S1, S2)


# -------------------------------------------------------- wider shapes

NEW_SHAPES = [
    # (B, H, T, dk, dv, C)
    (1, 2, 100, 64, 64, 16),
    (2, 2, 77, 128, 128, 16),
    (1, 3, 150, 32, 64, 32),
    (1, 2, 130, 32, 32, 64),
    (1, 2, 200, 96, 192, 64),
    (1, 2, 97, 96, 96, 32),
    (1, 2, 150, 256, 64, 32),
    (1, 1, 70, 256, 128, 16),
    (16, 16, 65, 64, 64, 16),     # four scan waves, 16-token chunks
    (1, 2, 150, 16, 64, 64),      # d_k 16: zero-padded to the d_k 32 kernel
    (1, 3, 97, 16, 32, 32),
    (2, 2, 70, 16, 48, 16),
    (8, 16, 130, 16, 64, 64),     # d_k 16 with two scan waves
]


@pytest.mark.parametrize("B,H,T,dk,dv,C", NEW_SHAPES)
def test_fast_path_shapes(B, H, T, dk, dv, C):
    x = make_random(B, H, T, dk, dv, dtype="bf16", chunk=C, seed=7 * T + dk, s0_std=0.02)
    say(f"case: bf16 B{B} H{H} T{T} dk{dk} dv{dv} C{C}")
    d = to_dev(x)
    O, S = nan_outputs(x)
    gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], chunk_size=C,
                      O=O, S_final=S)
    torch.cuda.synchronize()
    check_all(x, O, S, TOL["bf16"], f"bf16 {B}x{H}x{T} dk{dk} dv{dv} C{C}")


def test_olmo_hybrid_head_shape():
    """"从电路复杂性理论的角度分析大模型的可并行性和表达能力--Olmo Hybrid 系列",
    Olmo Hybrid architecture: 30 heads, q/k head dim 96, v head dim 192, the
    erase strength in (0, 2) (beta replaced by 2 beta).  B * H = 60 is not a
    multiple of 8, so the workgroups of one head are not grouped on one XCD."""
    B, H, T, dk, dv, C = 2, 30, 600, 96, 192, 64
    x = make_random(B, H, T, dk, dv, dtype="bf16", chunk=C, seed=30, s0_std=0.02)
    x["beta"] = (2.0 * x["beta"]).contiguous()
    say("case: Olmo-Hybrid heads B2 H30 T600 dk96 dv192 C64, beta in (0, 2)")
    d = to_dev(x)
    O, S = nan_outputs(x)
    gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], chunk_size=C,
                      O=O, S_final=S)
    torch.cuda.synchronize()
    check_all(x, O, S, TOL["bf16"], "olmo B2 H30 T600")


# ------------------------------------------------- precise (split-bf16) path

def reflections(B, H, T, dk, dv, seed):
    x = make_random(B, H, T, dk, dv, dtype="bf16", chunk=64, seed=seed, s0_std=0.5)
    kk = (x["k"].float() ** 2).sum(-1)
    x["beta"] = (2.0 / kk).float().contiguous()
    x["alpha"] = None
    return x


def test_precise_path_long_reflections():
    """Every token a Householder reflection and no decay over 32 chunks: the
    state keeps every rounding.  The split-bf16 path stays near 1e-5; the
    fast path's error is printed beside it (it grows about as the square
    root of the number of chunks)."""
    x = reflections(1, 2, 2048, 128, 128, seed=43)
    d = to_dev(x)
    say("case: all reflections, alpha = 1, T2048: precise vs fast")
    O, S = nan_outputs(x)
    gdn.gdn_chunk_fwd_precise(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                              chunk_size=64, O=O, S_final=S)
    torch.cuda.synchronize()
    check_all(x, O, S, 1e-4, "precise, reflections T2048")
    Of, Sf = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], chunk_size=64)
    torch.cuda.synchronize()
    Or, Sr = oracle_all(x)
    say(f"  fast path on the same input: O {rel_err(Of.cpu().numpy(), Or):.3e} "
        f"S {rel_err(Sf.cpu().numpy(), Sr):.3e}")


@pytest.mark.parametrize("B,H,T,dk,dv,C", [
    (4, 16, 333, 128, 128, 64),
    (1, 2, 200, 64, 64, 32),
    (1, 2, 100, 32, 64, 64),      # generic split kernel (d_k 32)
])
def test_precise_path_shapes(B, H, T, dk, dv, C):
    x = make_random(B, H, T, dk, dv, dtype="bf16", chunk=C, seed=T + 5, s0_std=0.02)
    d = to_dev(x)
    say(f"case: precise B{B} H{H} T{T} dk{dk} dv{dv} C{C}")
    O, S = nan_outputs(x)
    gdn.gdn_chunk_fwd_precise(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                              chunk_size=C, O=O, S_final=S)
    torch.cuda.synchronize()
    check_all(x, O, S, 1e-4, f"precise {B}x{H}x{T} dk{dk} C{C}")
