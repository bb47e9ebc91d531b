"""The rest of the shape matrix the boundary accepts: fp32 inputs with
d_k 128 and 256 (on the generic kernel), and d_k 256 with 64-token chunks
(bf16 and fp32; computed as 32-token chunks),
through gdn_chunk_fwd, gdn_chunk_fwd_eta and gdn_chunk_fwd_precise, every
(b, h) sequence against the fp64 oracle, with NaN-prefilled outputs; and
the stage kernel's T, W, U at the new shapes against the pages' chunk
matrices ("从零开始的 GDN 推导", UT transform and S update; S of size
d_v x d_k with no restriction on either, "RNN的复兴03", section 4).
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

SHAPES = [
    # (dtype, B, H, T, dk, dv, C)
    ("f32", 1, 2, 150, 128, 64, 64),
    ("f32", 2, 2, 77, 128, 128, 32),
    ("f32", 1, 3, 50, 128, 32, 16),
    ("f32", 1, 2, 70, 256, 64, 32),
    ("f32", 1, 1, 45, 256, 48, 16),
    ("f32", 8, 8, 100, 128, 64, 32),    # 64 heads: several waves per workgroup
    ("f32", 1, 2, 150, 256, 64, 64),    # chunk 64 at d_k 256: run as 32-token chunks
    ("bf16", 1, 2, 150, 256, 64, 64),
]


def check(x, O, S, tol, label, eta=None):
    Or, Sr = oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"], eta=eta)
    Og, Sg = O.float().cpu().numpy(), S.cpu().numpy()
    assert np.isfinite(Og).all() and np.isfinite(Sg).all(), "unwritten or non-finite output"
    eo, es = rel_err(Og, Or), rel_err(Sg, Sr)
    say(f"{label}: O {eo:.3e}  S {es:.3e}  (tol {tol:.0e}); elementwise O {elem_err(Og, Or):.3e} "
        f"S {elem_err(Sg, Sr):.3e}")
    assert eo < tol and es < tol


@pytest.mark.parametrize("dtype,B,H,T,dk,dv,C", SHAPES)
def test_boundary_shapes(dtype, B, H, T, dk, dv, C):
    x = make_random(B, H, T, dk, dv, dtype=dtype, chunk=C, seed=3 * T + dk, s0_std=0.02)
    say(f"case: {dtype} B{B} H{H} T{T} dk{dk} dv{dv} C{C}")
    d = to_dev(x)
    O, S = nan_outputs(x)
    gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], chunk_size=C,
                      O=O, S_final=S)
    torch.cuda.synchronize()
    check(x, O, S, TOL[dtype], f"{dtype} dk{dk} C{C}")


@pytest.mark.parametrize("dtype,B,H,T,dk,dv,C", [SHAPES[1], SHAPES[3]])
def test_boundary_shapes_eta_and_precise(dtype, B, H, T, dk, dv, C):
    x = make_random(B, H, T, dk, dv, dtype=dtype, chunk=C, seed=T + 11, s0_std=0.02)
    g = torch.Generator().manual_seed(T)
    eta = 1.5 * torch.rand(x["beta"].shape, generator=g)
    say(f"case: eta + precise {dtype} B{B} H{H} T{T} dk{dk} dv{dv} C{C}")
    d = to_dev(x)
    O, S = nan_outputs(x)
    gdn.gdn_chunk_fwd_eta(d["q"], d["k"], d["v"], d["alpha"], d["beta"], eta.cuda(), d["S0"],
                          chunk_size=C, O=O, S_final=S)
    torch.cuda.synchronize()
    check(x, O, S, TOL[dtype], "eta", eta=eta)
    O, S = nan_outputs(x)
    gdn.gdn_chunk_fwd_precise(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                              chunk_size=C, O=O, S_final=S)
    torch.cuda.synchronize()
    check(x, O, S, TOL[dtype], "precise")


@pytest.mark.parametrize("dtype,T,dk,dv,C", [("f32", 70, 128, 32, 32), ("f32", 40, 256, 16, 16),
                                             ("f32", 130, 128, 16, 64)])
def test_stage_kernel_new_shapes(dtype, T, dk, dv, C):
    x = make_random(1, 2, T, dk, dv, dtype=dtype, chunk=C, seed=T)
    say(f"case: prep {dtype} T{T} dk{dk} dv{dv} C{C}")
    d = {k_: (None if x[k_] is None else x[k_].cuda()) for k_ in ("k", "v", "alpha", "beta")}
    out = gdn.gdn_chunk_prep(d["k"], d["v"], d["alpha"], d["beta"], chunk_size=C)
    torch.cuda.synchronize()
    tol = 1e-4 if dtype == "bf16" else 1e-5
    k64, v64 = x["k"].double().numpy(), x["v"].double().numpy()
    a64, b64 = x["alpha"].double().numpy(), x["beta"].double().numpy()
    for h in range(2):
        for c, t0 in enumerate(range(0, T, C)):
            t1 = min(T, t0 + C)
            m = cr.gated_chunk_matrices(k64[0, h, t0:t1], v64[0, h, t0:t1], a64[0, h, t0:t1],
                                        b64[0, h, t0:t1])
            L = t1 - t0
            assert rel_err(out["T"][0, h, c].cpu().double().numpy()[:L, :L], m["T"]) < tol
            assert rel_err(out["W"][0, h, t0:t1].cpu().numpy(), m["W"]) < tol
            assert rel_err(out["U"][0, h, t0:t1].cpu().numpy(), m["U"]) < tol
