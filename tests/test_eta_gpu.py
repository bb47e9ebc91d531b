"""Separate write strength eta on the GPU paths (gdn_chunk_fwd_eta,
gdn_recurrent_fwd_eta), against the fp64 oracle and against a closed form.

With erase strength beta = 0, write strength eta = 1 and a zero initial
state the method is gated linear attention ("从电路复杂性理论的角度分析大模型
的可并行性和表达能力", GLA): O = ((Q K^T) * Gamma) V with
Gamma_ij = gamma_i / gamma_j (i >= j), gamma_i = prod_{l <= i} alpha_l, and
S_T = sum_t (gamma_T / gamma_t) v_t k_t^T.  That closed form is evaluated here
in fp64 from the same rounded inputs and pins the GPU paths directly.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_13_amd as gdn
from gated_delta_rule_13_amd.workloads import make_random
from tests.gpu_helpers import TOL, rel_err, run_oracle, say, to_dev

import oracle

pytestmark = pytest.mark.gpu


def gla_closed_form(x):
    q = x["q"].double().numpy()
    k = x["k"].double().numpy()
    v = x["v"].double().numpy()
    a = x["alpha"].double().numpy()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    O = np.zeros((B, H, T, dv))
    S = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            g = np.cumsum(np.log(a[b, h]))
            gam = np.tril(np.exp(g[:, None] - g[None, :]))
            O[b, h] = ((q[b, h] @ k[b, h].T) * gam) @ v[b, h]
            S[b, h] = (v[b, h] * np.exp(g[-1] - g)[:, None]).T @ k[b, h]
    return O, S


def oracle_eta(x, eta):
    return oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"], eta=eta)


def gla_inputs(T, dk, dv, dtype, seed):
    x = make_random(2, 2, T, dk, dv, dtype=dtype, seed=seed, alpha_scale=0.1)
    x["beta"] = torch.zeros_like(x["beta"])
    return x, torch.ones_like(x["beta"])


@pytest.mark.parametrize("path,dtype,T,dk,dv,chunk", [
    ("chunked", "bf16", 300, 128, 128, 64),
    ("chunked", "bf16", 97, 64, 96, 32),
    ("chunked", "f32", 70, 32, 48, 16),
    ("recurrent", "bf16", 9, 128, 128, None),
    ("recurrent", "f32", 5, 96, 192, None),
])
def test_gla_reduction_closed_form(path, dtype, T, dk, dv, chunk):
    x, eta = gla_inputs(T, dk, dv, dtype, seed=T + dk)
    say(f"case: GLA (beta 0, eta 1) {path} {dtype} T{T} dk{dk} dv{dv}")
    d = to_dev(x)
    if path == "chunked":
        O, S = gdn.gdn_chunk_fwd_eta(d["q"], d["k"], d["v"], d["alpha"], d["beta"], eta.cuda(),
                                     None, chunk_size=chunk)
    else:
        O, S = gdn.gdn_recurrent_fwd_eta(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                         eta.cuda(), None)
    torch.cuda.synchronize()
    Oc, Sc = gla_closed_form(x)
    eo, es = rel_err(O.cpu().numpy(), Oc), rel_err(S.cpu().numpy(), Sc)
    say(f"  vs closed form: O {eo:.3e}  S {es:.3e}")
    assert eo < TOL[dtype] and es < TOL[dtype]
    Or, Sr = oracle_eta(x, eta)
    assert rel_err(O.cpu().numpy(), Or) < TOL[dtype]
    assert rel_err(S.cpu().numpy(), Sr) < TOL[dtype]


@pytest.mark.parametrize("path,dtype,T,dk,dv,chunk", [
    ("chunked", "bf16", 333, 128, 128, 64),
    ("chunked", "bf16", 130, 128, 64, 32),
    ("chunked", "bf16", 200, 32, 64, 64),     # older fused kernel (d_k 32)
    ("chunked", "f32", 77, 64, 32, 32),
    ("recurrent", "bf16", 6, 128, 128, None),
    ("recurrent", "f32", 4, 16, 16, None),
])
def test_random_eta_vs_oracle(path, dtype, T, dk, dv, chunk):
    x = make_random(2, 3, T, dk, dv, dtype=dtype, seed=7 * T + dk, s0_std=0.05)
    g = torch.Generator().manual_seed(T)
    eta = 1.5 * torch.rand(x["beta"].shape, generator=g)
    say(f"case: random eta {path} {dtype} T{T} dk{dk} dv{dv}")
    d = to_dev(x)
    if path == "chunked":
        O, S = gdn.gdn_chunk_fwd_eta(d["q"], d["k"], d["v"], d["alpha"], d["beta"], eta.cuda(),
                                     d["S0"], chunk_size=chunk)
    else:
        O, S = gdn.gdn_recurrent_fwd_eta(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                         eta.cuda(), d["S0"])
    torch.cuda.synchronize()
    Or, Sr = oracle_eta(x, eta)
    eo, es = rel_err(O.cpu().numpy(), Or), rel_err(S.cpu().numpy(), Sr)
    say(f"  O {eo:.3e}  S {es:.3e}")
    assert eo < TOL[dtype] and es < TOL[dtype]


def test_null_eta_is_the_plain_entry():
    x = make_random(2, 2, 150, 128, 128, seed=3, s0_std=0.05)
    d = to_dev(x)
    say("case: eta = NULL and eta = beta vs the plain entry")
    O0, S0 = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    O1, S1 = gdn.gdn_chunk_fwd_eta(d["q"], d["k"], d["v"], d["alpha"], d["beta"], None, d["S0"])
    O2, S2 = gdn.gdn_chunk_fwd_eta(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                   d["beta"].clone(), d["S0"])
    torch.cuda.synchronize()
    assert torch.equal(O0, O1) and torch.equal(S0, S1)
    # eta given explicitly takes the unfactored right-hand side
    # diag(eta) V - diag(beta exp g) K S^T: the same values up to rounding,
    # so both lie within the tolerance of the exact result
    Or, Sr = oracle_eta(x, None)
    for O_, S_ in ((O0, S0), (O2, S2)):
        assert rel_err(O_.cpu().numpy(), Or) < TOL["bf16"]
        assert rel_err(S_.cpu().numpy(), Sr) < TOL["bf16"]


@pytest.mark.parametrize("B,H,T,dk,dv,C,waves", [
    (4, 16, 200, 128, 128, 64, "two scan waves"),
    (2, 30, 150, 96, 192, 64, "three scan waves"),
    (16, 16, 97, 128, 128, 32, "four scan waves, six prep waves"),
    (8, 32, 70, 64, 64, 64, "four scan waves, four prep waves"),
])
def test_random_eta_scan_wave_counts_ragged(B, H, T, dk, dv, C, waves):
    """Random eta on head counts that run two, three or four scan waves per
    workgroup, ragged T, every head against the oracle."""
    x = make_random(B, H, T, dk, dv, chunk=C, seed=23 + T, s0_std=0.05)
    g = torch.Generator().manual_seed(23 + T)
    eta = 1.5 * torch.rand(x["beta"].shape, generator=g)
    say(f"case: random eta, B{B} H{H} T{T} dk{dk} dv{dv} C{C} ({waves}, all heads)")
    d = to_dev(x)
    O, S = gdn.gdn_chunk_fwd_eta(d["q"], d["k"], d["v"], d["alpha"], d["beta"], eta.cuda(),
                                 d["S0"], chunk_size=C)
    torch.cuda.synchronize()
    Or, Sr = oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"], eta=eta)
    eo, es = rel_err(O.cpu().numpy(), Or), rel_err(S.cpu().numpy(), Sr)
    say(f"  O {eo:.3e}  S {es:.3e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]
