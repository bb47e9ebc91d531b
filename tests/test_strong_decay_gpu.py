"""Strong gates on the GPU path, against the fp64 oracle (all heads).

The decay-masked matrices of a chunk use the ratios exp(g_r - g_i) of the
chunk-local cumulative log-gate g ("从零开始的 GDN 推导", UT transform: the
Gamma and Gamma^{-1} factors only enter as such ratios).  Within a chunk the
kernel forms them either as a product of a row factor and a column factor
(when the chunk's whole decay range keeps both far inside fp32) or as one
exponential per ratio.  Weak gates (alpha near 1) take the first form; the
gates here (alpha = exp(-softplus(N) * s) with s up to 8, i.e. alpha down to
about 1e-3) drive the second, alone and interleaved chunk by chunk with
weakly gated chunks, at both chunk sizes, with one, two and four scan waves,
ragged T, with and without a separate write strength.
"""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_13_amd as gdn
from gated_delta_rule_13_amd.workloads import chunk_scaled_alpha, make_random
from tests.gpu_helpers import TOL, elem_err, nan_outputs, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

# (B, H, T, d_k, d_v, C, gate scales per chunk, with eta)
# scan waves per workgroup follow from the launch's rounds of workgroups
# (see test_parity_gpu); four scan waves at C = 32 run beside six prep waves
CASES = [
    (1, 2, 333, 128, 128, 64, (4.0,), False),            # one scan wave, all strong
    (1, 2, 333, 128, 128, 64, (0.05, 4.0), False),       # alternating weak / strong
    (1, 3, 201, 64, 64, 32, (4.0, 0.05, 8.0), False),    # C = 32, d_k 64
    (1, 2, 150, 128, 128, 32, (0.05, 4.0), True),        # eta, C = 32
    (4, 16, 150, 128, 128, 64, (0.05, 4.0), False),      # two scan waves
    (4, 16, 97, 64, 128, 32, (4.0,), True),              # two scan waves, d_k 64, eta
    (8, 16, 150, 128, 128, 64, (4.0, 0.05), False),      # four scan waves
    (16, 16, 97, 128, 128, 32, (8.0, 0.05), True),       # four scan waves, C = 32, eta
    (8, 32, 130, 64, 64, 64, (0.05, 4.0), False),        # four scan waves, d_k 64
    (2, 30, 150, 96, 192, 64, (0.05, 4.0), False),       # three scan waves
    (2, 30, 97, 96, 192, 64, (4.0,), True),              # three scan waves, eta
]


def decay_range_log2(alpha: torch.Tensor, chunk: int) -> float:
    """Largest span of the cumulative log2-gate within one chunk."""
    T = alpha.shape[-1]
    worst = 0.0
    for t0 in range(0, T, chunk):
        a = alpha[..., t0:t0 + chunk].double()
        worst = max(worst, float((-torch.log2(a)).sum(-1).max()))
    return worst


@pytest.mark.parametrize("B,H,T,dk,dv,C,scales,with_eta", CASES)
def test_strong_gates_match_oracle(B, H, T, dk, dv, C, scales, with_eta):
    seed = B * 1000 + T + dk
    x = make_random(B, H, T, dk, dv, dtype="bf16", chunk=C, seed=seed, s0_std=0.02)
    x["alpha"] = chunk_scaled_alpha(B, H, T, C, scales, seed=seed + 1)
    eta = None
    if with_eta:
        g = torch.Generator().manual_seed(seed + 2)
        eta = torch.rand(B, H, T, generator=g).float()
    span = decay_range_log2(x["alpha"], C)
    say(f"case: strong gates B{B} H{H} T{T} dk{dk} dv{dv} C{C} scales {scales} "
        f"eta {with_eta}: largest in-chunk log2 decay span {span:.0f}")
    # the per-ratio exponential form must be exercised (span > 96)
    assert span > 96
    d = to_dev(x)
    O, S = nan_outputs(x)
    gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], chunk_size=C,
                      O=O, S_final=S, eta=None if eta is None else eta.cuda())
    torch.cuda.synchronize()
    Or, Sr = oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"], eta=eta)
    Og, Sg = O.cpu().numpy(), S.cpu().numpy()
    assert np.isfinite(Og).all() and np.isfinite(Sg).all()
    eo, es = rel_err(Og, Or), rel_err(Sg, Sr)
    say(f"  O rel err {eo:.3e}  S rel err {es:.3e}; elementwise O {elem_err(Og, Or):.3e} "
        f"S {elem_err(Sg, Sr):.3e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


def test_gate_underflow_to_zero():
    """Gates so strong that exp(g) underflows fp32 inside every chunk
    (alpha about 1e-6 per token): the state is forgotten almost at once and
    each output is dominated by its own token's write."""
    B, H, T, dk, dv, C = 1, 2, 200, 128, 128, 64
    x = make_random(B, H, T, dk, dv, dtype="bf16", chunk=C, seed=31, s0_std=0.5)
    x["alpha"] = torch.full((B, H, T), 1e-6)
    say("case: alpha = 1e-6 everywhere (exp(g) underflows within a chunk)")
    d = to_dev(x)
    O, S = nan_outputs(x)
    gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], chunk_size=C,
                      O=O, S_final=S)
    torch.cuda.synchronize()
    Or, Sr = oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"])
    Og, Sg = O.cpu().numpy(), S.cpu().numpy()
    assert np.isfinite(Og).all() and np.isfinite(Sg).all()
    eo, es = rel_err(Og, Or), rel_err(Sg, Sr)
    say(f"  O rel err {eo:.3e}  S rel err {es:.3e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]
