"""The algebra the sequence-parallel form rests on, checked on the CPU with
the fp64 oracle alone (no GPU code involved).

The state recurrence S_t = S_{t-1} A_t + eta_t v_t k_t^T, A_t = alpha_t (I -
beta_t k_t k_t^T), is affine in the state ("Параллельность RNN?", section
"Уровень 2": a linear recurrence is associative).  Over a segment that starts
from X:
    end state  = X M + E0,       o_t = o0_t + X qm_t,
with M = A_first ... A_last (the recurrence from S0 = I with zero values,
d_v = d_k), qm_t that run's outputs, and E0, o0 the run from a zero state.
Composing the pieces of every segment, with X_1 = the first segment's end
state and X_{j+1} = X_j M_j + E0_j, must reproduce the plain recurrence over
the whole sequence to fp64 rounding, for any cut into segments.
"""
import numpy as np
import pytest

import oracle
from gated_delta_rule_13_amd.workloads import make_random


def run(x, a, b, S0, eta, zero_values=False, identity=False):
    cut = lambda t: None if t is None else t[..., a:b, :] if t.dim() == 4 else t[..., a:b]
    q, k, v = cut(x["q"]), cut(x["k"]), cut(x["v"])
    B, H, _, dk = q.shape
    if zero_values:
        v = np.zeros((B, H, b - a, dk))
    if identity:
        S0 = np.broadcast_to(np.eye(dk), (B, H, dk, dk)).copy()
    return oracle.recurrent(q, k, v, cut(x["alpha"]), cut(x["beta"]), S0=S0, eta=cut(eta))


@pytest.mark.parametrize("cuts,with_eta", [((40,), False), ((16, 50, 90), True),
                                           ((1, 2, 3, 100), False), ((64,), True)])
def test_segments_compose_to_the_recurrence(cuts, with_eta):
    import torch
    B, H, T, dk, dv = 1, 2, 120, 8, 6
    x = make_random(B, H, T, dk, dv, dtype="f32", chunk=16, seed=len(cuts) + 3,
                    alpha_scale=0.3, s0_std=0.5)
    eta = None
    if with_eta:
        eta = torch.rand(B, H, T, generator=torch.Generator().manual_seed(9)) * 1.5
    O_ref, S_ref = oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"],
                                    eta=eta)
    bounds = [0, *cuts, T]
    O = np.zeros_like(O_ref)
    X = None
    for j in range(len(bounds) - 1):
        a, b = bounds[j], bounds[j + 1]
        if j == 0:
            O[:, :, a:b], X = run(x, a, b, x["S0"], eta)
            continue
        o0, E0 = run(x, a, b, None, eta)
        qm, M = run(x, a, b, None, eta, zero_values=True, identity=True)
        # o_t = o0_t + X qm_t ; end = X M + E0
        O[:, :, a:b] = o0 + np.einsum("bhck,bhtk->bhtc", X, qm)
        X = np.einsum("bhck,bhkd->bhcd", X, M) + E0
    scale_o, scale_s = np.abs(O_ref).max(), np.abs(S_ref).max()
    assert np.abs(O - O_ref).max() <= 1e-12 * scale_o
    assert np.abs(X - S_ref).max() <= 1e-12 * scale_s


def test_transition_is_the_product_of_generalised_householder_factors():
    """M from the identity-start run equals the explicit ordered product of
    alpha_t (I - beta_t k_t k_t^T) (the pages' transition), written out."""
    B, H, T, dk, dv = 1, 1, 7, 5, 3
    x = make_random(B, H, T, dk, dv, dtype="f32", chunk=16, seed=2, alpha_scale=0.5)
    _, M = run(x, 0, T, None, None, zero_values=True, identity=True)
    k = x["k"][0, 0].double().numpy()
    alpha = x["alpha"][0, 0].double().numpy()
    beta = x["beta"][0, 0].double().numpy()
    P = np.eye(dk)
    for t in range(T):
        P = P @ (alpha[t] * (np.eye(dk) - beta[t] * np.outer(k[t], k[t])))
    assert np.abs(M[0, 0] - P).max() <= 1e-13
