"""Pins of the fp64 recurrent oracle against what the pages and mathematics fix.

Each ``pin_*`` takes ``orc(q, k, v, alpha, beta, S0=None, eta=None) -> (O, S)``
(batched numpy arrays, the oracle's calling convention) and raises
AssertionError when the oracle disagrees with the pinned value.  None of them
re-types the oracle's own update: each compares against a closed form, an
invariant, a second formulation from another page, or the chunked WY/UT form.
``tests/test_oracle_mutants.py`` checks that every planted mistake in the
oracle trips at least one of them.
"""
from __future__ import annotations

import numpy as np

from oracle import chunked_ref as cr

RNG_SEED = 1234


def _rng(salt=0):
    return np.random.default_rng(RNG_SEED + salt)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rel(x, ref):
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-300))


def _inputs(B=1, H=2, T=24, dk=6, dv=5, salt=0, s0=True):
    r = _rng(salt)
    q = _unit(r.standard_normal((B, H, T, dk)))
    k = _unit(r.standard_normal((B, H, T, dk)))
    v = r.standard_normal((B, H, T, dv))
    alpha = r.uniform(0.6, 1.0, (B, H, T))
    beta = r.uniform(0.05, 1.9, (B, H, T))
    S0 = 0.3 * r.standard_normal((B, H, dv, dk)) if s0 else None
    return q, k, v, alpha, beta, S0


def pin_linear_attention(orc, tol=1e-12):
    """Circuit-complexity page, "类 RNN 模型训练": S_t = S_{t-1} + v_t k_t^T,
    o_t = S_t q_t, whose parallel form is O = (Q K^T ⊙ M) V with a causal M
    that keeps the diagonal.  Reached with alpha = 1, erase 0, write 1,
    S0 = 0; then also S_T = V^T K."""
    q, k, v, _, _, _ = _inputs(dk=6, dv=6, salt=1)
    B, H, T, _ = q.shape
    zeros, ones = np.zeros((B, H, T)), np.ones((B, H, T))
    O, S = orc(q, k, v, None, zeros, S0=None, eta=ones)
    for b in range(B):
        for h in range(H):
            Q, K, V = q[b, h], k[b, h], v[b, h]
            O_ref = np.tril(Q @ K.T) @ V
            assert _rel(O[b, h], O_ref) < tol, "linear attention output"
            assert _rel(S[b, h], V.T @ K) < tol, "linear attention state"


def gla_closed_form(Q, K, V, alpha):
    """Circuit-complexity page, gated linear attention: gamma_j = prod_{i<=j}
    alpha_i, O = ((Q K^T) ⊙ Gamma) V with Gamma_ij = gamma_i / gamma_j for
    i >= j, zero otherwise; the state is sum_i (gamma_T / gamma_i) v_i k_i^T."""
    gamma = np.cumprod(alpha)
    Gam = np.tril(gamma[:, None] / gamma[None, :])
    O = ((Q @ K.T) * Gam) @ V
    S = (V * (gamma[-1] / gamma)[:, None]).T @ K
    return O, S


def pin_gated_linear_attention(orc, tol=1e-12):
    """Erase strength 0 and write strength 1 turn the recurrence into gated
    linear attention (circuit-complexity page, Mamba2 form)."""
    q, k, v, alpha, _, _ = _inputs(dk=5, dv=7, salt=2)
    B, H, T, _ = q.shape
    O, S = orc(q, k, v, alpha, np.zeros((B, H, T)), S0=None, eta=np.ones((B, H, T)))
    for b in range(B):
        for h in range(H):
            O_ref, S_ref = gla_closed_form(q[b, h], k[b, h], v[b, h], alpha[b, h])
            assert _rel(O[b, h], O_ref) < tol, "GLA output"
            assert _rel(S[b, h], S_ref) < tol, "GLA state"


def pin_gla_small_beta_limit(orc, tol=1e-6):
    """Second reading of "beta = 0 reduces to gated linear attention" with the
    write tied to beta: O(beta = eps) / eps tends to the GLA output as eps -> 0
    (error O(eps))."""
    q, k, v, alpha, _, _ = _inputs(dk=5, dv=4, salt=3)
    B, H, T, _ = q.shape
    eps = 1e-8
    O, _ = orc(q, k, v, alpha, np.full((B, H, T), eps), S0=None)
    for b in range(B):
        for h in range(H):
            O_ref, _ = gla_closed_form(q[b, h], k[b, h], v[b, h], alpha[b, h])
            assert _rel(O[b, h] / eps, O_ref) < tol, "small-beta limit"


def pin_householder_orthogonality(orc, tol=1e-12):
    """First page, section 1: with beta = 2 / (k^T k) the transition E - beta k k^T
    is a Householder reflection (orthogonal, an involution).  With alpha = 1
    and no writes (v = 0) the state is S_T = S_0 H_1 ... H_T, so its Frobenius
    norm and singular values are those of S_0 (circuit-complexity page:
    orthogonal maps preserve length), and two identical consecutive
    reflections leave S_0 unchanged."""
    r = _rng(4)
    B, H, T, dk, dv = 1, 2, 9, 6, 4
    q = _unit(r.standard_normal((B, H, T, dk)))
    k = r.standard_normal((B, H, T, dk))          # not normalised on purpose
    v = np.zeros((B, H, T, dv))
    beta = 2.0 / np.sum(k * k, axis=-1)
    S0 = r.standard_normal((B, H, dv, dk))
    O, S = orc(q, k, v, None, beta, S0=S0)
    for b in range(B):
        for h in range(H):
            P = cr.householder_like_product(k[b, h], beta[b, h])
            assert np.abs(P.T @ P - np.eye(dk)).max() < tol, "reflection product orthogonal"
            assert _rel(S[b, h], S0[b, h] @ P) < tol, "state = S0 times reflections"
            assert abs(np.linalg.norm(S[b, h]) - np.linalg.norm(S0[b, h])) < tol * np.linalg.norm(S0[b, h])
            sv = np.linalg.svd(S[b, h], compute_uv=False)
            sv0 = np.linalg.svd(S0[b, h], compute_uv=False)
            assert np.abs(sv - sv0).max() < tol * sv0.max(), "singular values preserved"
    # two identical reflections in a row cancel
    k2 = np.repeat(k[:, :, :1], 2, axis=2)
    beta2 = 2.0 / np.sum(k2 * k2, axis=-1)
    _, S2 = orc(q[:, :, :2], k2, v[:, :, :2], None, beta2, S0=S0)
    assert _rel(S2, S0) < tol, "reflection is an involution"


def pin_delta_retrieval(orc, tol=1e-12):
    """Circuit-complexity page, DeltaNet: with write strength 1 and a unit key,
    the state retrieves what was just written, S_t k_t = v_t, whatever the
    earlier state and the gate.  Reading with q_t = k_t: o_t = v_t."""
    q, k, v, alpha, _, S0 = _inputs(dk=7, dv=5, salt=5)
    B, H, T, _ = k.shape
    O, _ = orc(k, k, v, alpha, np.ones((B, H, T)), S0=S0)
    assert _rel(O, v) < tol, "exact retrieval"


def pin_old_new_value_form(orc, tol=1e-13):
    """Circuit-complexity page, DeltaNet: S_t = S_{t-1} - v_old k_t^T + v_new k_t^T
    with v_old = S_{t-1} k_t and v_new = beta_t v_t + (1 - beta_t) v_old (no gate)."""
    q, k, v, _, beta, S0 = _inputs(dk=6, dv=3, salt=6)
    beta = np.clip(beta, 0.0, 1.0)
    B, H, T, _ = q.shape
    O, S = orc(q, k, v, None, beta, S0=S0)
    for b in range(B):
        for h in range(H):
            St = S0[b, h].copy()
            Oref = np.zeros((T, v.shape[-1]))
            for t in range(T):
                kt = k[b, h, t]
                v_old = St @ kt
                v_new = beta[b, h, t] * v[b, h, t] + (1 - beta[b, h, t]) * v_old
                St = St - np.outer(v_old, kt) + np.outer(v_new, kt)
                Oref[t] = St @ q[b, h, t]
            assert _rel(O[b, h], Oref) < tol and _rel(S[b, h], St) < tol, "v_old/v_new form"


def pin_recurrent_equals_chunked(orc, tol=1e-12):
    """"从零开始的 GDN 推导": the chunkwise pass (UT transform, W and U, state
    and output per chunk, chunks chained) equals the recurrence for any chunk
    length, a ragged last chunk included."""
    q, k, v, alpha, beta, S0 = _inputs(B=1, H=2, T=37, dk=6, dv=5, salt=7)
    O, S = orc(q, k, v, alpha, beta, S0=S0)
    for C in (1, 3, 8, 16, 37, 64):
        for h in range(2):
            Oc, Sc = cr.chunked_forward(q[0, h], k[0, h], v[0, h], alpha[0, h], beta[0, h],
                                        S0[0, h], chunk_size=C)
            assert _rel(O[0, h], Oc) < tol and _rel(S[0, h], Sc) < tol, f"chunked C={C}"


def pin_state_parallel_form(orc, tol=1e-12):
    """First page, section 3.1: with no gate,
    S_t = S_0 (E - W^T K) + U^T K, W and U from their row recursions
    (w_t with beta, u_t with the separate write strength eta)."""
    q, k, v, _, beta, S0 = _inputs(dk=6, dv=4, salt=8)
    eta = _rng(9).uniform(0.1, 1.5, beta.shape)
    B, H, T, dk = q.shape
    _, S = orc(q, k, v, None, beta, S0=S0, eta=eta)
    for b in range(B):
        for h in range(H):
            W = cr.w_recursion(k[b, h], beta[b, h])
            U = cr.u_recursion(k[b, h], v[b, h], beta[b, h], eta[b, h])
            S_ref = S0[b, h] @ (np.eye(dk) - W.T @ k[b, h]) + U.T @ k[b, h]
            assert _rel(S[b, h], S_ref) < tol, "state-parallel form"


def pin_chaining(orc, tol=1e-13):
    """"从零开始的 GDN 推导", summary: each chunk's output state is the next
    chunk's input state, so splitting the sequence anywhere and feeding
    S_final back as S0 gives the same result."""
    q, k, v, alpha, beta, S0 = _inputs(T=29, salt=10)
    O, S = orc(q, k, v, alpha, beta, S0=S0)
    t1 = 11
    O1, S1 = orc(q[:, :, :t1], k[:, :, :t1], v[:, :, :t1], alpha[:, :, :t1], beta[:, :, :t1], S0=S0)
    O2, S2 = orc(q[:, :, t1:], k[:, :, t1:], v[:, :, t1:], alpha[:, :, t1:], beta[:, :, t1:], S0=S1)
    assert _rel(np.concatenate([O1, O2], axis=2), O) < tol and _rel(S2, S) < tol, "chaining"


def pin_linearity(orc, tol=1e-12):
    """The map (V, S0) -> (O, S_T) is linear for fixed q, k, alpha, beta (every
    transition is affine in the state with the write linear in v)."""
    q, k, v, alpha, beta, S0 = _inputs(salt=11)
    r = _rng(12)
    v2 = r.standard_normal(v.shape)
    S02 = r.standard_normal(S0.shape)
    Oa, Sa = orc(q, k, v, alpha, beta, S0=S0)
    Ob, Sb = orc(q, k, v2, alpha, beta, S0=S02)
    Oc, Sc = orc(q, k, 2.5 * v - 0.5 * v2, alpha, beta, S0=2.5 * S0 - 0.5 * S02)
    assert _rel(Oc, 2.5 * Oa - 0.5 * Ob) < tol and _rel(Sc, 2.5 * Sa - 0.5 * Sb) < tol, "linearity"


ALL_PINS = [
    pin_linear_attention,
    pin_gated_linear_attention,
    pin_gla_small_beta_limit,
    pin_householder_orthogonality,
    pin_delta_retrieval,
    pin_old_new_value_form,
    pin_recurrent_equals_chunked,
    pin_state_parallel_form,
    pin_chaining,
    pin_linearity,
]
