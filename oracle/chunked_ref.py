"""fp64 numpy forms of the WY / UT algebra and of the chunkwise forward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Shares no code with
the GPU library.

Orientation: the state S is d_v x d_k and o = S q, as on
"RNN的复兴03:现代RNN的并行计算" (section 4 states dim S = d_v x d_k) and on the
circuit-complexity page ("类 RNN 模型训练").  "从零开始的 GDN 推导" writes the
transpose (keys and values as row vectors, S of d_k x d_v); its formulas are
transposed on use and each function says where.  The lower-triangular
matrices follow the first page's naming: A is strictly lower with
A_ij = -beta_i k_j^T k_i (i > j) and T = (E - A)^{-1}.  The second page calls
L = StrictLower(B Gamma K K^T Gamma^{-1}) and names (I + L)^{-1} "A"; here
that matrix is T and A = -L.

Every function takes plain numpy arrays of one sequence (no batch / head
axes) and returns float64 arrays.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "householder_like_product",
    "w_recursion",
    "u_recursion",
    "strict_lower_A",
    "forward_substitution",
    "gated_chunk_matrices",
    "chunked_forward",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def householder_like_product(K, beta):
    """Explicit P = H_1 H_2 ... H_t with H_tau = E - beta_tau k_tau k_tau^T.

    First page, section 2.1, equation (3): the product is taken in token order,
    each new factor multiplied on the right (the proof there appends
    [E - beta_t k_t k_t^T] on the right of the product of the first t-1).
    K is t x d (rows k_tau)."""
    K, beta = _f64(K), _f64(beta)
    d = K.shape[1]
    P = np.eye(d)
    for tau in range(K.shape[0]):
        k = K[tau]
        P = P @ (np.eye(d) - beta[tau] * np.outer(k, k))
    return P


def w_recursion(K, beta):
    """Rows w_t of W from the first page, section 2.1, the construction that
    closes the proof of equation (3):
        w_t = beta_t k_t - beta_t sum_{tau < t} (k_tau^T k_t) w_tau .
    Then prod_tau (E - beta_tau k_tau k_tau^T) = E - W^T K."""
    K, beta = _f64(K), _f64(beta)
    t, d = K.shape
    W = np.zeros((t, d))
    for n in range(t):
        acc = beta[n] * K[n]
        for tau in range(n):
            acc = acc - beta[n] * (K[tau] @ K[n]) * W[tau]
        W[n] = acc
    return W


def u_recursion(K, V, beta, eta):
    """Rows u_t of U from the first page, section 3.1, the construction that
    closes the proof of the state-parallel theorem:
        u_t = eta_t v_t - beta_t sum_{tau < t} (k_tau^T k_t) u_tau ,
    so that sum_tau eta_tau v_tau k_tau^T prod_{i > tau} H_i = U^T K."""
    K, V, beta, eta = _f64(K), _f64(V), _f64(beta), _f64(eta)
    t = K.shape[0]
    U = np.zeros((t, V.shape[1]))
    for n in range(t):
        acc = eta[n] * V[n]
        for tau in range(n):
            acc = acc - beta[n] * (K[tau] @ K[n]) * U[tau]
        U[n] = acc
    return U


def strict_lower_A(K, beta):
    """First page, section 2.2: A strictly lower, A_ij = -beta_i (k_j^T k_i)
    for i > j, zero elsewhere, so that W = B + A W with B = diag(beta) K."""
    K, beta = _f64(K), _f64(beta)
    t = K.shape[0]
    A = np.zeros((t, t))
    for i in range(t):
        for j in range(i):
            A[i, j] = -beta[i] * (K[j] @ K[i])
    return A


def forward_substitution(A):
    """T = (E - A)^{-1} for strictly lower A, first page, section 2.3.1:
    column by column, T[i,j] = 0 (i < j), 1 (i = j) and
    T[i,j] = sum_{k=j}^{i-1} A[i,k] T[k,j] (i > j)."""
    A = _f64(A)
    C = A.shape[0]
    T = np.zeros((C, C))
    for j in range(C):
        T[j, j] = 1.0
        for i in range(j + 1, C):
            s = 0.0
            for k in range(j, i):
                s += A[i, k] * T[k, j]
            T[i, j] = s
    return T


def gated_chunk_matrices(K, V, alpha, beta, eta=None):
    """Chunk-local matrices of "从零开始的 GDN 推导" (UT transform, then the
    summary's first two steps), transposed to the d_v x d_k state.

    gamma_i = prod_{j < i} alpha_j with gamma_0 = 1 (section "推导
    WY-representation"); Gamma = diag(gamma_1 .. gamma_C) (UT transform);
    L = StrictLower(B Gamma K K^T Gamma^{-1}); T = (I + L)^{-1};
    W = T B Gamma K and U = T B V (section "S 的推导").  With a separate
    write strength eta (first page, section 3.2, U = T diag(eta) V) the U
    product uses diag(eta) in place of B.

    Returns dict with gamma (length C+1), Gamma, L, A (= -L), T, W, U."""
    K, V = _f64(K), _f64(V)
    alpha, beta = _f64(alpha), _f64(beta)
    eta = beta if eta is None else _f64(eta)
    C = K.shape[0]
    gamma = np.ones(C + 1)
    for i in range(1, C + 1):
        gamma[i] = gamma[i - 1] * alpha[i - 1]
    Gamma = np.diag(gamma[1:])
    Gamma_inv = np.diag(1.0 / gamma[1:])
    Bm = np.diag(beta)
    L = np.tril(Bm @ Gamma @ K @ K.T @ Gamma_inv, k=-1)
    A = -L
    T = forward_substitution(A)          # (I - A)^{-1} = (I + L)^{-1}
    W = T @ Bm @ Gamma @ K
    U = T @ np.diag(eta) @ V
    return {"gamma": gamma, "Gamma": Gamma, "Gamma_inv": Gamma_inv,
            "L": L, "A": A, "T": T, "W": W, "U": U}


def chunked_forward(q, k, v, alpha, beta, S0=None, chunk_size=64, eta=None):
    """Chunkwise-parallel forward pass of one sequence, following the four
    steps that close "从零开始的 GDN 推导" (A; U and W; S update; O update),
    each chunk's output state feeding the next chunk, transposed to the
    d_v x d_k state:

        S_[c+1] = gamma_C S_[c] + gamma_C (U - W S_[c]^T)^T Gamma^{-1} K
        O_[c]   = Gamma Q S_[c]^T + Gamma Lower(Q K^T) Gamma^{-1} (U - W S_[c]^T)

    Lower keeps the diagonal (token t sees itself).  The last chunk may be
    shorter than chunk_size ("当前 chunk 的长度为 C").
    q, k: [T, dk]; v: [T, dv]; alpha, beta, eta: [T] (alpha None => 1);
    S0: [dv, dk] or None.  Returns (O [T, dv], S_final [dv, dk])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Tlen, dk = k.shape
    dv = v.shape[1]
    alpha = np.ones(Tlen) if alpha is None else _f64(alpha)
    beta = _f64(beta)
    eta = beta if eta is None else _f64(eta)
    S = np.zeros((dv, dk)) if S0 is None else _f64(S0).copy()
    O = np.zeros((Tlen, dv))
    for t0 in range(0, Tlen, chunk_size):
        t1 = min(t0 + chunk_size, Tlen)
        Qc, Kc, Vc = q[t0:t1], k[t0:t1], v[t0:t1]
        m = gated_chunk_matrices(Kc, Vc, alpha[t0:t1], beta[t0:t1], eta[t0:t1])
        gC = m["gamma"][-1]
        Gam, Gam_inv = m["Gamma"], m["Gamma_inv"]
        Vp = m["U"] - m["W"] @ S.T                      # U - W S^T
        O[t0:t1] = Gam @ Qc @ S.T + Gam @ np.tril(Qc @ Kc.T) @ Gam_inv @ Vp
        S = gC * S + gC * (Vp.T @ Gam_inv @ Kc)
    return O, S
