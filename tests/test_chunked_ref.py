"""The fp64 WY / UT algebra of ``oracle.chunked_ref`` against the pages'
worked example, closed forms and textbook routines (CPU only)."""
import os

import numpy as np
import pytest

from oracle import chunked_ref as cr

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_matrices(path):
    """Parse a golden text fixture: a name line, then rows of numbers."""
    mats, name, rows = {}, None, []
    for line in open(path, encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line[0].isalpha():
            if name:
                mats[name] = np.array(rows, dtype=np.float64)
            name, rows = line, []
        else:
            rows.append([float(x) for x in line.split()])
    if name:
        mats[name] = np.array(rows, dtype=np.float64)
    return mats


def test_forward_substitution_worked_example():
    """First page, section 2.3.1: T for the 4 x 4 example, and section 2.4:
    A^2, A^3 and A^4 = 0 for the same A."""
    m = read_matrices(os.path.join(GOLDEN, "forward_substitution_4x4.txt"))
    A = m["A"]
    assert np.array_equal(cr.forward_substitution(A), m["T"])
    assert np.array_equal(A @ A, m["A2"])
    assert np.array_equal(A @ A @ A, m["A3"])
    assert np.array_equal(A @ A @ A @ A, m["A4"])


def test_forward_substitution_symbolic_entries_random():
    """The printed 4 x 4 polynomials at random real A (T41 with A43 A32 A21)."""
    r = np.random.default_rng(3)
    A = np.tril(r.standard_normal((4, 4)), -1)
    T = cr.forward_substitution(A)
    a = lambda i, j: A[i - 1, j - 1]
    expect = {
        (2, 1): a(2, 1), (3, 1): a(3, 1) + a(3, 2) * a(2, 1), (3, 2): a(3, 2),
        (4, 1): a(4, 1) + a(4, 2) * a(2, 1) + a(4, 3) * a(3, 1) + a(4, 3) * a(3, 2) * a(2, 1),
        (4, 2): a(4, 2) + a(4, 3) * a(3, 2), (4, 3): a(4, 3),
    }
    for (i, j), val in expect.items():
        assert abs(T[i - 1, j - 1] - val) < 1e-14
    assert np.array_equal(np.diag(T), np.ones(4)) and np.all(np.triu(T, 1) == 0)


@pytest.mark.parametrize("C", [4, 16, 64])
def test_forward_substitution_matches_neumann_and_inverse(C):
    """Strictly lower A is nilpotent (A^C = 0), so the Neumann series of the
    first page, section 2.3.2, is exact after C terms; both equal the textbook
    inverse of (E - A)."""
    r = np.random.default_rng(C)
    A = np.tril(r.uniform(-0.3, 0.3, (C, C)), -1)
    T = cr.forward_substitution(A)
    neumann, P = np.eye(C), np.eye(C)
    for _ in range(1, C):
        P = P @ A
        neumann += P
    assert np.abs(P @ A).max() == 0.0
    inv = np.linalg.inv(np.eye(C) - A)
    assert np.abs(T - neumann).max() < 1e-13
    assert np.abs(T - inv).max() < 1e-12
    assert np.abs((np.eye(C) - A) @ T - np.eye(C)).max() < 1e-13


@pytest.mark.parametrize("t,d", [(1, 3), (4, 4), (8, 8), (7, 3)])
def test_wy_product_identity(t, d):
    """First page, section 2.1, equation (3): prod (E - beta k k^T) = E - W^T K
    with w_t from the recursion, for beta in (0, 2); and section 2.2's matrix
    form W = (E - A)^{-1} diag(beta) K."""
    r = np.random.default_rng(10 * t + d)
    K = r.standard_normal((t, d))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    beta = r.uniform(0.0, 2.0, t)
    P = cr.householder_like_product(K, beta)
    W = cr.w_recursion(K, beta)
    scale = max(1.0, np.abs(P).max())
    assert np.abs(P - (np.eye(d) - W.T @ K)).max() < 1e-13 * scale
    T = cr.forward_substitution(cr.strict_lower_A(K, beta))
    assert np.abs(W - T @ np.diag(beta) @ K).max() < 1e-13 * max(1.0, np.abs(W).max())


def test_w_and_u_expansions_t4():
    """First page, sections 2.4 and 3.3: expansions of w_1..w_4 and u_1..u_4 as
    path sums with edge weights A_ij = -beta_i k_j^T k_i."""
    r = np.random.default_rng(7)
    K = r.standard_normal((4, 5))
    V = r.standard_normal((4, 3))
    beta = r.uniform(0.1, 1.5, 4)
    eta = r.uniform(0.1, 1.5, 4)
    A = cr.strict_lower_A(K, beta)
    a = lambda i, j: A[i - 1, j - 1]
    for X, rows in ((cr.w_recursion(K, beta), beta[:, None] * K),
                    (cr.u_recursion(K, V, beta, eta), eta[:, None] * V)):
        n = lambda i: rows[i - 1]
        expect = [
            n(1),
            n(2) + a(2, 1) * n(1),
            n(3) + a(3, 1) * n(1) + a(3, 2) * n(2) + a(3, 2) * a(2, 1) * n(1),
            n(4) + a(4, 1) * n(1) + a(4, 2) * n(2) + a(4, 3) * n(3)
            + a(4, 2) * a(2, 1) * n(1) + a(4, 3) * a(3, 1) * n(1) + a(4, 3) * a(3, 2) * n(2)
            + a(4, 3) * a(3, 2) * a(2, 1) * n(1),
        ]
        for i in range(4):
            assert np.abs(X[i] - expect[i]).max() < 1e-13


def test_gated_chunk_matrices_match_y_recursion():
    """"从零开始的 GDN 推导", WY proof: y_n = beta_n x_n - beta_n k_n
    sum_{i<n} (gamma_{n+1} / gamma_{i+1}) k_i^T y_i, solved in matrix form by
    the UT transform Y = (I + L)^{-1} B X.  W is Y with x_i = gamma_{i+1} k_i,
    U is Y with x_i = v_i."""
    r = np.random.default_rng(8)
    C, dk, dv = 12, 6, 5
    K = r.standard_normal((C, dk)) / np.sqrt(dk)
    V = r.standard_normal((C, dv))
    alpha = r.uniform(0.5, 1.0, C)
    beta = r.uniform(0.0, 1.5, C)
    m = cr.gated_chunk_matrices(K, V, alpha, beta)
    gamma = m["gamma"]

    def y_rec(X):
        Y = np.zeros_like(X)
        for n in range(C):
            s = np.zeros(X.shape[1])
            for i in range(n):
                s += (gamma[n + 1] / gamma[i + 1]) * (K[n] @ K[i]) * Y[i]
            Y[n] = beta[n] * X[n] - beta[n] * s
        return Y

    assert np.abs(m["W"] - y_rec(gamma[1:, None] * K)).max() < 1e-13
    assert np.abs(m["U"] - y_rec(V)).max() < 1e-13
    assert np.abs(m["T"] - np.linalg.inv(np.eye(C) + m["L"])).max() < 1e-12


def test_chunked_with_unit_gate_matches_state_parallel_form():
    """With alpha = 1 and a single chunk, the chunked state equals the first
    page's S_t = S_0 + (U - W S_0^T)^T K (section 4)."""
    r = np.random.default_rng(9)
    T, dk, dv = 10, 5, 4
    q = r.standard_normal((T, dk))
    K = r.standard_normal((T, dk)) / 2
    V = r.standard_normal((T, dv))
    beta = r.uniform(0, 1, T)
    S0 = r.standard_normal((dv, dk))
    _, S = cr.chunked_forward(q, K, V, None, beta, S0, chunk_size=T)
    W, U = cr.w_recursion(K, beta), cr.u_recursion(K, V, beta, beta)
    assert np.abs(S - (S0 + (U - W @ S0.T).T @ K)).max() < 1e-12
