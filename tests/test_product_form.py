"""The product form of the chunk's triangular inverse, emulated on the CPU:
why the fused kernel solves for T by substitution instead.

"RNN的复兴03:现代RNN的并行计算", section 2.3.2, expands (I - A)^{-1} as a
Neumann series, and section 2.4 notes that the strictly lower triangular A
of a chunk is nilpotent (A^C = 0), so the series is finite and regroups into
log2(C) factors,

    (I - A)^{-1} = sum_{j<C} A^j = (I + A)(I + A^2)(I + A^4) ... (I + A^{C/2}),

a form with only dense products (squarings and multiplications) and no
serial substitution.  This file pins that identity in fp64 against the
oracle's forward substitution, then shows what it does in the precisions a
GPU would use for it (fp32 products, and fp16 operands with fp32 sums as in
the fused kernel's MFMAs):

* on a chunk of one repeated unit key with beta = 2 (every token the same
  Householder reflection) the powers of A grow like 2^j times binomial
  coefficients while T itself only holds entries of magnitude 2, and the
  product form loses everything (error of order one, or overflow);
* row substitution in the same precisions stays accurate there;
* on chunks drawn like the benchmark workloads (unit keys in d_k = 64 / 128,
  beta in (0, 1) or 2 / |k|^2 on reflection tokens, mild gates) both are
  accurate: the product form would only be unsafe, never needed.

Runs on the CPU only.
"""
import numpy as np
import pytest

from oracle import chunked_ref as cr
from gated_delta_rule_13_amd.workloads import WORKLOADS, make_inputs


def product_form(A, dtype=np.float64, f16_operands=False):
    """(I + A)(I + A^2)...(I + A^{C/2}) with every product rounded to
    ``dtype``; with ``f16_operands`` each product's operands are rounded to
    fp16 first (fp32 sums), like an MFMA with fp16 inputs."""
    C = A.shape[0]
    rnd = lambda m: m.astype(np.float16).astype(dtype) if f16_operands else m
    I = np.eye(C, dtype=dtype)
    P = (I + A).astype(dtype)
    Pw = A.astype(dtype)
    j = 1
    while (1 << j) < C:
        with np.errstate(over="ignore", invalid="ignore"):
            Pw = (rnd(Pw) @ rnd(Pw)).astype(dtype)          # A^{2^j}
            P = (rnd(P) @ rnd(I + Pw)).astype(dtype)
        j += 1
    return P


def substitution(A, dtype):
    """Row substitution T = I + T A from the last column down, in ``dtype``
    (the order the fused kernel uses for its diagonal blocks)."""
    C = A.shape[0]
    A = A.astype(dtype)
    T = np.eye(C, dtype=dtype)
    for i in range(C):
        for k in range(i - 1, -1, -1):
            T[i, k] = T[i, k + 1:i + 1] @ A[k + 1:i + 1, k]
    return T


def rel(a, b):
    a = a.astype(np.float64)
    if not np.all(np.isfinite(a)):
        return np.inf
    return float(np.abs(a - b).max() / np.abs(b).max())


def chunk_A(K, alpha, beta):
    return cr.gated_chunk_matrices(K, np.zeros((K.shape[0], 1)), alpha, beta)["A"]


@pytest.mark.parametrize("C", [4, 16, 64])
def test_product_form_is_the_inverse_in_fp64(C):
    rng = np.random.default_rng(C)
    K = rng.standard_normal((C, 32))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    A = chunk_A(K, np.exp(-0.1 * rng.random(C)), rng.random(C))
    T = cr.forward_substitution(A)
    assert np.allclose(product_form(A), T, rtol=0, atol=1e-12)
    assert np.allclose(substitution(A, np.float64), T, rtol=0, atol=1e-12)
    # nilpotent: the last factor's power vanishes
    Ap = np.linalg.matrix_power(A, C)
    assert np.abs(Ap).max() == 0.0


def repeated_reflection(C, dk=128, seed=0):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal(dk)
    k /= np.linalg.norm(k)
    K = np.tile(k, (C, 1))
    return chunk_A(K, np.ones(C), np.full(C, 2.0 / (k @ k)))


def test_repeated_reflection_breaks_the_product_form():
    C = 64
    A = repeated_reflection(C)
    T = cr.forward_substitution(A)
    # T of a repeated reflection alternates +-2 below the diagonal: small
    assert np.abs(T).max() <= 2.0 + 1e-12
    # while the powers the product form squares grow without bound
    assert np.abs(np.linalg.matrix_power(A, 8)).max() > 1e5
    e32 = rel(product_form(A, np.float32), T)
    e16 = rel(product_form(A, np.float32, f16_operands=True), T)
    s32 = rel(substitution(A, np.float32), T)
    print(f"\nrepeated reflection C={C}: product form fp32 {e32:.3g}, fp16 operands {e16:.3g}; "
          f"substitution fp32 {s32:.3g}")
    assert e32 > 0.1 and e16 > 0.1
    assert s32 < 1e-5


@pytest.mark.parametrize("name", ["deltanet", "main", "long", "many_short"])
def test_workload_chunks(name):
    """Both schemes on the first chunks of the workload's own inputs (the
    workload's key, gate and strength distributions; shapes cut to a few
    sequences)."""
    w = WORKLOADS[name].with_shape(B=1, H=2, T=4 * WORKLOADS[name].chunk)
    x = make_inputs(w, seed=0)
    C = w.chunk
    worst_p = worst_s = 0.0
    for h in range(w.H):
        for c in range(w.T // C):
            sl = slice(c * C, (c + 1) * C)
            K = x["k"][0, h, sl].double().numpy()
            a = np.ones(C) if x["alpha"] is None else x["alpha"][0, h, sl].double().numpy()
            A = chunk_A(K, a, x["beta"][0, h, sl].double().numpy())
            T = cr.forward_substitution(A)
            worst_p = max(worst_p, rel(product_form(A, np.float32, f16_operands=True), T))
            worst_s = max(worst_s, rel(substitution(A, np.float32), T))
    print(f"\n{name}: worst chunk, product form (fp16 operands) {worst_p:.3g}, "
          f"substitution fp32 {worst_s:.3g}")
    assert worst_s < 1e-5
    assert worst_p < 5e-3
