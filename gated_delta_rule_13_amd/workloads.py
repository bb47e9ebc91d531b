"""Seeded synthetic inputs for the gated delta rule forward pass.

This module holds input generation only -- none of the method's arithmetic --
so that the GPU path and the CPU oracle can both be fed from it without
sharing any code with each other.

Seven workloads, named by what they are.  All draws come from one CPU
``torch.Generator`` seeded with ``seed``, in the fixed order
q, k, v, S0, beta source, alpha source, reflection mask; each is drawn in
float32 with the full shape.  q and k are L2-normalised per row in float32
and then rounded to the workload's dtype (round-to-nearest-even); the
rounded tensors are what both sides consume.

=============  ==========================================  ======  ============================
name           shape (B, H, T, d_k, d_v, chunk)            dtype   gates / state
=============  ==========================================  ======  ============================
tiny           1, 1, 64, 16, 16, 16                        f32     beta = sigmoid(N), alpha = exp(-softplus(N) * 0.1), S0 = 0
deltanet       2, 4, 1024, 64, 64, 64                      bf16    beta = sigmoid(N), alpha = 1, S0 = 0.02 N
main           4, 16, 4096, 128, 128, 64                   bf16    beta = sigmoid(N), alpha = exp(-softplus(N) * 0.05), S0 = 0
long           1, 32, 32768, 128, 256, 64                  bf16    beta = sigmoid(N), alpha = exp(-softplus(N) * 0.01), S0 = 0.02 N
many_short     64, 8, 512, 128, 128, 32                    bf16    beta ~ U(0,1), alpha ~ U(0.9,1); 1% of tokens (Bernoulli per token)
                                                                   are reflections: beta = 2 / (k^T k), alpha = 1; S0 = 0
decode         64, 16, 1, 128, 128, -                      bf16    beta = sigmoid(N), alpha = exp(-softplus(N) * 0.05),
                                                                   S0 = 0.02 N: one decode step of the recurrent form
olmo_hybrid    2, 30, 4096, 96, 192, 64                    bf16    beta = 2 sigmoid(N) (erase strength in (0, 2)),
                                                                   alpha = exp(-softplus(N) * 0.05), S0 = 0
=============  ==========================================  ======  ============================

v ~ N(0, 1) everywhere.  Alpha of exactly one is passed as ``None`` (the
API's "no gate"); a zero S0 is passed as ``None``.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_random", "chunk_scaled_alpha",
           "algorithmic_bytes", "algorithmic_flops"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    dtype: str                 # "bf16" or "f32": dtype of q, k, v
    beta_kind: str = "sigmoid"  # "sigmoid" | "sigmoid2" (2 sigmoid) | "uniform"
    alpha_kind: str = "softplus"  # "softplus" | "one" | "uniform"
    alpha_scale: float = 0.0   # s in exp(-softplus(N) * s)
    s0_std: float = 0.0        # 0 => S0 = None
    reflection_rate: float = 0.0

    def with_shape(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def head_tokens(self) -> int:
        return self.B * self.H * self.T


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 64, 16, 16, 16, "f32", alpha_scale=0.1),
    "deltanet": Workload("deltanet", 2, 4, 1024, 64, 64, 64, "bf16", alpha_kind="one",
                         s0_std=0.02),
    "main": Workload("main", 4, 16, 4096, 128, 128, 64, "bf16", alpha_scale=0.05),
    "long": Workload("long", 1, 32, 32768, 128, 256, 64, "bf16", alpha_scale=0.01,
                     s0_std=0.02),
    "many_short": Workload("many_short", 64, 8, 512, 128, 128, 32, "bf16",
                           beta_kind="uniform", alpha_kind="uniform", reflection_rate=0.01),
    # one token per sequence against a resident state (recurrent form; the
    # chunk field is unused there)
    "decode": Workload("decode", 64, 16, 1, 128, 128, 64, "bf16", alpha_scale=0.05,
                       s0_std=0.02),
    # the head shape of the Olmo Hybrid models' gated delta rule layers (30
    # heads, q/k dimension 96, v dimension 192, erase strength 2 beta)
    "olmo_hybrid": Workload("olmo_hybrid", 2, 30, 4096, 96, 192, 64, "bf16",
                            beta_kind="sigmoid2", alpha_scale=0.05),
}

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """CPU tensors for workload ``w``: q, k, v (w.dtype), alpha (f32 or None),
    beta (f32), S0 (f32 or None), reflection_mask (bool or None)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    dt = _TORCH_DTYPE[w.dtype]
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    q = _unit_rows(torch.randn(B, H, T, dk, generator=g)).to(dt)
    k = _unit_rows(torch.randn(B, H, T, dk, generator=g)).to(dt)
    v = torch.randn(B, H, T, dv, generator=g).to(dt)
    S0 = None
    if w.s0_std > 0:
        S0 = w.s0_std * torch.randn(B, H, dv, dk, generator=g)
    if w.beta_kind == "sigmoid":
        beta = torch.sigmoid(torch.randn(B, H, T, generator=g))
    elif w.beta_kind == "sigmoid2":
        beta = 2.0 * torch.sigmoid(torch.randn(B, H, T, generator=g))
    elif w.beta_kind == "uniform":
        beta = torch.rand(B, H, T, generator=g)
    else:
        raise ValueError(w.beta_kind)
    if w.alpha_kind == "one":
        alpha = None
    elif w.alpha_kind == "softplus":
        alpha = torch.exp(-torch.nn.functional.softplus(torch.randn(B, H, T, generator=g))
                          * w.alpha_scale)
    elif w.alpha_kind == "uniform":
        alpha = 0.9 + 0.1 * torch.rand(B, H, T, generator=g)
    else:
        raise ValueError(w.alpha_kind)
    mask = None
    if w.reflection_rate > 0:
        mask = torch.rand(B, H, T, generator=g) < w.reflection_rate
        # reflection tokens: beta = 2 / (k^T k) of the rounded k, in fp32; no decay
        kk = (k.float() * k.float()).sum(-1)
        beta = torch.where(mask, 2.0 / kk, beta)
        if alpha is not None:
            alpha = torch.where(mask, torch.ones_like(alpha), alpha)
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(),
            "alpha": None if alpha is None else alpha.float().contiguous(),
            "beta": beta.float().contiguous(),
            "S0": None if S0 is None else S0.float().contiguous(),
            "reflection_mask": mask, "chunk": w.chunk, "workload": w}


def make_random(B, H, T, dk, dv, dtype="bf16", chunk=64, seed=0, alpha_scale=0.05,
                s0_std=0.0, beta_kind="sigmoid", alpha_kind="softplus") -> dict:
    """Inputs of the same distributions at an arbitrary shape (for parity
    cases at sizes the oracle finishes quickly)."""
    w = Workload("custom", B, H, T, dk, dv, chunk, dtype, beta_kind=beta_kind,
                 alpha_kind=alpha_kind, alpha_scale=alpha_scale, s0_std=s0_std)
    return make_inputs(w, seed)


def chunk_scaled_alpha(B, H, T, chunk, scales, seed=0) -> torch.Tensor:
    """Gates alpha = exp(-softplus(N(0,1)) * s) whose scale s changes from
    chunk to chunk, cycling through ``scales`` (chunk c of every sequence
    uses scales[c % len(scales)]).  Large scales give strong gates (alpha
    near 0.04 at s = 4), so that one chunk's decay spans hundreds of binary
    orders of magnitude; mixing scales puts weakly and strongly gated chunks
    side by side in one sequence."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    n = torch.randn(B, H, T, generator=g)
    idx = (torch.arange(T) // chunk) % len(scales)
    s = torch.tensor([float(v) for v in scales])[idx]
    return torch.exp(-torch.nn.functional.softplus(n) * s).float().contiguous()


def algorithmic_bytes(w: Workload, o_bytes: int = 4, with_alpha: bool | None = None,
                      with_s0: bool | None = None) -> int:
    """Bytes the method must move at least once: read q, k, v, alpha, beta
    (and S0 if given), write O and S_final."""
    s_in = 2 if w.dtype == "bf16" else 4
    a = (w.alpha_kind != "one") if with_alpha is None else with_alpha
    s0 = (w.s0_std > 0) if with_s0 is None else with_s0
    per_tok = (2 * w.dk + w.dv) * s_in + 4 * (1 + int(a)) + w.dv * o_bytes
    state = w.B * w.H * w.dk * w.dv * 4 * (1 + int(s0))
    return w.head_tokens * per_tok + state


def algorithmic_flops(w: Workload) -> int:
    """Flops of the chunked method as the pages state it, at full chunk
    tiles, per head-token: the three state-side products 6 d_k d_v
    (W S^T, Q S^T, the state update), the C x d_k products 6 C d_k
    (Gram K K^T, scores Q K^T, W = T B Gamma K), the C x d_v products
    4 C d_v (U = T B V, scores times pseudo-values) and the triangular
    solve C^2 / 3."""
    C = w.chunk
    per = 6 * w.dk * w.dv + 6 * C * w.dk + 4 * C * w.dv + (C * C) // 3
    return w.head_tokens * per
