"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, run the fp64 oracle on the same seeded inputs, compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import gated_delta_rule_13_amd as gdn

# Tolerances: max relative error, normwise per tensor
#   max_i |x_i - x_ref_i| / max_i |x_ref_i|
# bf16 inputs with fp32 state: 2e-3; all-fp32: 1e-5.
TOL = {"bf16": 2e-3, "f32": 1e-5}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: dict, device="cuda") -> dict:
    out = {}
    for key in ("q", "k", "v", "alpha", "beta", "S0"):
        t = x.get(key)
        out[key] = None if t is None else t.to(device)
    return out


def nan_outputs(x: dict, o_dtype=torch.float32, device="cuda"):
    """O and S_final buffers pre-filled with NaN: an element the kernel never
    writes stays NaN and fails the finiteness check."""
    B, H, T, dk = x["q"].shape
    dv = x["v"].shape[-1]
    O = torch.full((B, H, T, dv), float("nan"), dtype=o_dtype, device=device)
    S = torch.full((B, H, dv, dk), float("nan"), dtype=torch.float32, device=device)
    return O, S


def run_gpu(x: dict, chunk: int, o_dtype=torch.float32, S0=None, **kw):
    d = to_dev(x)
    s0 = d["S0"] if S0 is None else S0
    if "O" not in kw and "S_final" not in kw:
        kw["O"], kw["S_final"] = nan_outputs(x, o_dtype)
    O, S = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], s0,
                             chunk_size=chunk, o_dtype=o_dtype, **kw)
    torch.cuda.synchronize()
    return O, S


def run_oracle(x: dict, heads=None):
    """fp64 oracle on all heads, or on a list of (b, h) pairs."""
    sel = lambda t: None if t is None else t
    if heads is None:
        return oracle.recurrent(x["q"], x["k"], x["v"], sel(x["alpha"]), x["beta"], S0=x["S0"])
    Os, Ss = [], []
    for b, h in heads:
        pick = lambda t: None if t is None else t[b:b + 1, h:h + 1]
        O, S = oracle.recurrent(pick(x["q"]), pick(x["k"]), pick(x["v"]), pick(x["alpha"]),
                                pick(x["beta"]), S0=pick(x["S0"]))
        Os.append(O[0, 0])
        Ss.append(S[0, 0])
    return np.stack(Os), np.stack(Ss)


def rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.abs(ref).max()
    if denom == 0:
        return float(np.abs(x).max())
    return float(np.abs(x - ref).max() / denom)


def elem_err(x, ref) -> float:
    """Elementwise diagnostic (reported, not gated): max_i |x_i - ref_i| /
    max(|ref_i|, 1e-3 max_j |ref_j|)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    floor = 1e-3 * np.abs(ref).max()
    if floor == 0:
        return float(np.abs(x).max())
    return float((np.abs(x - ref) / np.maximum(np.abs(ref), floor)).max())


def gpu_heads(t: torch.Tensor, heads):
    t = t.detach().float().cpu().numpy()
    return np.stack([t[b, h] for b, h in heads])
