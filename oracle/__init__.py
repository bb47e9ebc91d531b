"""fp64 CPU oracle of the gated delta rule forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares
no code with the GPU library and never imports it; the GPU library never
imports it either.

* :func:`recurrent` -- the plain token-by-token recurrence (C, fp64, OpenMP
  over the independent (b, h) sequences).  This is the parity reference.
* :mod:`oracle.chunked_ref` -- fp64 numpy forms of the WY / UT algebra and of
  the chunkwise pass, kept literal to the pages, used to pin the recurrence
  (recurrent == chunked) and to check intermediate quantities.

Inputs are numpy arrays; they are converted to contiguous float64 (an exact
up-cast from bf16 or fp32).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import build_oracle, library_path

_LIBS: dict = {}


def load(path: str | None = None):
    """Load (building if needed) the oracle library; cached per path."""
    path = path or library_path()
    lib = _LIBS.get(path)
    if lib is not None:
        return lib
    if not os.path.exists(path):
        if path == library_path():
            build_oracle()
        else:
            raise FileNotFoundError(path)
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.gdn_oracle_recurrent_f64.argtypes = [i64, i64, i64, i64, i64,
                                             dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                             ctypes.c_int]
    lib.gdn_oracle_recurrent_f64.restype = ctypes.c_int
    lib.gdn_oracle_max_threads.restype = ctypes.c_int
    _LIBS[path] = lib
    return lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # a CPU torch tensor
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return ctypes.POINTER(ctypes.c_double)()
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrent(q, k, v, alpha, beta, S0=None, eta=None, nthreads: int = 0, lib=None):
    """fp64 recurrence.  Shapes: q, k [B,H,T,dk]; v [B,H,T,dv];
    alpha, beta, eta [B,H,T] (alpha None => 1, eta None => beta);
    S0 [B,H,dv,dk] or None (zero).  Returns (O [B,H,T,dv], S_final [B,H,dv,dk])."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, beta, eta, S0 = _f64(alpha), _f64(beta), _f64(eta), _f64(S0)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if k.shape != (B, H, T, dk) or v.shape != (B, H, T, dv):
        raise ValueError("q, k, v shapes disagree")
    for name, a in (("alpha", alpha), ("beta", beta), ("eta", eta)):
        if a is not None and a.shape != (B, H, T):
            raise ValueError(f"{name} must have shape {(B, H, T)}")
    if S0 is not None and S0.shape != (B, H, dv, dk):
        raise ValueError("S0 must have shape [B,H,dv,dk]")
    O = np.empty((B, H, T, dv), dtype=np.float64)
    S = np.empty((B, H, dv, dk), dtype=np.float64)
    rc = lib.gdn_oracle_recurrent_f64(B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(alpha), _ptr(beta), _ptr(eta), _ptr(S0),
                                      _ptr(O), _ptr(S), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle returned {rc}")
    return O, S


def max_threads(lib=None) -> int:
    return (lib or load()).gdn_oracle_max_threads()
