"""MI355X (gfx950) chunkwise-parallel gated delta rule forward pass.

Thin Python binding over the C ABI of ``include/gdn.h``: same names, argument
marshalling only -- every step of the computation runs in the HIP kernels of
``libgdn.so``.  PyTorch supplies device memory and the current stream.

    O, S_final = gdn_chunk_fwd(q, k, v, alpha, beta, S0=None, chunk_size=64)

computes, for every (b, h) sequence and with S of shape [d_v, d_k],
    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t.
"""
from __future__ import annotations

import ctypes

from ._lib import (EXPORTS, GDN_BF16, GDN_F32, GdnError, GdnShape, check, load)

__all__ = ["gdn_chunk_fwd", "gdn_chunk_fwd_eta", "gdn_chunk_fwd_precise", "gdn_chunk_fwd_stages",
           "gdn_chunk_fwd_seq", "gdn_chunk_fwd_seq_workspace_bytes", "gdn_chunk_fwd_seq_noalloc",
           "gdn_chunk_prep", "gdn_chunk_fwd_workspace_bytes",
           "gdn_recurrent_fwd", "gdn_recurrent_fwd_eta",
           "gdn_status_string", "gdn_last_error", "gdn_version", "GdnError", "GdnShape",
           "EXPORTS"]


def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.bfloat16:
        return GDN_BF16
    if dt == torch.float32:
        return GDN_F32
    raise TypeError(f"unsupported dtype {dt}; use torch.bfloat16 or torch.float32")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _check_tensor(name, t, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(device, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def make_shape(B, H, T, d_k, d_v, chunk_size, qkv_dtype, o_dtype=None) -> GdnShape:
    torch = _torch()
    o_dtype = torch.float32 if o_dtype is None else o_dtype
    return GdnShape(B, H, T, d_k, d_v, chunk_size, _dtype_code(qkv_dtype), _dtype_code(o_dtype))


def gdn_chunk_fwd_workspace_bytes(shape: GdnShape) -> int:
    n = load().gdn_chunk_fwd_workspace_bytes(ctypes.byref(shape))
    if n == ctypes.c_size_t(-1).value:
        raise GdnError(4, load().gdn_last_error().decode())
    return int(n)


def gdn_chunk_fwd_seq_workspace_bytes(shape: GdnShape, seg_chunks: int) -> int:
    n = load().gdn_chunk_fwd_seq_workspace_bytes(ctypes.byref(shape), int(seg_chunks))
    if n == ctypes.c_size_t(-1).value:
        raise GdnError(4, load().gdn_last_error().decode())
    return int(n)


def _workspace(nbytes, dev):
    """Device workspace of nbytes (256-byte aligned), or None."""
    if not nbytes:
        return None
    torch = _torch()
    return torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)


def _ws_ptr(ws) -> int | None:
    if ws is None:
        return None
    return (ws.data_ptr() + 255) // 256 * 256


def _chunk_call(entry, q, k, v, alpha, beta, S0, chunk_size, o_dtype, O, S_final, stream, eta,
                extra=()):
    torch = _torch()
    lib = load()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn_chunk_fwd runs on the GPU: tensors must be on a cuda device")
    o_dtype = torch.float32 if o_dtype is None else o_dtype
    _check_tensor("q", q, (B, H, T, dk), q.dtype, dev)
    _check_tensor("k", k, (B, H, T, dk), q.dtype, dev)
    _check_tensor("v", v, (B, H, T, dv), q.dtype, dev)
    _check_tensor("alpha", alpha, (B, H, T), torch.float32, dev)
    _check_tensor("beta", beta, (B, H, T), torch.float32, dev)
    _check_tensor("eta", eta, (B, H, T), torch.float32, dev)
    _check_tensor("S0", S0, (B, H, dv, dk), torch.float32, dev)
    if O is None:
        O = torch.empty((B, H, T, dv), dtype=o_dtype, device=dev)
    _check_tensor("O", O, (B, H, T, dv), o_dtype, dev)
    if S_final is None:
        S_final = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    _check_tensor("S_final", S_final, (B, H, dv, dk), torch.float32, dev)
    shape = make_shape(B, H, T, dk, dv, chunk_size, q.dtype, o_dtype)
    hs = _stream_handle(dev, stream)
    if entry == "fast":
        ws_bytes = gdn_chunk_fwd_workspace_bytes(shape)
        ws = _workspace(ws_bytes, dev)
        if eta is None:
            st = lib.gdn_chunk_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                   _ptr(beta), _ptr(S0), _ptr(O), _ptr(S_final), _ws_ptr(ws),
                                   ws_bytes, hs)
        else:
            st = lib.gdn_chunk_fwd_eta(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(alpha), _ptr(beta), _ptr(eta), _ptr(S0), _ptr(O),
                                       _ptr(S_final), _ws_ptr(ws), ws_bytes, hs)
    elif entry == "seq":
        seg_chunks, ws = extra
        ws_bytes = gdn_chunk_fwd_seq_workspace_bytes(shape, seg_chunks)
        if ws is None:
            ws = _workspace(ws_bytes, dev)
        elif ws.numel() < ws_bytes + 256 or ws.dtype != torch.uint8 or ws.device != dev:
            raise ValueError(f"workspace must be a uint8 tensor of at least {ws_bytes + 256} "
                             f"bytes on {dev}")
        st = lib.gdn_chunk_fwd_seq(ctypes.byref(shape), int(seg_chunks), _ptr(q), _ptr(k),
                                   _ptr(v), _ptr(alpha), _ptr(beta), _ptr(eta), _ptr(S0),
                                   _ptr(O), _ptr(S_final), _ws_ptr(ws), ws_bytes, hs)
    elif entry == "noalloc":
        (seg_chunks,) = extra
        st = lib.gdn_chunk_fwd_seq_noalloc(ctypes.byref(shape), int(seg_chunks), _ptr(q), _ptr(k),
                                           _ptr(v), _ptr(alpha), _ptr(beta), _ptr(eta), _ptr(S0),
                                           _ptr(O), _ptr(S_final), hs)
    elif entry == "precise":
        st = lib.gdn_chunk_fwd_precise(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(alpha), _ptr(beta), _ptr(eta), _ptr(S0), _ptr(O),
                                       _ptr(S_final), hs)
    else:
        T_out, Vp_out = extra
        st = lib.gdn_chunk_fwd_stages(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(alpha), _ptr(beta), _ptr(eta), _ptr(S0), _ptr(O),
                                      _ptr(S_final), _ptr(T_out), _ptr(Vp_out), hs)
    check(st)
    return O, S_final


def gdn_chunk_fwd(q, k, v, alpha, beta, S0=None, chunk_size: int = 64, o_dtype=None,
                  O=None, S_final=None, stream=None, eta=None):
    """Forward pass on the GPU.  q, k [B,H,T,d_k] and v [B,H,T,d_v] (bf16 or
    fp32, one dtype); alpha (or None = 1), beta [B,H,T] fp32; S0 [B,H,d_v,d_k]
    fp32 or None (zero).  Returns (O [B,H,T,d_v] in o_dtype (fp32 default),
    S_final [B,H,d_v,d_k] fp32).  O / S_final may be passed in (S_final may
    be S0: in-place state update).  Runs on the current stream, asynchronously.
    eta [B,H,T] fp32, if given, is a separate write strength (the C entry
    gdn_chunk_fwd_eta); None means eta = beta.  bf16 inputs take the fp16-
    operand kernel (gdn_chunk_fwd_precise is the split-bf16 alternative)."""
    return _chunk_call("fast", q, k, v, alpha, beta, S0, chunk_size, o_dtype, O, S_final,
                       stream, eta)


def gdn_chunk_fwd_seq(q, k, v, alpha, beta, S0=None, chunk_size: int = 64, seg_chunks: int = 0,
                      o_dtype=None, O=None, S_final=None, stream=None, eta=None, workspace=None):
    """gdn_chunk_fwd with the sequence-parallel form chosen by the caller:
    segments of seg_chunks chunks run at once, then a combine over segments
    and a correction of the later segments' outputs (0: the choice
    gdn_chunk_fwd makes).  workspace: None (allocated here) or a uint8 cuda
    tensor of at least gdn_chunk_fwd_seq_workspace_bytes + 256 bytes; its
    contents after the call are laid out as include/gdn.h states (the data
    starts at the first 256-byte aligned address of the tensor)."""
    return _chunk_call("seq", q, k, v, alpha, beta, S0, chunk_size, o_dtype, O, S_final,
                       stream, eta, extra=(seg_chunks, workspace))


def gdn_chunk_fwd_seq_noalloc(q, k, v, alpha, beta, S0=None, chunk_size: int = 64,
                              seg_chunks: int = 0, o_dtype=None, O=None, S_final=None,
                              stream=None, eta=None):
    """gdn_chunk_fwd_seq with the library's own 64 MiB scratch instead of a
    workspace (the C entry allocates nothing; pass O and S_final to keep the
    whole call free of allocation).  Calls that overlap on one GPU race."""
    return _chunk_call("noalloc", q, k, v, alpha, beta, S0, chunk_size, o_dtype, O, S_final,
                       stream, eta, extra=(seg_chunks,))


def gdn_chunk_fwd_precise(q, k, v, alpha, beta, S0=None, chunk_size: int = 64, o_dtype=None,
                          O=None, S_final=None, stream=None, eta=None):
    """The same pass through the split-bf16 kernels (every derived MFMA
    operand as a bf16 hi + lo pair: errors near 1e-5 whatever the gates)."""
    return _chunk_call("precise", q, k, v, alpha, beta, S0, chunk_size, o_dtype, O, S_final,
                       stream, eta)


def gdn_chunk_fwd_stages(q, k, v, alpha, beta, S0=None, chunk_size: int = 64, o_dtype=None,
                         eta=None, stream=None):
    """The default bf16 pass with its intermediates written out: returns
    (O, S_final, T [B,H,NT,C,C] = (I - A)^{-1} per chunk, V' [B,H,T,d_v] the
    pseudo-values), fp32."""
    torch = _torch()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    nt = (T + chunk_size - 1) // chunk_size
    T_out = torch.zeros((B, H, nt, chunk_size, chunk_size), dtype=torch.float32, device=q.device)
    Vp_out = torch.zeros((B, H, T, dv), dtype=torch.float32, device=q.device)
    O, S = _chunk_call("stages", q, k, v, alpha, beta, S0, chunk_size, o_dtype, None, None,
                       stream, eta, extra=(T_out, Vp_out))
    return O, S, T_out, Vp_out


def gdn_recurrent_fwd(q, k, v, alpha, beta, S0=None, o_dtype=None, O=None, S_final=None,
                      stream=None, eta=None):
    """Token-by-token forward pass on the GPU (short T, e.g. a decode step).
    Same tensors and conventions as gdn_chunk_fwd; S_final may be S0 (the
    state is then updated in place); eta as for gdn_chunk_fwd."""
    torch = _torch()
    lib = load()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn_recurrent_fwd runs on the GPU: tensors must be on a cuda device")
    o_dtype = torch.float32 if o_dtype is None else o_dtype
    _check_tensor("q", q, (B, H, T, dk), q.dtype, dev)
    _check_tensor("k", k, (B, H, T, dk), q.dtype, dev)
    _check_tensor("v", v, (B, H, T, dv), q.dtype, dev)
    _check_tensor("alpha", alpha, (B, H, T), torch.float32, dev)
    _check_tensor("beta", beta, (B, H, T), torch.float32, dev)
    _check_tensor("eta", eta, (B, H, T), torch.float32, dev)
    _check_tensor("S0", S0, (B, H, dv, dk), torch.float32, dev)
    if O is None:
        O = torch.empty((B, H, T, dv), dtype=o_dtype, device=dev)
    _check_tensor("O", O, (B, H, T, dv), o_dtype, dev)
    if S_final is None:
        S_final = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    _check_tensor("S_final", S_final, (B, H, dv, dk), torch.float32, dev)
    shape = make_shape(B, H, T, dk, dv, 1, q.dtype, o_dtype)
    if eta is None:
        st = lib.gdn_recurrent_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                   _ptr(beta), _ptr(S0), _ptr(O), _ptr(S_final),
                                   _stream_handle(dev, stream))
    else:
        st = lib.gdn_recurrent_fwd_eta(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                       _ptr(beta), _ptr(eta), _ptr(S0), _ptr(O), _ptr(S_final),
                                       _stream_handle(dev, stream))
    check(st)
    return O, S_final


def gdn_chunk_fwd_eta(q, k, v, alpha, beta, eta, S0=None, **kw):
    """gdn_chunk_fwd with a separate write strength eta [B,H,T] (None: eta = beta)."""
    return gdn_chunk_fwd(q, k, v, alpha, beta, S0, eta=eta, **kw)


def gdn_recurrent_fwd_eta(q, k, v, alpha, beta, eta, S0=None, **kw):
    """gdn_recurrent_fwd with a separate write strength eta [B,H,T] (None: eta = beta)."""
    return gdn_recurrent_fwd(q, k, v, alpha, beta, S0, eta=eta, **kw)


def gdn_chunk_prep(k, v, alpha, beta, chunk_size: int = 64, want=("T", "W", "U"), stream=None):
    """Chunk-local quantities on the GPU: T [B,H,NT,C,C], W [B,H,T,d_k],
    U [B,H,T,d_v] (fp32), as a dict with the requested keys."""
    torch = _torch()
    lib = load()
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    dev = k.device
    if dev.type != "cuda":
        raise ValueError("gdn_chunk_prep runs on the GPU")
    _check_tensor("v", v, (B, H, T, dv), k.dtype, dev)
    _check_tensor("alpha", alpha, (B, H, T), torch.float32, dev)
    _check_tensor("beta", beta, (B, H, T), torch.float32, dev)
    if not k.is_contiguous():
        raise ValueError("k must be contiguous")
    nt = (T + chunk_size - 1) // chunk_size
    out = {}
    if "T" in want:
        out["T"] = torch.empty((B, H, nt, chunk_size, chunk_size), dtype=torch.float32, device=dev)
    if "W" in want:
        out["W"] = torch.empty((B, H, T, dk), dtype=torch.float32, device=dev)
    if "U" in want:
        out["U"] = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
    shape = make_shape(B, H, T, dk, dv, chunk_size, k.dtype)
    st = lib.gdn_chunk_prep(ctypes.byref(shape), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                            _ptr(out.get("T")), _ptr(out.get("W")), _ptr(out.get("U")),
                            None, 0, _stream_handle(dev, stream))
    check(st)
    return out


def gdn_status_string(status: int) -> str:
    return load().gdn_status_string(status).decode()


def gdn_last_error() -> str:
    return load().gdn_last_error().decode()


def gdn_version() -> int:
    return int(load().gdn_version())
