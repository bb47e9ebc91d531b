"""ctypes view of ``libgdn.so`` (declarations mirror ``include/gdn.h``)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")

GDN_BF16 = 0
GDN_F32 = 1

STATUS = {
    0: "GDN_OK",
    1: "GDN_ERR_NULL_ARG",
    2: "GDN_ERR_BAD_SHAPE",
    3: "GDN_ERR_BAD_DTYPE",
    4: "GDN_ERR_UNSUPPORTED",
    5: "GDN_ERR_WORKSPACE",
    6: "GDN_ERR_HIP",
}

# Every symbol include/gdn.h declares.
EXPORTS = ("gdn_chunk_fwd_workspace_bytes", "gdn_chunk_fwd", "gdn_chunk_fwd_eta",
           "gdn_chunk_fwd_seq_workspace_bytes", "gdn_chunk_fwd_seq", "gdn_chunk_fwd_seq_noalloc",
           "gdn_chunk_fwd_precise", "gdn_chunk_fwd_stages",
           "gdn_chunk_prep", "gdn_recurrent_fwd", "gdn_recurrent_fwd_eta",
           "gdn_status_string", "gdn_last_error", "gdn_version")


class GdnShape(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in
                ("B", "H", "T", "d_k", "d_v", "chunk_size", "qkv_dtype", "o_dtype")]


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {message}")


_lib = None


def load():
    """Load the built library; fails loudly when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m gated_delta_rule_13_amd.build` "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sp = ctypes.c_void_p, ctypes.POINTER(GdnShape)
    lib.gdn_chunk_fwd_workspace_bytes.argtypes = [sp]
    lib.gdn_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_chunk_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.gdn_chunk_fwd.restype = ctypes.c_int
    lib.gdn_chunk_prep.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.gdn_chunk_prep.restype = ctypes.c_int
    lib.gdn_recurrent_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_recurrent_fwd.restype = ctypes.c_int
    lib.gdn_chunk_fwd_eta.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.gdn_chunk_fwd_eta.restype = ctypes.c_int
    lib.gdn_chunk_fwd_seq_workspace_bytes.argtypes = [sp, ctypes.c_int]
    lib.gdn_chunk_fwd_seq_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_chunk_fwd_seq.argtypes = [sp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      ctypes.c_size_t, vp]
    lib.gdn_chunk_fwd_seq.restype = ctypes.c_int
    lib.gdn_chunk_fwd_seq_noalloc.argtypes = [sp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp,
                                              vp, vp]
    lib.gdn_chunk_fwd_seq_noalloc.restype = ctypes.c_int
    lib.gdn_chunk_fwd_precise.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_chunk_fwd_precise.restype = ctypes.c_int
    lib.gdn_chunk_fwd_stages.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_chunk_fwd_stages.restype = ctypes.c_int
    lib.gdn_recurrent_fwd_eta.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_recurrent_fwd_eta.restype = ctypes.c_int
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_version.argtypes = []
    lib.gdn_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def check(status: int):
    if status != 0:
        lib = load()
        raise GdnError(status, lib.gdn_last_error().decode() or
                       lib.gdn_status_string(status).decode())
