"""C ABI of libgdn.so on the CPU: it loads, exports every function that
include/gdn.h declares, and rejects bad arguments before any launch.  No
compute call is made (every call here fails validation)."""
import ctypes
import os
import re
import subprocess

import pytest

import gated_delta_rule_13_amd as gdn
from gated_delta_rule_13_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def lib():
    # the sanitizer test runs this file against an instrumented build of the
    # same sources, named by GDN_TEST_LIB
    override = os.environ.get("GDN_TEST_LIB")
    if override:
        _lib.LIB_PATH = override
        _lib._lib = None
    elif not os.path.exists(_lib.LIB_PATH):
        from gated_delta_rule_13_amd.build import build
        build()
    return _lib.load()


@pytest.fixture
def lib_nogpu(lib):
    """The library, for calls with fake device pointers: every such call
    must fail validation before any launch.  Where a GPU is visible they are
    skipped, so that a validation regression can never launch a kernel on
    those addresses."""
    try:
        import torch
        visible = torch.cuda.device_count() > 0
    except Exception:
        visible = False
    if visible:
        pytest.skip("calls with fake device pointers run only where no GPU is visible")
    return lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_what_binding_expects():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gdn_[a-z_0-9]+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def shape(**kw):
    base = dict(B=1, H=2, T=100, d_k=128, d_v=128, chunk_size=64, qkv_dtype=0, o_dtype=1)
    base.update(kw)
    return _lib.GdnShape(**base)


FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first


def fwd(lib, s, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, alpha=None, beta=FAKE, S0=None, O=FAKE, S=FAKE)
    p.update(ptrs)
    sp = ctypes.byref(s) if s is not None else None
    return lib.gdn_chunk_fwd(sp, p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["S0"],
                             p["O"], p["S"], None, 0, None)


@pytest.mark.parametrize("kw,expected", [
    (dict(B=0), 2), (dict(H=-1), 2), (dict(T=0), 2), (dict(d_k=0), 2),
    (dict(qkv_dtype=7), 3), (dict(o_dtype=-1), 3),
    (dict(chunk_size=48), 4), (dict(d_k=512), 4), (dict(d_k=80), 4), (dict(d_k=8), 4),
    (dict(d_k=48), 4),
    (dict(d_v=40), 4), (dict(d_v=2048), 4), (dict(qkv_dtype=1, d_k=192), 4),
    (dict(qkv_dtype=1, d_k=96), 4), (dict(d_k=16, chunk_size=8), 4),
    (dict(T=5_000_000), 4),
])
def test_bad_shapes_rejected(lib_nogpu, kw, expected):
    lib = lib_nogpu
    # a mismatched q pointer (odd address) could never reach a launch either
    assert fwd(lib, shape(**kw), q=ctypes.c_void_p(0x10001)) == expected
    assert lib.gdn_last_error().decode() != ""
    assert lib.gdn_chunk_fwd_workspace_bytes(ctypes.byref(shape(**kw))) == ctypes.c_size_t(-1).value


def test_null_arguments_rejected(lib_nogpu):
    lib = lib_nogpu
    assert fwd(lib, None) == 1
    for name in ("q", "k", "v", "beta", "O", "S"):
        assert fwd(lib, shape(), **{name: None}) == 1, name


def test_misaligned_pointers_rejected(lib_nogpu):
    lib = lib_nogpu
    for name in ("q", "k", "v", "beta", "O", "S", "alpha", "S0"):
        assert fwd(lib, shape(), **{name: ctypes.c_void_p(0x10004)}) == 4, name


def test_prep_validation(lib_nogpu):
    lib = lib_nogpu
    s = shape()
    assert lib.gdn_chunk_prep(None, FAKE, FAKE, None, FAKE, None, None, None, None, 0, None) == 1
    assert lib.gdn_chunk_prep(ctypes.byref(shape(B=0)), FAKE, FAKE, None, FAKE, FAKE, None, None,
                              None, 0, None) == 2
    assert lib.gdn_chunk_prep(ctypes.byref(s), None, FAKE, None, FAKE, FAKE, None, None,
                              None, 0, None) == 1
    # nothing requested: no launch, OK
    assert lib.gdn_chunk_prep(ctypes.byref(s), FAKE, FAKE, None, FAKE, None, None, None,
                              None, 0, None) == 0


def test_new_entries_validate(lib_nogpu):
    """gdn_chunk_fwd_precise and gdn_chunk_fwd_stages reject before any launch."""
    lib = lib_nogpu
    sp = ctypes.byref(shape())
    odd = ctypes.c_void_p(0x10001)
    assert lib.gdn_chunk_fwd_precise(None, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, FAKE,
                                     None) == 1
    assert lib.gdn_chunk_fwd_precise(sp, odd, FAKE, FAKE, None, FAKE, None, None, FAKE, FAKE,
                                     None) == 4
    # bf16 chunk 16 has no split-bf16 kernel
    s16 = ctypes.byref(shape(chunk_size=16))
    assert lib.gdn_chunk_fwd_precise(s16, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, FAKE,
                                     None) == 4
    assert lib.gdn_chunk_fwd_stages(sp, None, FAKE, FAKE, None, FAKE, None, None, FAKE, FAKE,
                                    None, None, None) == 1
    assert lib.gdn_chunk_fwd_stages(sp, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, FAKE,
                                    ctypes.c_void_p(0x10004), None, None) == 4
    f32 = ctypes.byref(shape(qkv_dtype=1, d_k=64))
    assert lib.gdn_chunk_fwd_stages(f32, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, FAKE,
                                    None, None, None) == 4
    # d_k 256 at chunk 64 runs as 32-token chunks: no per-chunk T of 64 to give
    d256 = ctypes.byref(shape(d_k=256))
    assert lib.gdn_chunk_fwd_stages(d256, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, FAKE,
                                    None, None, None) == 4



def test_workspace_query_and_strings(lib):
    for kw in (dict(), dict(qkv_dtype=1, d_k=16, d_v=16, chunk_size=16),
               dict(chunk_size=32), dict(d_v=256), dict(chunk_size=16), dict(d_k=96, d_v=192),
               dict(qkv_dtype=1, d_k=128), dict(qkv_dtype=1, d_k=256, chunk_size=32),
               dict(d_k=256), dict(qkv_dtype=1, d_k=256)):
        assert lib.gdn_chunk_fwd_workspace_bytes(ctypes.byref(shape(**kw))) == 0
    for code in range(7):
        assert lib.gdn_status_string(code).decode()
    assert lib.gdn_version() >= 200


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 16)
    b = torch.zeros(1, 1, 4)
    with pytest.raises(ValueError, match="GPU"):
        gdn.gdn_chunk_fwd(x, x, x, None, b)


def rec(lib, s, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, alpha=None, beta=FAKE, S0=None, O=FAKE, S=FAKE)
    p.update(ptrs)
    sp = ctypes.byref(s) if s is not None else None
    return lib.gdn_recurrent_fwd(sp, p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["S0"],
                                 p["O"], p["S"], None)


@pytest.mark.parametrize("kw,expected", [
    (dict(B=0), 2), (dict(T=0), 2), (dict(d_v=0), 2), (dict(qkv_dtype=5), 3),
    (dict(d_k=48), 4), (dict(d_k=512), 4), (dict(d_v=70000), 4),
])
def test_recurrent_bad_shapes_rejected(lib_nogpu, kw, expected):
    lib = lib_nogpu
    # an odd q pointer as well: even a shape check that wrongly passed could
    # not reach a launch
    assert rec(lib, shape(**kw), q=ctypes.c_void_p(0x10001)) == expected
    assert lib.gdn_last_error().decode() != ""


def test_recurrent_null_and_misaligned_rejected(lib_nogpu):
    lib = lib_nogpu
    assert rec(lib, None) == 1
    for name in ("q", "k", "v", "beta", "O", "S"):
        assert rec(lib, shape(), **{name: None}) == 1, name
    for name in ("q", "k", "v", "beta", "O", "S", "alpha", "S0"):
        assert rec(lib, shape(), **{name: ctypes.c_void_p(0x10004)}) == 4, name


def seq(lib, s, seg_chunks, ws=None, ws_bytes=0, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, alpha=None, beta=FAKE, eta=None, S0=None, O=FAKE, S=FAKE)
    p.update(ptrs)
    return lib.gdn_chunk_fwd_seq(ctypes.byref(s), seg_chunks, p["q"], p["k"], p["v"], p["alpha"],
                                 p["beta"], p["eta"], p["S0"], p["O"], p["S"], ws, ws_bytes, None)


def test_seq_entry_validates(lib_nogpu):
    """gdn_chunk_fwd_seq rejects before any launch: a negative segment
    length, segments of fp32 inputs, a missing, short or misaligned
    workspace."""
    lib = lib_nogpu
    big = ctypes.c_size_t(-1).value
    s = shape(T=300)
    assert seq(lib, s, -1) == 2
    assert lib.gdn_chunk_fwd_seq_workspace_bytes(ctypes.byref(s), -1) == big
    assert seq(lib, shape(qkv_dtype=1, T=300), 1) == 4
    need = lib.gdn_chunk_fwd_seq_workspace_bytes(ctypes.byref(s), 1)
    assert need > 0
    assert seq(lib, s, 1) == 5
    assert seq(lib, s, 1, ctypes.c_void_p(0x100000), need - 1) == 5
    assert seq(lib, s, 1, ctypes.c_void_p(0x100010), need) == 4


def test_seq_workspace_layout(lib):
    """Workspace bytes of a forced segmentation follow the layout that
    include/gdn.h states: end states and transitions, carried queries, and
    (bf16 O) zero-state outputs, each region 256-byte aligned."""
    up = lambda n: (n + 255) // 256 * 256
    B, H, T, dk, dv, C, L = 2, 3, 300, 64, 96, 32, 2
    nseg = -(-T // (L * C))
    for o_dtype in (1, 0):
        s = shape(B=B, H=H, T=T, d_k=dk, d_v=dv, chunk_size=C, o_dtype=o_dtype)
        want = up(B * H * nseg * (dv + dk) * dk * 4) + B * H * T * dk * 4
        if o_dtype == 0:
            want = up(want) + B * H * T * dv * 4
        assert lib.gdn_chunk_fwd_seq_workspace_bytes(ctypes.byref(s), L) == want
    # one segment (or fp32 inputs): the plain form, no workspace
    s = shape(T=T)
    assert lib.gdn_chunk_fwd_seq_workspace_bytes(ctypes.byref(s), 5) == 0
    assert lib.gdn_chunk_fwd_seq_workspace_bytes(ctypes.byref(shape(qkv_dtype=1, T=T)), 1) == 0


def test_default_plan_host_logic(lib):
    """The default plan (a 256-CU device when none is present): segments for
    one head over 4096 tokens, none for the main shape or short sequences."""
    ws = lambda **kw: lib.gdn_chunk_fwd_workspace_bytes(ctypes.byref(shape(**kw)))
    assert ws(B=1, H=1, T=4096) > 0
    assert ws(B=2, H=4, T=1024, d_k=64, d_v=64) > 0
    assert ws(B=4, H=16, T=4096) == 0
    assert ws(B=1, H=32, T=32768, d_v=256) == 0
    assert ws(B=1, H=1, T=64) == 0


def test_noalloc_entry_rejects_before_launch(lib_nogpu):
    """gdn_chunk_fwd_seq_noalloc checks its scratch limit (64 MiB) on the
    host: a plan that needs more returns GDN_ERR_WORKSPACE, a negative
    segment length GDN_ERR_BAD_SHAPE, a bad shape its own error."""
    lib = lib_nogpu
    def call(s, seg):
        return lib.gdn_chunk_fwd_seq_noalloc(ctypes.byref(s), seg, FAKE, FAKE, FAKE, None, FAKE,
                                             None, None, FAKE, FAKE, None)
    big = shape(B=1, H=1, T=200000, d_k=128, d_v=128)
    assert lib.gdn_chunk_fwd_seq_workspace_bytes(ctypes.byref(big), 1) > 64 << 20
    assert call(big, 1) == 5
    assert "64 MiB" in lib.gdn_last_error().decode()
    assert call(shape(), -1) == 2
    assert call(shape(B=0), 0) == 2
    assert call(shape(d_k=48), 0) == 4
