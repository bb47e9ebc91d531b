"""gdn_chunk_fwd_seq_noalloc: the sequence-parallel entry with the library's
own scratch array instead of a caller's workspace, for callers that cannot
allocate.  Its outputs must equal those of gdn_chunk_fwd_seq (the same
kernels on the same inputs, with a workspace) on two calls in a row, the
second on a smaller input (the scratch keeps the first call's contents),
and both must stay within the bf16 tolerance of the fp64 oracle."""
import ctypes

import pytest
import torch

import oracle
import gated_delta_rule_13_amd as gdn
from gated_delta_rule_13_amd import _lib
from gated_delta_rule_13_amd.workloads import make_random
from tests.gpu_helpers import TOL, nan_outputs, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def run_both(B, H, T, dk, dv, C, seg, o_dtype, seed):
    x = make_random(B, H, T, dk, dv, dtype="bf16", chunk=C, seed=seed, s0_std=0.02)
    d = to_dev(x)
    lib = _lib.load()
    shape = gdn.make_shape(B, H, T, dk, dv, C, torch.bfloat16, o_dtype)
    sp = ctypes.byref(shape)
    hs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    need = lib.gdn_chunk_fwd_seq_workspace_bytes(sp, seg)
    assert 0 < need <= 64 << 20, need
    # the entry that allocates nothing
    Oa, Sa = nan_outputs(x, o_dtype)
    st = lib.gdn_chunk_fwd_seq_noalloc(sp, seg, _ptr(d["q"]), _ptr(d["k"]), _ptr(d["v"]),
                                       _ptr(d["alpha"]), _ptr(d["beta"]), None, _ptr(d["S0"]),
                                       _ptr(Oa), _ptr(Sa), hs)
    assert st == 0, lib.gdn_last_error().decode()
    torch.cuda.synchronize()
    # the existing entry with a workspace of its own
    Ob, Sb = nan_outputs(x, o_dtype)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    wp = ctypes.c_void_p((ws.data_ptr() + 255) // 256 * 256)
    st = lib.gdn_chunk_fwd_seq(sp, seg, _ptr(d["q"]), _ptr(d["k"]), _ptr(d["v"]),
                               _ptr(d["alpha"]), _ptr(d["beta"]), None, _ptr(d["S0"]),
                               _ptr(Ob), _ptr(Sb), wp, need, hs)
    assert st == 0, lib.gdn_last_error().decode()
    torch.cuda.synchronize()
    return x, (Oa, Sa), (Ob, Sb)


def test_noalloc_matches_workspace_entry_twice():
    # second call smaller than the first
    for case in ((2, 4, 1024, 64, 64, 64, 4, torch.float32, 1),
                 (1, 2, 333, 128, 128, 64, 2, torch.bfloat16, 2)):
        say(f"no-alloc case {case}")
        x, (Oa, Sa), (Ob, Sb) = run_both(*case)
        assert torch.isfinite(Oa.float()).all() and torch.isfinite(Sa).all()
        # same kernels, same inputs: identical results
        assert torch.equal(Oa, Ob) and torch.equal(Sa, Sb)
        Oref, Sref = oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"])
        tol_o = TOL["bf16"] + (2.0 ** -9 if Oa.dtype == torch.bfloat16 else 0.0)
        eo, es = rel_err(Oa.float().cpu().numpy(), Oref), rel_err(Sa.cpu().numpy(), Sref)
        say(f"  O {eo:.2e}  S {es:.2e}")
        assert eo < tol_o and es < TOL["bf16"]


def test_noalloc_plain_form_needs_no_scratch():
    """One segment: the plain form, which uses no scratch at all."""
    x = make_random(1, 2, 200, 64, 64, dtype="bf16", chunk=64, seed=3)
    d = to_dev(x)
    O, S = nan_outputs(x)
    gdn.gdn_chunk_fwd_seq_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                  chunk_size=64, seg_chunks=1000, O=O, S_final=S)
    torch.cuda.synchronize()
    Oref, Sref = oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"])
    assert rel_err(O.cpu().numpy(), Oref) < TOL["bf16"]
    assert rel_err(S.cpu().numpy(), Sref) < TOL["bf16"]
