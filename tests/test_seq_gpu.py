"""Sequence-parallel form of the default path on the GPU, against the fp64
oracle.

The state recurrence is linear in the state, so a sequence can be cut into
segments that run at once and are joined afterwards ("Параллельность RNN?",
section "Уровень 2": a linear recurrence is associative).  gdn_chunk_fwd_seq
runs every segment in the fused kernel (the later ones from a zero state,
with the d_k rows of their transition alongside), then a combine over
segments and a correction of the later segments' outputs.  These tests
check:
  * O and S_final against the oracle's plain recurrence over the whole
    sequence, for forced segment lengths over chunk sizes, d_k, d_v, ragged
    T, eta, bf16 output, a given or zero S0 and S_final aliasing S0;
  * the intermediates left in the workspace, each against its own oracle
    run: the transition M_j of a segment (the recurrence from the identity
    with zero values, d_v = d_k; stored transposed), the carried queries
    qm_t (that run's outputs), the zero-state end states of the later
    segments and the first segment's end state (the recurrence over it from
    S0);
  * that gdn_chunk_fwd picks this form by itself where it should (few heads
    on a long sequence) and not on the main shape.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_13_amd as gdn
from gated_delta_rule_13_amd.workloads import make_random
from tests.gpu_helpers import TOL, elem_err, nan_outputs, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

# (B, H, T, d_k, d_v, C, seg_chunks, with eta, O dtype, with S0)
CASES = [
    (1, 2, 333, 128, 128, 64, 1, False, "f32", True),    # six one-chunk segments, ragged last
    (1, 2, 333, 128, 128, 64, 2, True, "f32", False),    # eta, zero S0
    (2, 1, 200, 64, 64, 32, 3, False, "bf16", True),     # bf16 O: zero-state outputs in the workspace
    (1, 3, 130, 96, 192, 64, 1, False, "f32", True),     # the Olmo Hybrid head shape
    (1, 1, 100, 32, 48, 16, 2, True, "f32", True),       # d_k 32, C 16, d_v not a multiple of 64
    (1, 2, 200, 256, 64, 32, 2, False, "f32", True),     # d_k 256
    (2, 4, 1024, 64, 64, 64, 4, False, "f32", True),     # the DeltaNet shape, four segments
    (1, 1, 2000, 128, 128, 64, 3, False, "bf16", False),  # eleven segments, bf16 O
]

ODT = {"f32": torch.float32, "bf16": torch.bfloat16}


def make_case(B, H, T, dk, dv, C, with_eta, with_s0, seed):
    x = make_random(B, H, T, dk, dv, dtype="bf16", chunk=C, seed=seed,
                    s0_std=0.02 if with_s0 else 0.0)
    eta = None
    if with_eta:
        g = torch.Generator().manual_seed(seed + 7)
        eta = torch.rand(B, H, T, generator=g).float()
    return x, eta


def run_seq(x, eta, C, seg_chunks, o_dtype, workspace=None, S0=None, S_final=None):
    d = to_dev(x)
    O, S = nan_outputs(x, o_dtype)
    if S_final is not None:
        S = S_final
    s0 = d["S0"] if S0 is None else S0
    O, S = gdn.gdn_chunk_fwd_seq(d["q"], d["k"], d["v"], d["alpha"], d["beta"], s0,
                                 chunk_size=C, seg_chunks=seg_chunks, o_dtype=o_dtype, O=O,
                                 S_final=S, eta=None if eta is None else eta.cuda(),
                                 workspace=workspace)
    torch.cuda.synchronize()
    return O, S


@pytest.mark.parametrize("B,H,T,dk,dv,C,seg,with_eta,odt,with_s0", CASES)
def test_segments_match_oracle(B, H, T, dk, dv, C, seg, with_eta, odt, with_s0):
    say(f"seq case B={B} H={H} T={T} dk={dk} dv={dv} C={C} seg_chunks={seg} eta={with_eta} "
        f"O={odt} S0={with_s0}")
    x, eta = make_case(B, H, T, dk, dv, C, with_eta, with_s0, seed=T + dk + seg)
    O, S = run_seq(x, eta, C, seg, ODT[odt])
    On, Sn = O.float().cpu().numpy(), S.cpu().numpy()
    assert np.isfinite(On).all() and np.isfinite(Sn).all(), "unwritten or non-finite outputs"
    Oref, Sref = oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"],
                                  eta=eta)
    eo, es = rel_err(On, Oref), rel_err(Sn, Sref)
    say(f"  O {eo:.2e} (elementwise {elem_err(On, Oref):.2f})  S {es:.2e}")
    # rounding O to bf16 adds at most 2^-9 relative per element, as on the
    # plain form
    tol_o = TOL["bf16"] + (2.0 ** -9 if odt == "bf16" else 0.0)
    assert eo < tol_o and es < TOL["bf16"]


def test_segments_agree_with_plain_form():
    """Same inputs, one segment against five: both within the tolerance of
    the oracle and close to each other."""
    x, _ = make_case(1, 2, 300, 128, 128, 64, False, True, seed=11)
    O1, S1 = run_seq(x, None, 64, 1000, torch.float32)
    O5, S5 = run_seq(x, None, 64, 1, torch.float32)
    Oref, Sref = oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"])
    for O, S in ((O1, S1), (O5, S5)):
        assert rel_err(O.cpu().numpy(), Oref) < TOL["bf16"]
        assert rel_err(S.cpu().numpy(), Sref) < TOL["bf16"]
    assert rel_err(O5.cpu().numpy(), O1.cpu().numpy()) < TOL["bf16"]


def test_state_in_place():
    """S_final may be S0 in the segmented form too (S0 is read by the fused
    pass, S_final written by the finishing launch after it)."""
    x, _ = make_case(1, 2, 250, 64, 64, 32, False, True, seed=5)
    Oref, Sref = oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"])
    state = x["S0"].cuda().clone()
    O, S = run_seq(x, None, 32, 2, torch.float32, S0=state, S_final=state)
    assert S.data_ptr() == state.data_ptr()
    assert rel_err(O.cpu().numpy(), Oref) < TOL["bf16"]
    assert rel_err(state.cpu().numpy(), Sref) < TOL["bf16"]


def _ws_views(ws: torch.Tensor, B, H, T, dk, dv, nseg):
    """The workspace's regions as float arrays (layout of include/gdn.h)."""
    base = (256 - ws.data_ptr() % 256) % 256
    raw = ws.cpu().numpy()[base:]
    up = lambda n: (n + 255) // 256 * 256
    bh = B * H
    n_state = bh * nseg * (dv + dk) * dk
    state = raw[:n_state * 4].view(np.float32).reshape(B, H, nseg, dv + dk, dk)
    off_q = up(n_state * 4)
    qm = raw[off_q:off_q + bh * T * dk * 4].view(np.float32).reshape(B, H, T, dk)
    return state, qm


def test_workspace_intermediates_match_oracle():
    B, H, T, dk, dv, C, L = 1, 2, 290, 64, 96, 32, 2
    seg_len = L * C
    nseg = (T + seg_len - 1) // seg_len
    x, eta = make_case(B, H, T, dk, dv, C, True, True, seed=29)
    shape = gdn.make_shape(B, H, T, dk, dv, C, torch.bfloat16, torch.float32)
    nbytes = gdn.gdn_chunk_fwd_seq_workspace_bytes(shape, L)
    ws = torch.full((nbytes + 256,), 0xFF, dtype=torch.uint8, device="cuda")
    O, S = run_seq(x, eta, C, L, torch.float32, workspace=ws)
    state, qm = _ws_views(ws, B, H, T, dk, dv, nseg)
    cut = lambda t, a, b: None if t is None else t[..., a:b].contiguous() if t.dim() == 3 \
        else t[:, :, a:b].contiguous()
    eye = torch.eye(dk, dtype=torch.float64).expand(B, H, dk, dk).contiguous()
    for j in range(nseg):
        a, b = j * seg_len, min(T, (j + 1) * seg_len)
        q, k, v = (cut(x[n], a, b) for n in ("q", "k", "v"))
        al, be = cut(x["alpha"], a, b), cut(x["beta"], a, b)
        et = cut(eta, a, b)
        # end state of the segment: from S0 for the first, from zero after
        _, Send = oracle.recurrent(q, k, v, al, be, S0=x["S0"] if j == 0 else None, eta=et)
        e = rel_err(state[:, :, j, :dv], Send)
        say(f"  segment {j}: end state {e:.2e}")
        assert e < TOL["bf16"]
        if j == 0:
            continue
        # transition and carried queries: identity start, zero values
        zeros = torch.zeros(B, H, b - a, dk, dtype=torch.float32)
        qm_ref, M_ref = oracle.recurrent(q, k, zeros, al, be, S0=eye, eta=et)
        em = rel_err(state[:, :, j, dv:], np.swapaxes(M_ref, -1, -2))
        eq = rel_err(qm[:, :, a:b], qm_ref)
        say(f"  segment {j}: transition {em:.2e}  carried queries {eq:.2e}")
        assert em < TOL["bf16"] and eq < TOL["bf16"]
    Oref, Sref = oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"],
                                  eta=eta)
    assert rel_err(O.cpu().numpy(), Oref) < TOL["bf16"]
    assert rel_err(S.cpu().numpy(), Sref) < TOL["bf16"]


def test_default_plan_choice():
    """gdn_chunk_fwd takes the segmented form for few heads on long
    sequences (workspace > 0) and the plain form on the main shape."""
    few = gdn.make_shape(1, 1, 4096, 128, 128, 64, torch.bfloat16, torch.float32)
    main = gdn.make_shape(4, 16, 4096, 128, 128, 64, torch.bfloat16, torch.float32)
    assert gdn.gdn_chunk_fwd_workspace_bytes(few) > 0
    assert gdn.gdn_chunk_fwd_workspace_bytes(main) == 0


def test_default_plan_few_heads_matches_oracle():
    x, _ = make_case(1, 1, 4000, 128, 128, 64, False, True, seed=3)
    shape = gdn.make_shape(1, 1, 4000, 128, 128, 64, torch.bfloat16, torch.float32)
    assert gdn.gdn_chunk_fwd_workspace_bytes(shape) > 0
    d = to_dev(x)
    O, S = nan_outputs(x)
    gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], chunk_size=64,
                      O=O, S_final=S)
    torch.cuda.synchronize()
    Oref, Sref = oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"])
    eo, es = rel_err(O.cpu().numpy(), Oref), rel_err(S.cpu().numpy(), Sref)
    say(f"default plan, 1 head x 4000 tokens: O {eo:.2e}  S {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


def test_workspace_too_small_is_rejected():
    x, _ = make_case(1, 1, 256, 64, 64, 64, False, False, seed=1)
    d = to_dev(x)
    shape = gdn.make_shape(1, 1, 256, 64, 64, 64, torch.bfloat16, torch.float32)
    need = gdn.gdn_chunk_fwd_seq_workspace_bytes(shape, 1)
    assert need > 0
    lib = gdn.load()
    O, S = nan_outputs(x)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    p = (ws.data_ptr() + 255) // 256 * 256
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    hs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.gdn_chunk_fwd_seq(ctypes.byref(shape), 1, ptr(d["q"]), ptr(d["k"]), ptr(d["v"]),
                               ptr(d["alpha"]), ptr(d["beta"]), None, None, ptr(O), ptr(S),
                               ctypes.c_void_p(p), need - 1, hs)
    assert st == 5
    torch.cuda.synchronize()
    assert torch.isnan(O).all(), "nothing may be written when the call is rejected"
