"""ss_fwd_noalloc (the forward for callers that cannot allocate) against ss_fwd.

The entry point keeps the time-chunked scan's workspace in a fixed device
array; its results must be those of ss_fwd with a caller-provided workspace.
Two calls in a row share the array (the second on a smaller problem, which
leaves part of the first call's contents behind), each checked bit for bit
against ss_fwd on the same inputs.  A host check confirms that every forward
plan fits the array.
"""
import ctypes

import numpy as np
import pytest
import torch

from _util import inputs, say, to_dev


def _ss():
    from mamba_selective_scan_fwd_amd import ss
    ss.load_library()
    return ss


def test_every_plan_fits_the_array():
    """Host only: the least workspace of every forward plan (the time-chunked scan's) up to the
    sizes where time stops being split is within the fixed array."""
    ss = _ss()
    lib = ss.load_library()
    cap = lib.ss_fwd_noalloc_max_workspace()
    worst = 0
    for B in (1, 2, 3, 4, 7, 8, 16, 64, 255, 256):
        for D in (1, 15, 16, 17, 48, 63, 64, 100, 255, 256, 1000, 1023, 1024, 4096):
            for L in (1, 63, 64, 65, 2048, 1 << 20, 1 << 24):
                pr = ss.problem(B, D, 16, L, torch.float16)
                worst = max(worst, lib.ss_fwd_workspace_min(ctypes.byref(pr)))
    assert 0 < worst <= cap, (worst, cap)


def _call_noalloc(ss, g, y, last, seq=None, h0=None):
    lib = ss.load_library()
    Bsz, Dd, L = g["u"].shape
    pr = ss.problem(Bsz, Dd, g["A"].shape[1], L, g["u"].dtype)
    p = ss._ptr
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.ss_fwd_noalloc(ctypes.byref(pr), p(g["u"]), p(g["delta"]), p(g["A"]), p(g["Bm"]), p(g["Cm"]),
                              p(g["D"]), p(g["z"]), p(g["bias"]), p(g.get("lengths")), p(seq), p(h0), p(y), p(last),
                              None, st)


def _compare(ss, prob, seq=None, h0=None):
    g = to_dev(prob)
    Bsz, Dd, L = prob["u"].shape
    N = prob["A"].shape[1]
    pr = ss.problem(Bsz, Dd, N, L, g["u"].dtype)
    assert ss.load_library().ss_fwd_workspace_min(ctypes.byref(pr)) > 0, "not a time-chunked problem"
    y_ref, last_ref, _ = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"],
                                delta_bias=g["bias"], lengths=g["lengths"], seq_idx=seq, h0=h0)
    y = torch.full_like(y_ref, float("nan"))
    last = torch.full_like(last_ref, float("nan"))
    assert _call_noalloc(ss, g, y, last, seq=seq, h0=h0) == 0
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.equal(last, last_ref)
    assert torch.isfinite(y.float()).all()


@pytest.mark.gpu
def test_noalloc_matches_fwd_twice_second_smaller():
    ss = _ss()
    # the long-sequence workload: 16 channels over 32768 steps (time-chunked)
    say("ss_fwd_noalloc: B=1 D=16 N=16 L=32768 f32")
    _compare(ss, inputs.make_config(1))
    # then a smaller problem on the same array, fp16, with documents and an initial state
    say("ss_fwd_noalloc: B=2 D=8 N=12 L=3001 f16, seq_idx, h0")
    prob = inputs.make_problem(2, 8, 12, 3001, "f16", seed=5)
    seq = inputs.packed_documents(3001, 2, 700, seed=6).to("cuda")
    h0 = torch.randn((2, 8, 12), dtype=torch.float32, device="cuda")
    _compare(ss, prob, seq=seq, h0=h0)


@pytest.mark.gpu
def test_noalloc_without_time_split_needs_no_array():
    """A problem with channels enough to fill the GPU: no workspace at all, same results."""
    ss = _ss()
    say("ss_fwd_noalloc: B=4 D=1024 N=16 L=300 bf16 (no time split)")
    prob = inputs.make_problem(4, 1024, 16, 300, "bf16", seed=9)
    g = to_dev(prob)
    pr = ss.problem(4, 1024, 16, 300, torch.bfloat16)
    assert ss.load_library().ss_fwd_workspace_min(ctypes.byref(pr)) == 0
    y_ref, last_ref, _ = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"],
                                delta_bias=g["bias"])
    y = torch.empty_like(y_ref)
    last = torch.empty_like(last_ref)
    assert _call_noalloc(ss, g, y, last) == 0
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(last, last_ref)
