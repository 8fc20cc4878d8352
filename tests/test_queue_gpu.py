"""The forward's work queue against the float64 oracle.

ss_fwd takes the queue for ragged rows and for more 16-channel row blocks than the GPU holds
at once when they do not fill it evenly: units of 2048 steps of a row block, handed out longest
row first, each continuing from the state the previous unit of its row block published.  These
problems are large enough not to split time (4 x 1024 channels, 5 x 2560), so every one runs
the queue; y, the final state and the per-64-step checkpoints are compared over the whole
tensors, masked tails must be exactly 0, and the queue's error word must stay 0.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from _util import TOL, f64, full_compare, inputs, say, to_dev

pytestmark = pytest.mark.gpu


def _ss():
    from mamba_selective_scan_fwd_amd import ss
    ss.load_library()
    return ss


def _run(prob, lengths=None, seq=None, h0=None):
    ss = _ss()
    g = to_dev(prob)
    Bsz, Dd, L = prob["u"].shape
    N = prob["A"].shape[1]
    lib = ss.load_library()
    pr = ss.problem(Bsz, Dd, N, L, g["u"].dtype)
    assert lib.ss_fwd_workspace_min(ctypes.byref(pr)) == 0, "time would be split"
    wsz = lib.ss_fwd_workspace_size(ctypes.byref(pr))
    ws = torch.full(((wsz + 3) // 4,), -1, dtype=torch.int32, device="cuda")   # dirty on entry
    y, last, ck = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"],
                         lengths=lengths, seq_idx=seq, h0=h0, return_ckpt=True, workspace=ws,
                         y=torch.full((Bsz, Dd, L), float("nan"), dtype=g["u"].dtype, device="cuda"))
    torch.cuda.synchronize()
    assert int(ws[1].item()) == 0, "a wait between queue units gave up"
    return y, last, ck


def _check(prob, y, last, ck, lens=None, seq=None, h0=None, tol=None):
    tol = tol or TOL[prob["io"]]
    Bsz, Dd, L = prob["u"].shape
    yr, lr, sr = oracle.fwd(f64(prob["u"]), f64(prob["delta"]), f64(prob["A"]), f64(prob["Bm"]), f64(prob["Cm"]),
                            D=f64(prob["D"]), z=f64(prob["z"]), bias=f64(prob["bias"]), lengths=lens,
                            seq_idx=None if seq is None else seq.cpu().numpy(),
                            h0=None if h0 is None else h0.cpu().double().numpy(), states_every=64)
    from _util import rel_err
    ey, el, ec = rel_err(f64(y), yr), rel_err(f64(last), lr), rel_err(f64(ck), sr)
    say("  y %.2e  last %.2e  ckpt %.2e" % (ey, el, ec))
    assert ey <= tol and el <= tol and ec <= tol, (ey, el, ec)
    if lens is not None:
        for b, ln in enumerate(lens):
            assert bool((y[b, :, int(ln):] == 0).all())


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_queue_ragged_rows(io):
    """Rows of length 0, 1, 2049 (a unit and one step) and the whole row (three units)."""
    L = 4200
    prob = inputs.make_problem(4, 1024, 16, L, io, seed=61)
    lens = np.array([0, 1, 2049, L])
    say("queue ragged %s lengths %s" % (io, lens.tolist()))
    y, last, ck = _run(prob, lengths=torch.tensor(lens, dtype=torch.int32, device="cuda"))
    _check(prob, y, last, ck, lens=lens)


def test_queue_ragged_documents_and_initial_state():
    """Ragged rows with packed documents and an initial state: the unit boundaries (2048 steps)
    cut documents, and the state a unit continues from must carry the resets and h0."""
    L = 4600
    prob = inputs.make_problem(4, 1024, 16, L, "f32", seed=62)
    lens = np.array([4100, 2047, 4600, 2048])
    seq = inputs.packed_documents(L, 4, 300, seed=63).to("cuda")
    h0 = torch.randn((4, 1024, 16), dtype=torch.float32, device="cuda")
    say("queue ragged + documents + h0, lengths %s" % lens.tolist())
    y, last, ck = _run(prob, lengths=torch.tensor(lens, dtype=torch.int32, device="cuda"), seq=seq, h0=h0)
    _check(prob, y, last, ck, lens=lens, seq=seq, h0=h0)


def test_queue_uneven_row_blocks():
    """No lengths, but 5 x 160 = 800 row blocks: more than 3 per CU and not a multiple of the
    slots, so the queue balances them."""
    prob = inputs.make_problem(5, 2560, 16, 2100, "f16", seed=64)
    say("queue uneven 5 x 2560, L=2100, f16")
    y, last, ck = _run(prob)
    _check(prob, y, last, ck)


def test_queue_matches_the_direct_scan_bit_for_bit():
    """The queue changes only the schedule: with a workspace too small for it the same problem
    runs one workgroup per row block, and every output is bit-identical."""
    ss = _ss()
    L = 4400
    prob = inputs.make_problem(4, 1024, 16, L, "bf16", seed=65)
    lens = torch.tensor([2500, 4400, 3, 4100], dtype=torch.int32, device="cuda")
    g = to_dev(prob)
    yq, lq, cq = _run(prob, lengths=lens)
    yd, ld, cd = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"],
                        lengths=lens, return_ckpt=True, workspace=torch.empty(16, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(yq, yd) and torch.equal(lq, ld) and torch.equal(cq, cd)


def test_config3_ragged_queue_every_channel():
    """The ragged mamba-2.8b workload, through the queue, every channel against the oracle."""
    prob = inputs.make_config(3)
    say("config3 via the queue, lengths %s" % prob["lengths"].tolist())
    g = to_dev(prob)
    y, last, _ = _run(prob, lengths=g["lengths"])
    ey, el, _ = full_compare(prob, y, last)
    say("  y %.2e  last %.2e" % (ey, el))
    assert ey <= TOL["bf16"] and el <= TOL["bf16"]


def test_queue_graph_replays_match_eager():
    """The work queue (its clearing kernel and the persistent scan) captured in a HIP graph and
    replayed three times, with eager work between the replays: every replay equals the eager
    result bit for bit, so its counter and flags start cleared on each replay."""
    ss = _ss()
    L = 2600
    prob = inputs.make_problem(3, 2048, 16, L, "bf16", seed=67)
    lens = torch.tensor([2600, 5, 2100], dtype=torch.int32, device="cuda")
    g = to_dev(prob)
    y_e = torch.empty_like(g["u"])
    s_e = torch.empty((3, 2048, 16), dtype=torch.float32, device="cuda")
    ss.FwdCall(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"],
               lengths=lens, y=y_e, last_state=s_e)()
    torch.cuda.synchronize()
    y = torch.empty_like(y_e)
    s = torch.empty_like(s_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call = ss.FwdCall(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"],
                          lengths=lens, y=y, last_state=s, stream=side)
        call()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ss.FwdCall(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"],
                   lengths=lens, y=y, last_state=s, stream=torch.cuda.current_stream())()
    for rep in range(3):
        y.fill_(float("nan"))
        junk = torch.randn(1 << 16, device="cuda").mul_(2.0).sum()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        say("queue graph replay %d" % rep)
        assert torch.equal(y, y_e) and torch.equal(s, s_e)
