"""GPU parity of the one-launch time-chunked forward against the float64 oracle.

Problems with too few channels to fill the GPU split time into K chunks; each
chunk's entry state comes from the chunk pairs (page "Mamba", Part V, the
associative combine for h_t = a_t h_{t-1} + b_t), composed in two levels:
groups of G chunks (G the least power of two with G * G >= K).  The shapes
below give K from 2 to 256 and every position of a chunk in its group; the
optional inputs (ragged lengths, packed documents, an initial state,
checkpoints) are each crossed with the chunking.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from _util import TOL, f64, inputs, oracle_args, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


def _ss():
    from mamba_selective_scan_fwd_amd import ss
    ss.load_library()
    return ss


def plan(Bsz, Dd, L):
    """(K, G, number of groups) the library's planner picks (it splits time below 1024
    wavefronts of 16 states x 4 channels, into chunks of an even number of 64-step tiles,
    whose two halves a workgroup scans at once)."""
    waves = Bsz * ((Dd + 15) // 16) * 4
    tiles = (L + 63) // 64
    k = 1
    if waves < 1024:
        k = min((1024 + waves - 1) // waves, tiles)
    tpc = (tiles + k - 1) // k
    if k > 1:
        tpc += tpc & 1
    chunk = tpc * 64
    K = (L + chunk - 1) // chunk
    G = 1
    while G * G < K:
        G *= 2
    return K, G, (K + G - 1) // G


def _check(prob, seq=None, h0=None, workspace=None):
    ss = _ss()
    g = to_dev(prob)
    Bsz, Dd, L = prob["u"].shape
    y = torch.full((Bsz, Dd, L), float("nan"), dtype=g["u"].dtype, device="cuda")
    y, last, ck = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"],
                         lengths=g["lengths"], y=y, seq_idx=None if seq is None else seq.to("cuda"),
                         h0=None if h0 is None else h0.to("cuda"), return_ckpt=True, workspace=workspace)
    torch.cuda.synchronize()
    lens = None if prob.get("lengths") is None else prob["lengths"].numpy()
    yr, lr, sr = oracle.fwd(**oracle_args(prob), lengths=lens, seq_idx=None if seq is None else seq.numpy(),
                            h0=None if h0 is None else f64(h0), states_every=64)
    tol = TOL[prob["io"]]
    ey, el, ec = rel_err(f64(y), yr), rel_err(f64(last), lr), rel_err(f64(ck), sr)
    say("  errors y=%.2e last=%.2e ckpt=%.2e" % (ey, el, ec))
    assert ey <= tol and el <= tol and ec <= tol, (ey, el, ec)
    if lens is not None:
        yh = f64(y)
        for b, ln in enumerate(lens):
            assert np.all(yh[b, :, ln:] == 0.0)
    return y, last, ck


# (B, D, L, io) -> K, G, groups
SHAPES = [
    ((1, 4080, 200, "f16"), (2, 2, 1)),     # two chunks, one group; the last chunk's halves of 64 and 8 steps
    ((1, 16, 320, "f32"), (3, 2, 2)),       # the second group has one chunk, whose second half is empty
    ((1, 16, 2176, "f16"), (17, 8, 3)),     # a last group of one chunk
    ((1, 5, 4000, "bf16"), (32, 8, 4)),     # a partial channel block, ragged last chunk (one partial half)
    ((3, 16, 16389, "f32"), (65, 16, 5)),   # 256-step chunks (two tiles a half), three row blocks
]


@pytest.mark.parametrize("shape,expect", SHAPES, ids=["K%d" % e[0] for _, e in SHAPES])
def test_chunk_counts(shape, expect):
    Bsz, Dd, L, io = shape
    assert plan(Bsz, Dd, L) == expect
    say("lookback B=%d D=%d L=%d io=%s K,G,groups=%s" % (Bsz, Dd, L, io, expect))
    _check(inputs.make_problem(Bsz, Dd, 16, L, io, seed=301))


def test_lengths_documents_and_h0():
    """Ragged rows (one of length 1, one ending inside a chunk), packed documents and an
    initial state on a 24-chunk plan with three channel blocks (the last one partial)."""
    Bsz, Dd, L = 3, 40, 3000
    assert plan(Bsz, Dd, L) == (24, 8, 3)
    prob = inputs.make_problem(Bsz, Dd, 16, L, "f32", seed=302)
    prob["lengths"] = torch.tensor([L, 1, 1234], dtype=torch.int32)
    seq = inputs.packed_documents(L, Bsz, 500, seed=303)
    h0 = torch.from_numpy(np.random.default_rng(304).standard_normal((Bsz, Dd, 16))).float()
    say("lookback lengths+docs+h0 B=%d D=%d L=%d" % (Bsz, Dd, L))
    _check(prob, seq=seq, h0=h0)


def test_empty_and_one_step_rows():
    """Rows of length 0 (the output is exactly zero and the final state is h0) and 1 next to a
    full row, on a plan whose rows end in different chunks and groups."""
    Bsz, Dd, L = 4, 16, 5000
    prob = inputs.make_problem(Bsz, Dd, 16, L, "f32", seed=311)
    prob["lengths"] = torch.tensor([0, L, 1, 4097], dtype=torch.int32)
    h0 = torch.from_numpy(np.random.default_rng(312).standard_normal((Bsz, Dd, 16))).float()
    say("lookback empty rows plan=%s" % (plan(Bsz, Dd, L),))
    y, last, _ = _check(prob, h0=h0)
    assert torch.equal(last[0].cpu(), h0[0])


def test_dstate_below_16_and_h0():
    prob = inputs.make_problem(2, 16, 7, 2500, "bf16", seed=305)
    h0 = torch.from_numpy(np.random.default_rng(306).standard_normal((2, 16, 7))).float()
    say("lookback N=7 B=2 D=16 L=2500 plan=%s" % (plan(2, 16, 2500),))
    _check(prob, h0=h0)


def test_dirty_workspace_reused_across_paths():
    """The workspace's contents on entry do not matter (a kernel at the start of each call
    resets what the call polls), so one workspace, dirty to begin with, serves a sequence of
    calls: two time-chunked problems of different plans, a ragged problem through the work
    queue, then a time-chunked one again, each over what the previous one left.  No wait
    gave up."""
    ss = _ss()
    lib = ss.load_library()
    shapes = [((1, 16, 8192), None, 307), ((2, 24, 700), None, 308), ((3, 2048, 600), [600, 1, 333], 309),
              ((1, 40, 5000), None, 310)]
    wsz = 0
    for (Bsz, Dd, L), lens, _ in shapes:
        wsz = max(wsz, lib.ss_fwd_workspace_size(ctypes.byref(ss.problem(Bsz, Dd, 16, L, torch.float32))))
    ws = torch.full((wsz // 4 + 64,), -1, dtype=torch.int32, device="cuda")
    for (Bsz, Dd, L), lens, seed in shapes:
        say("lookback reuse shape=%s lengths=%s plan=%s" % ((Bsz, Dd, L), lens, plan(Bsz, Dd, L)))
        prob = inputs.make_problem(Bsz, Dd, 16, L, "f32", seed=seed)
        if lens is not None:
            prob["lengths"] = torch.tensor(lens, dtype=torch.int32)
        if Dd > 1000:  # the queue problem: a few sampled channels are enough here
            _check_sampled(prob, workspace=ws)
        else:
            _check(prob, workspace=ws)
        assert int(ws[1].item()) == 0, "a wait between workgroups gave up"


def _check_sampled(prob, workspace):
    ss = _ss()
    g = to_dev(prob)
    Bsz, Dd, L = prob["u"].shape
    y, last, _ = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"],
                        lengths=g["lengths"], workspace=workspace)
    torch.cuda.synchronize()
    rows = np.array([0 * Dd + 5, 1 * Dd + 1000, 2 * Dd + 2047])
    yr, lr = oracle.fwd(**oracle_args(prob), lengths=prob["lengths"].numpy(), rows=rows)
    yg, lg = f64(y).reshape(Bsz * Dd, L), f64(last).reshape(Bsz * Dd, -1)
    ey = rel_err(yg[rows], yr.reshape(Bsz * Dd, L)[rows])
    el = rel_err(lg[rows], lr.reshape(Bsz * Dd, -1)[rows])
    assert ey <= TOL["f32"] and el <= TOL["f32"], (ey, el)


def test_repeated_calls_bit_identical():
    """The schedule varies from call to call (the unit counter), the arithmetic does not."""
    ss = _ss()
    prob = inputs.make_config(1)
    g = to_dev(prob)
    outs = []
    for _ in range(3):
        y, last, _ = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"],
                            delta_bias=g["bias"])
        outs.append((y.clone(), last.clone()))
    torch.cuda.synchronize()
    for y, last in outs[1:]:
        assert torch.equal(y, outs[0][0]) and torch.equal(last, outs[0][1])
