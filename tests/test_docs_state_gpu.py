"""GPU parity of packed-document resets (seq_idx), the initial state (h0) and the
state gradients (dlast in, dh0 out) against the float64 oracle, through the C ABI.

"niverel-mamba" README, "seq_idx strict reset": the state restarts from zero at
every change of document id, certified over nine structural cases and at
L = 8192; the cache contract of the same README and of the "mamba-metal"
README (prefill in pieces == one prefill == steps) motivates h0.
"""
import numpy as np
import pytest
import torch

import oracle
from _util import GRAD_TOL, TOL, f64, inputs, oracle_args, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


def _ss():
    from mamba_selective_scan_fwd_amd import ss
    ss.load_library()
    return ss


def _fwd_check(prob, seq, h0=None, tol=None, rows=None):
    ss = _ss()
    g = to_dev(prob)
    Bsz, Dd, L = prob["u"].shape
    y = torch.full((Bsz, Dd, L), float("nan"), dtype=g["u"].dtype, device="cuda")
    seq_d = None if seq is None else seq.to("cuda")
    h0_d = None if h0 is None else h0.to("cuda")
    y, last, ck = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"],
                         lengths=g["lengths"], y=y, seq_idx=seq_d, h0=h0_d, return_ckpt=True)
    torch.cuda.synchronize()
    lens = None if prob.get("lengths") is None else prob["lengths"].numpy()
    yr, lr, sr = oracle.fwd(**oracle_args(prob), lengths=lens, seq_idx=None if seq is None else seq.numpy(),
                            h0=None if h0 is None else f64(h0), states_every=64)
    tol = tol or TOL[prob["io"]]
    ey, el, ec = rel_err(f64(y), yr), rel_err(f64(last), lr), rel_err(f64(ck), sr)
    say("  errors y=%.2e last=%.2e ckpt=%.2e" % (ey, el, ec))
    assert ey <= tol and el <= tol and ec <= tol
    if lens is not None:
        yh = f64(y)
        for b, ln in enumerate(lens):
            assert np.all(yh[b, :, ln:] == 0.0)
    return y, last, ck


# --------------------------------------------------------------- forward resets

@pytest.mark.parametrize("case", inputs.SEQ_CASES)
@pytest.mark.parametrize("shape", ["single_pass", "chunked"])
def test_forward_nine_cases(case, shape):
    """Both kernel paths: enough channels for one pass over time (B*D/4 >= 1024 waves),
    and a few channels over a long row (time-chunked scan, chunk edges inside documents)."""
    if shape == "single_pass":
        Bsz, Dd, L, io = 2, 2048, 200, "f16"
    else:
        Bsz, Dd, L, io = 2, 16, 1500, "f32"
    say("seq case=%s shape=%s B=%d D=%d L=%d io=%s" % (case, shape, Bsz, Dd, L, io))
    prob = inputs.make_problem(Bsz, Dd, 16, L, io, seed=101)
    seq = inputs.make_seq_idx(case, Bsz, L, seed=102)
    _fwd_check(prob, seq)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_forward_resets_with_lengths_and_h0(io):
    prob = inputs.make_problem(3, 40, 16, 700, io, seed=103, ragged=True)
    seq = inputs.make_seq_idx("misaligned_rows", 3, 700, seed=104)
    h0 = torch.from_numpy(np.random.default_rng(105).standard_normal((3, 40, 16))).float()
    say("seq + lengths %s + h0, io=%s" % (prob["lengths"].tolist(), io))
    _fwd_check(prob, seq, h0=h0)


def test_forward_resets_long_rows():
    """L = 8192 (the README's certification length), many short documents, both paths."""
    for Bsz, Dd in [(2, 64), (1, 4096)]:
        prob = inputs.make_problem(Bsz, Dd, 16, 8192, "f32", seed=106)
        seq = inputs.packed_documents(8192, Bsz, 700, seed=107)
        say("long rows B=%d D=%d L=8192" % (Bsz, Dd))
        if Bsz * Dd <= 128:
            _fwd_check(prob, seq)
        else:   # large: compare sampled channels
            ss = _ss()
            g = to_dev(prob)
            y, last, _ = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"],
                                delta_bias=g["bias"], seq_idx=seq.to("cuda"))
            torch.cuda.synchronize()
            ds = torch.tensor([0, 1, 17, 1000, 2048, 4095])
            sl = lambda t: f64(t[:, ds])
            yr, lr = oracle.fwd(sl(prob["u"]), sl(prob["delta"]), f64(prob["A"][ds]), f64(prob["Bm"]),
                                f64(prob["Cm"]), D=f64(prob["D"][ds]), z=sl(prob["z"]), bias=f64(prob["bias"][ds]),
                                seq_idx=seq.numpy())
            assert rel_err(f64(y[:, ds.cuda()]), yr) <= 1e-5
            assert rel_err(f64(last[:, ds.cuda()]), lr) <= 1e-5


def test_packed_documents_h0_mamba130m_layer():
    """The benchmarked packed-document workload: the mamba-130m layer (B=8, d_inner=1536,
    L=2048, fp16) with documents of U[1, 512] steps and an initial state, in the launch
    configuration the bench times; 64 sampled channels against the oracle."""
    ss = _ss()
    prob = inputs.make_config(2, decode_steps=0)
    seq = inputs.packed_documents(2048, 8, 512, seed=7)
    h0 = torch.from_numpy(np.random.default_rng(17).standard_normal((8, 1536, 16))).float()
    g = to_dev(prob)
    y, last, _ = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"],
                        seq_idx=seq.to("cuda"), h0=h0.to("cuda"))
    torch.cuda.synchronize()
    ds = torch.tensor(sorted(set(np.random.default_rng(18).choice(1536, 60, replace=False).tolist()) | {0, 1535}))
    sl = lambda t: f64(t[:, ds])
    yr, lr = oracle.fwd(sl(prob["u"]), sl(prob["delta"]), f64(prob["A"][ds]), f64(prob["Bm"]), f64(prob["Cm"]),
                        D=f64(prob["D"][ds]), z=sl(prob["z"]), bias=f64(prob["bias"][ds]), seq_idx=seq.numpy(),
                        h0=f64(h0[:, ds]))
    ey, el = rel_err(f64(y[:, ds.cuda()]), yr), rel_err(f64(last[:, ds.cuda()]), lr)
    say("  mamba-130m packed documents + h0: %d documents, errors y=%.2e last=%.2e"
        % (int((seq[:, 1:] != seq[:, :-1]).sum()) + 8, ey, el))
    assert ey <= TOL["f16"] and el <= TOL["f16"]


def test_packed_equals_documents_on_device():
    """model(x, seq_idx) == concat(model(doc_i)) with both sides on the GPU."""
    ss = _ss()
    Bsz, Dd, L = 1, 48, 400
    prob = inputs.make_problem(Bsz, Dd, 16, L, "f32", seed=108)
    g = to_dev(prob)
    seq = inputs.make_seq_idx("inside_one_tile", Bsz, L, seed=109)
    y, last, _ = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"],
                        seq_idx=seq.to("cuda"))
    row = seq[0].tolist()
    cuts = [0] + [t for t in range(1, L) if row[t] != row[t - 1]] + [L]
    for s0, s1 in zip(cuts[:-1], cuts[1:]):
        sl = lambda t: t[..., s0:s1].contiguous()
        yd, ld, _ = ss.fwd(sl(g["u"]), sl(g["delta"]), g["A"], sl(g["Bm"]), sl(g["Cm"]), D=g["D"], z=sl(g["z"]),
                           delta_bias=g["bias"])
        torch.cuda.synchronize()
        assert rel_err(f64(y[..., s0:s1]), f64(yd)) <= 1e-6
    assert rel_err(f64(last), f64(ld)) <= 1e-6


# --------------------------------------------------------------- initial state

@pytest.mark.parametrize("Bsz,Dd,L", [(2, 2048, 300), (1, 16, 3000)])
def test_initial_state(Bsz, Dd, L):
    prob = inputs.make_problem(Bsz, Dd, 16, L, "f32", seed=110)
    h0 = torch.from_numpy(np.random.default_rng(111).standard_normal((Bsz, Dd, 16))).float()
    say("h0 B=%d D=%d L=%d" % (Bsz, Dd, L))
    _, _, ck = _fwd_check(prob, None, h0=h0)
    assert torch.equal(ck[:, :, 0].cpu(), h0)


def test_prefill_in_pieces_equals_one_prefill():
    """fwd(x[:k]) -> last_state -> fwd(x[k:], h0=last_state) == fwd(x), on the device."""
    ss = _ss()
    prob = inputs.make_problem(2, 40, 16, 1000, "f32", seed=112)
    g = to_dev(prob)
    y, last, _ = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"])
    k = 333
    a = lambda t: t[..., :k].contiguous()
    b = lambda t: t[..., k:].contiguous()
    y1, s1, _ = ss.fwd(a(g["u"]), a(g["delta"]), g["A"], a(g["Bm"]), a(g["Cm"]), D=g["D"], z=a(g["z"]),
                       delta_bias=g["bias"])
    y2, s2, _ = ss.fwd(b(g["u"]), b(g["delta"]), g["A"], b(g["Bm"]), b(g["Cm"]), D=g["D"], z=b(g["z"]),
                       delta_bias=g["bias"], h0=s1)
    torch.cuda.synchronize()
    assert rel_err(f64(torch.cat([y1, y2], dim=-1)), f64(y)) <= 1e-5
    assert rel_err(f64(s2), f64(last)) <= 1e-5


# --------------------------------------------------------------- backward

def _bwd_check(prob, seq=None, h0=None, dlast=None):
    ss = _ss()
    g = to_dev(prob)
    seq_d = None if seq is None else seq.to("cuda")
    h0_d = None if h0 is None else h0.to("cuda")
    _, _, ck = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"],
                      return_last_state=False, return_ckpt=True, seq_idx=seq_d, h0=h0_d)
    got = ss.bwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], ck, g["dy"], D=g["D"], z=g["z"],
                 delta_bias=g["bias"], seq_idx=seq_d, dlast=None if dlast is None else dlast.to("cuda"),
                 want_dh0=True)
    torch.cuda.synchronize()
    ref = oracle.bwd(**oracle_args(prob), dy=f64(prob["dy"]), seq_idx=None if seq is None else seq.numpy(),
                     h0=None if h0 is None else f64(h0), dlast=None if dlast is None else f64(dlast), want_dh0=True)
    tol = GRAD_TOL if prob["io"] == "f32" else TOL[prob["io"]]
    errs = {k: rel_err(f64(got[k]), ref[k]) for k in ref}
    say("  errors " + " ".join("%s=%.2e" % kv for kv in sorted(errs.items())))
    for k, e in errs.items():
        assert e <= tol, (k, e)


@pytest.mark.parametrize("case", ["length1_docs", "tile_edges", "inside_one_tile", "terminal_padding",
                                  "many_short_docs"])
def test_backward_resets(case):
    Bsz, Dd, L = 2, 40, 500
    say("bwd seq case=%s B=%d D=%d L=%d" % (case, Bsz, Dd, L))
    prob = inputs.make_problem(Bsz, Dd, 16, L, "f32", seed=113, with_dy=True)
    _bwd_check(prob, seq=inputs.make_seq_idx(case, Bsz, L, seed=114))


@pytest.mark.parametrize("L", [1, 64, 300])
def test_backward_initial_and_final_state(L):
    Bsz, Dd = 2, 36
    rng = np.random.default_rng(115)
    h0 = torch.from_numpy(rng.standard_normal((Bsz, Dd, 16))).float()
    dlast = torch.from_numpy(rng.standard_normal((Bsz, Dd, 16))).float()
    say("bwd h0/dlast B=%d D=%d L=%d" % (Bsz, Dd, L))
    prob = inputs.make_problem(Bsz, Dd, 16, L, "f32", seed=116, with_dy=True)
    _bwd_check(prob, h0=h0, dlast=dlast)
    if L > 1:
        _bwd_check(prob, seq=inputs.make_seq_idx("misaligned_rows", Bsz, L, seed=117), h0=h0, dlast=dlast)


def test_backward_resets_many_segments_per_workgroup():
    """One channel block over 1100 chunks: each backward workgroup walks two or three
    (batch row, chunk) segments, chunks with and without document starts mixed."""
    Bsz, Dd, L = 1, 16, 64 * 1100
    prob = inputs.make_problem(Bsz, Dd, 16, L, "f32", seed=120, with_dy=True)
    say("bwd many segments B=%d D=%d L=%d" % (Bsz, Dd, L))
    _bwd_check(prob, seq=inputs.packed_documents(L, Bsz, 600, seed=121))


def test_backward_resets_workload_shape():
    """The backward workload's shape (B=4, d_inner=1536, L=4097) with packed documents and a
    final-state gradient, dh0 out: the benchmarked configuration."""
    prob = inputs.make_config(4)
    seq = inputs.packed_documents(4097, 4, 600, seed=118)
    dlast = torch.from_numpy(np.random.default_rng(119).standard_normal((4, 1536, 16))).float()
    say("bwd workload shape with packed documents and dlast")
    _bwd_check(prob, seq=seq, dlast=dlast)


def test_autograd_initial_and_last_state():
    """selective_scan_fn with h0 (requires grad) and return_last_state: torch autograd
    gradients against the oracle's, for the loss sum(dy*y) + sum(dlast*last)."""
    ss = _ss()
    Bsz, Dd, L = 2, 20, 150
    prob = inputs.make_problem(Bsz, Dd, 16, L, "f32", seed=119, with_dy=True)
    rng = np.random.default_rng(120)
    h0 = torch.from_numpy(rng.standard_normal((Bsz, Dd, 16))).float()
    dlast = torch.from_numpy(rng.standard_normal((Bsz, Dd, 16))).float()
    seq = inputs.make_seq_idx("consecutive_boundaries", Bsz, L, seed=121)
    g = to_dev(prob)
    leaves = {k: g[k].clone().requires_grad_(True) for k in ("u", "delta", "A", "Bm", "Cm", "D", "z", "bias")}
    h0_l = h0.to("cuda").requires_grad_(True)
    y, last = ss.selective_scan_fn(leaves["u"], leaves["delta"], leaves["A"], leaves["Bm"], leaves["Cm"],
                                   D=leaves["D"], z=leaves["z"], delta_bias=leaves["bias"], delta_softplus=True,
                                   return_last_state=True, seq_idx=seq.to("cuda"), h0=h0_l)
    loss = (y * g["dy"]).sum() + (last * dlast.to("cuda")).sum()
    loss.backward()
    ref = oracle.bwd(**oracle_args(prob), dy=f64(prob["dy"]), seq_idx=seq.numpy(), h0=f64(h0), dlast=f64(dlast),
                     want_dh0=True)
    names = {"u": "du", "delta": "ddelta", "A": "dA", "Bm": "dB", "Cm": "dC", "D": "dD", "z": "dz",
             "bias": "dbias"}
    for k, gk in names.items():
        assert rel_err(f64(leaves[k].grad), ref[gk]) <= GRAD_TOL, k
    assert rel_err(f64(h0_l.grad), ref["dh0"]) <= GRAD_TOL
