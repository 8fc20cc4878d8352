"""GPU parity of ss_conv1d_fwd / ss_conv1d_step (depthwise causal conv1d + SiLU, the
step before the scan) against the float64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from _util import TOL, f64, inputs, rel_err, say

pytestmark = pytest.mark.gpu


def _ss():
    from mamba_selective_scan_fwd_amd import ss
    ss.load_library()
    return ss


def _data(Bsz, Dd, L, W, io, seed):
    rng = np.random.default_rng(seed)
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[io]
    x = torch.from_numpy(rng.standard_normal((Bsz, Dd, L))).to(dt)
    w = torch.from_numpy(rng.standard_normal((Dd, W)) * 0.5).float()
    bias = torch.from_numpy(rng.standard_normal(Dd) * 0.1).float()
    return x, w, bias


def _check(Bsz, Dd, L, W, io, silu=True, seq=None, init=None, seed=0, use_bias=True):
    ss = _ss()
    x, w, bias = _data(Bsz, Dd, L, W, io, seed)
    if not use_bias:
        bias = None
    say("conv B=%d D=%d L=%d W=%d io=%s silu=%s seq=%s init=%s" % (Bsz, Dd, L, W, io, silu, seq is not None,
                                                                   init is not None))
    out = torch.full_like(x, float("nan"), device="cuda")
    out, fin = ss.conv1d(x.cuda(), w.cuda(), None if bias is None else bias.cuda(), silu=silu,
                         seq_idx=None if seq is None else seq.cuda(), conv_init=None if init is None else init.cuda(),
                         return_final=True, out=out)
    torch.cuda.synchronize()
    ref, rfin = oracle.conv1d_fwd(f64(x), f64(w), None if bias is None else f64(bias), silu=silu,
                                  seq_idx=None if seq is None else seq.numpy(), conv_init=None if init is None else
                                  f64(init))
    e = rel_err(f64(out), ref)
    assert e <= TOL[io], e
    if W > 1:
        assert np.array_equal(f64(fin), rfin)     # the window holds inputs verbatim
    return out, fin


# rows whose length is a multiple of 8 run the vector kernel, the others the scalar one
@pytest.mark.parametrize("L", [1500, 1504])
@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("io", ["f32", "f16", "bf16"])
def test_widths_and_dtypes(W, io, L):
    _check(2, 37, L, W, io, seed=W)


@pytest.mark.parametrize("L", [1, 2, 3, 4, 5, 8, 16, 1023, 1024, 1025, 2040, 2048, 2056, 3000])
def test_lengths(L):
    _check(3, 20, L, 4, "f32", seed=L)


def test_no_silu_no_bias():
    _check(2, 16, 300, 4, "f32", silu=False, use_bias=False, seed=5)


@pytest.mark.parametrize("L", [700, 704])
@pytest.mark.parametrize("case", inputs.SEQ_CASES)
def test_document_resets(case, L):
    seq = inputs.make_seq_idx(case, 2, L, seed=61)
    _check(2, 24, L, 4, "f16", seq=seq, seed=6)


@pytest.mark.parametrize("L", [90, 96])
@pytest.mark.parametrize("with_seq", [False, True])
def test_initial_window(with_seq, L):
    rng = np.random.default_rng(62)
    init = torch.from_numpy(rng.standard_normal((2, 24, 3))).float()
    seq = inputs.make_seq_idx("consecutive_boundaries", 2, L, seed=63) if with_seq else None
    _check(2, 24, L, 4, "f32", seq=seq, init=init, seed=7)
    _check(2, 24, 2, 4, "f32", init=init, seed=8)     # a row shorter than the window
    _check(2, 24, 8, 3, "bf16", init=init[..., :2].contiguous(), seq=None if seq is None else seq[:, :8].contiguous(),
           seed=9)


def test_prefill_in_pieces_and_decode():
    """conv(x[:k]) -> window -> conv(x[k:m], conv_init=window) -> steps for t >= m, all on the
    device, equal to one conv over the whole row."""
    ss = _ss()
    x, w, bias = _data(2, 40, 500, 4, "f32", 9)
    xd, wd, bd = x.cuda(), w.cuda(), bias.cuda()
    full = ss.conv1d(xd, wd, bd)
    k, m = 123, 480
    o1, f1 = ss.conv1d(xd[..., :128].contiguous(), wd, bd, return_final=True)   # vector kernel pieces
    o2, f2 = ss.conv1d(xd[..., 128:496].contiguous(), wd, bd, conv_init=f1, return_final=True)
    torch.cuda.synchronize()
    assert rel_err(f64(torch.cat([o1, o2], dim=-1)), f64(full[..., :496])) <= 1e-6
    o1, f1 = ss.conv1d(xd[..., :k].contiguous(), wd, bd, return_final=True)
    o2, f2 = ss.conv1d(xd[..., k:m].contiguous(), wd, bd, conv_init=f1, return_final=True)
    outs = [o1, o2]
    win = f2.clone()
    for t in range(m, 500):
        o, win = ss.conv1d_step(xd[..., t].contiguous(), wd, win, bd)
        outs.append(o.unsqueeze(-1))
    torch.cuda.synchronize()
    assert rel_err(f64(torch.cat(outs, dim=-1)), f64(full)) <= 1e-6


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_step_against_oracle(io):
    ss = _ss()
    rng = np.random.default_rng(64)
    Bsz, Dd, W = 3, 70, 4
    x, w, bias = _data(Bsz, Dd, 5, W, io, 10)
    win = torch.from_numpy(rng.standard_normal((Bsz, Dd, W - 1))).float()
    win_d = win.cuda()
    ref_win = f64(win)
    for t in range(5):
        xt = x[..., t].contiguous()
        o, win_d = ss.conv1d_step(xt.cuda(), w.cuda(), win_d, bias.cuda())
        ro, ref_win = oracle.conv1d_step(f64(xt), f64(w), ref_win, f64(bias))
        torch.cuda.synchronize()
        assert rel_err(f64(o), ro) <= TOL[io]
        assert np.array_equal(f64(win_d), ref_win)


def test_prepared_step_matches_checked_step():
    """ConvStepCall (validated once, buffers refilled in place) gives the checked call's
    outputs and windows bit for bit over 8 steps."""
    ss = _ss()
    Bsz, Dd, W = 2, 40, 4
    x, w, bias = _data(Bsz, Dd, 8, W, "f16", 12)
    xd, wd, bd = x.cuda(), w.cuda(), bias.cuda()
    win_a = torch.zeros((Bsz, Dd, W - 1), dtype=torch.float32, device="cuda")
    win_b = win_a.clone()
    xt = torch.empty((Bsz, Dd), dtype=torch.float16, device="cuda")
    ot = torch.empty_like(xt)
    call = ss.ConvStepCall(xt, wd, win_b, ot, bias=bd)
    for t in range(8):
        oa, win_a = ss.conv1d_step(xd[..., t].contiguous(), wd, win_a, bd)
        xt.copy_(xd[..., t])
        call()
        torch.cuda.synchronize()
        assert torch.equal(oa, ot) and torch.equal(win_a, win_b)


def test_mamba130m_layer_shape():
    """B=8, d_inner=1536, L=2048, fp16, width 4: sampled channels against the oracle."""
    ss = _ss()
    x, w, bias = _data(8, 1536, 2048, 4, "f16", 11)
    out = ss.conv1d(x.cuda(), w.cuda(), bias.cuda())
    torch.cuda.synchronize()
    ds = torch.tensor([0, 1, 15, 16, 700, 1535])
    ref, _ = oracle.conv1d_fwd(f64(x[:, ds]), f64(w[ds]), f64(bias[ds]))
    assert rel_err(f64(out[:, ds.cuda()]), ref) <= TOL["f16"]
