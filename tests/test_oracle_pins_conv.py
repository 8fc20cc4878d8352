"""Pins of the oracle's depthwise causal conv1d + SiLU and its decode window.

"Mamba" walkthrough, Part IV Stage 2: depthwise (one filter per channel),
causal (left padding only, position t sees t-W+1 .. t), width d_conv = 4,
then SiLU.  Checked against numpy's convolution and torch's grouped conv1d
(library routines), the packed-document identity of the "niverel-mamba"
README ("seq_idx strict reset": the convolution state resets too), prefill
in pieces through conv_init/conv_final, and decode steps continuing a
prefill.  CPU only.
"""
import numpy as np
import pytest
import torch

import oracle
from mamba_selective_scan_fwd_amd import inputs


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _silu(v):
    return v / (1.0 + np.exp(-v))


def _data(seed, Bsz=2, Dd=5, L=37, W=4):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((Bsz, Dd, L)), rng.standard_normal((Dd, W)), rng.standard_normal(Dd)


@pytest.mark.parametrize("W", [2, 3, 4])
@pytest.mark.parametrize("silu", [False, True])
def test_matches_numpy_convolve(W, silu):
    x, w, bias = _data(41, W=W)
    out, fin = oracle.conv1d_fwd(x, w, bias, silu=silu)
    for b in range(x.shape[0]):
        for d in range(x.shape[1]):
            pre = np.convolve(x[b, d], w[d][::-1])[: x.shape[2]] + bias[d]
            ref = _silu(pre) if silu else pre
            assert _rel(out[b, d], ref) < 1e-14
    assert np.array_equal(fin, x[:, :, x.shape[2] - (W - 1):])


def test_matches_torch_grouped_conv1d():
    x, w, bias = _data(42, Bsz=3, Dd=7, L=50)
    out, _ = oracle.conv1d_fwd(x, w, bias, silu=True)
    xt = torch.from_numpy(x)
    ref = torch.nn.functional.conv1d(xt, torch.from_numpy(w).unsqueeze(1), torch.from_numpy(bias),
                                     padding=w.shape[1] - 1, groups=x.shape[1])[..., : x.shape[2]]
    assert _rel(out, torch.nn.functional.silu(ref).numpy()) < 1e-14


@pytest.mark.parametrize("case", inputs.SEQ_CASES)
def test_packed_equals_documents(case):
    x, w, bias = _data(43, Bsz=3, Dd=4, L=120)
    seq = inputs.make_seq_idx(case, 3, 120, seed=44).numpy()
    out, fin = oracle.conv1d_fwd(x, w, bias, seq_idx=seq)
    for b in range(3):
        row = seq[b]
        cuts = [0] + [t for t in range(1, 120) if row[t] != row[t - 1]] + [120]
        for s0, s1 in zip(cuts[:-1], cuts[1:]):
            od, fd = oracle.conv1d_fwd(x[b:b + 1, :, s0:s1], w, bias)
            assert _rel(out[b:b + 1, :, s0:s1], od) < 1e-14
        assert _rel(fin[b:b + 1], fd) < 1e-14 or np.all(fin[b:b + 1] == fd)   # last document's window


def test_prefill_in_pieces():
    x, w, bias = _data(45, L=60)
    full, fin = oracle.conv1d_fwd(x, w, bias)
    for k in (1, 2, 3, 4, 29):
        o1, f1 = oracle.conv1d_fwd(x[:, :, :k], w, bias)
        o2, f2 = oracle.conv1d_fwd(x[:, :, k:], w, bias, conv_init=f1)
        assert _rel(np.concatenate([o1, o2], axis=2), full) < 1e-14
        assert np.array_equal(f2, fin)


def test_steps_continue_a_prefill():
    x, w, bias = _data(46, L=40)
    full, _ = oracle.conv1d_fwd(x, w, bias)
    L0 = 25
    _, win = oracle.conv1d_fwd(x[:, :, :L0], w, bias)
    for t in range(L0, 40):
        o, win = oracle.conv1d_step(x[:, :, t], w, win, bias)
        assert _rel(o, full[:, :, t]) < 1e-14


def test_steps_from_an_empty_window_equal_the_prefill():
    x, w, bias = _data(47, L=9, W=4)
    full, _ = oracle.conv1d_fwd(x, w, bias)
    win = np.zeros((x.shape[0], x.shape[1], 3))
    for t in range(9):
        o, win = oracle.conv1d_step(x[:, :, t], w, win, bias)
        assert _rel(o, full[:, :, t]) < 1e-14
