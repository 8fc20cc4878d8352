"""GPU parity of ss_fwd / ss_fwd_step against the float64 oracle (through the C ABI)."""
import itertools

import numpy as np
import pytest
import torch

import oracle
from _util import TOL, f64, full_compare, inputs, oracle_args, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


def _ss():
    from mamba_selective_scan_fwd_amd import ss
    ss.load_library()
    return ss


def _run(prob, softplus=True, ckpt=False, poison=True):
    ss = _ss()
    g = to_dev(prob)
    Bsz, Dd, L = prob["u"].shape
    y = torch.full((Bsz, Dd, L), float("nan"), dtype=g["u"].dtype, device="cuda") if poison else None
    out = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"],
                 delta_softplus=softplus, lengths=g["lengths"], return_ckpt=ckpt, y=y)
    torch.cuda.synchronize()
    return out


def _check_full(prob, softplus=True, tol=None):
    say("case B=%d D=%d N=%d L=%d io=%s" % (prob["batch"], prob["dim"], prob["dstate"], prob["seqlen"], prob["io"]))
    y, last, _ = _run(prob, softplus)
    lens = None if prob.get("lengths") is None else prob["lengths"].numpy()
    yr, lr = oracle.fwd(**oracle_args(prob), softplus=softplus, lengths=lens)
    tol = tol or TOL[prob["io"]]
    ey, el = rel_err(f64(y), yr), rel_err(f64(last), lr)
    assert ey <= tol, ("y", ey)
    assert el <= tol, ("last_state", el)
    if lens is not None:
        yh = f64(y)
        for b, ln in enumerate(lens):
            assert np.all(yh[b, :, ln:] == 0.0)
    return ey, el


# --------------------------------------------------------------- workloads

def test_config0_fp32():
    _check_full(inputs.make_config(0))


def test_config1_fp32_long_chunked():
    """L = 32768 with 16 channels: runs the time-chunked scan."""
    _check_full(inputs.make_config(1))


def test_config2_fp16_full_and_decode():
    """mamba-130m layer shape (fp16) at full size, every channel against the oracle (y and the
    final state), then 64 decode steps from the device's final state, every channel against the
    oracle's continued sequence."""
    prob = inputs.make_config(2)
    ss = _ss()
    say("config2 fwd (all 12288 channels)")
    y, last, _ = _run(prob)
    ey, el, st_ref = full_compare(prob, y, last)
    say("config2 fwd: y %.3e, last_state %.3e" % (ey, el))
    assert ey <= TOL["f16"], ("y", ey)
    assert el <= TOL["f16"], ("last_state", el)
    # decode continues from the device's final state; the oracle from its own
    g = to_dev(prob)
    state = last.clone()
    A, D, bias = f64(prob["A"]), f64(prob["D"]), f64(prob["bias"])
    say("config2 decode (64 steps, all channels)")
    worst = 0.0
    for k, tok in enumerate(prob["decode"]):
        gt = {key: v.to("cuda") for key, v in tok.items()}
        yt, state = ss.step(gt["u_t"], gt["delta_t"], g["A"], gt["B_t"], gt["C_t"], state, D=g["D"],
                            z_t=gt["z_t"], delta_bias=g["bias"], state_out=state)
        yr, st_ref = oracle.step(f64(tok["u_t"]), f64(tok["delta_t"]), A, f64(tok["B_t"]), f64(tok["C_t"]), st_ref,
                                 D=D, z_t=f64(tok["z_t"]), bias=bias)
        torch.cuda.synchronize()
        e = rel_err(f64(yt), yr)
        worst = max(worst, e)
        assert e <= TOL["f16"], ("step", k, e)
    es = rel_err(f64(state), st_ref)
    say("config2 decode: worst step y %.3e, state after 64 steps %.3e" % (worst, es))
    assert es <= TOL["f16"]


def test_config3_bf16_ragged_full():
    """mamba-2.8b layer shape (bf16) with ragged rows at full size: every channel of every row
    against the oracle, and every masked tail exactly zero (checked on the device)."""
    prob = inputs.make_config(3)
    say("config3 lengths %s (all 20480 channels)" % prob["lengths"].tolist())
    y, last, _ = _run(prob)
    lens = prob["lengths"].numpy()
    for b, ln in enumerate(lens):
        tail = y[b, :, int(ln):]
        assert tail.numel() == 0 or bool((tail == 0).all())
    ey, el, _ = full_compare(prob, y, last)
    say("config3: y %.3e, last_state %.3e" % (ey, el))
    assert ey <= TOL["bf16"], ("y", ey)
    assert el <= TOL["bf16"], ("last_state", el)


# --------------------------------------------------------------- flags / dtypes

@pytest.mark.parametrize("io", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("use_D,use_z,use_bias,softplus", list(itertools.product([False, True], repeat=4)))
def test_flag_matrix(io, use_D, use_z, use_bias, softplus):
    prob = inputs.make_problem(2, 40, 16, 200, io, seed=31, with_D=use_D, with_z=use_z, with_bias=use_bias)
    if not softplus:
        # without softplus Delta = delta + bias must stay positive for a decaying scan
        dl = prob["delta"].float().abs() * 0.05 + 0.01
        if use_bias:
            dl = dl - prob["bias"][None, :, None]
        prob["delta"] = dl.to(prob["delta"].dtype)
    _check_full(prob, softplus)


# --------------------------------------------------------------- edge shapes

@pytest.mark.parametrize("Bsz,Dd,N,L", [
    (1, 1, 16, 1), (1, 16, 16, 1), (3, 17, 16, 63), (2, 33, 16, 64), (1, 40, 16, 65), (2, 5, 7, 129),
    (1, 3, 1, 100), (4, 64, 16, 257), (1, 16, 16, 4096), (2, 1, 16, 3000), (5, 100, 4, 77)])
def test_edge_shapes(Bsz, Dd, N, L):
    for io in ("f32", "bf16"):
        prob = inputs.make_problem(Bsz, Dd, N, L, io, seed=Bsz * 1000 + Dd * 10 + N + L)
        _check_full(prob)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_max_seqlen(io):
    """The longest sequence the ABI accepts, L = 2^24 (one step past it is rejected on
    the host): two channels of one row, so the time-chunked path runs with 2^18 tiles
    per row and the 32-bit buffer offsets at their largest; whole y and final state
    against the oracle."""
    _check_full(inputs.make_problem(1, 2, 16, 1 << 24, io, seed=2424))


def test_max_channels():
    """2^24 channels (two rows of d_inner = 2^23) at L = 2: 2^20 workgroups for the scan
    and for the decode step, with 64-bit channel and weight indices; y and the final
    state against the oracle, then one decode step from the device's final state."""
    Bsz, Dd, N, L = 2, 1 << 23, 16, 2
    prob = inputs.make_problem(Bsz, Dd, N, L, "f16", seed=2426, decode_steps=1)
    say("max channels B=%d D=%d L=%d" % (Bsz, Dd, L))
    ss = _ss()
    y, last, _ = _run(prob)
    yr, lr = oracle.fwd(**oracle_args(prob))
    assert rel_err(f64(y), yr) <= TOL["f16"]
    assert rel_err(f64(last), lr) <= TOL["f16"]
    del y, yr
    g = to_dev(prob)
    tok = prob["decode"][0]
    gt = {key: v.to("cuda") for key, v in tok.items()}
    yt, st = ss.step(gt["u_t"], gt["delta_t"], g["A"], gt["B_t"], gt["C_t"], last, D=g["D"], z_t=gt["z_t"],
                     delta_bias=g["bias"])
    torch.cuda.synchronize()
    ytr, str_ = oracle.step(f64(tok["u_t"]), f64(tok["delta_t"]), f64(prob["A"]), f64(tok["B_t"]), f64(tok["C_t"]),
                            f64(last), D=f64(prob["D"]), z_t=f64(tok["z_t"]), bias=f64(prob["bias"]))
    assert rel_err(f64(yt), ytr) <= TOL["f16"]
    assert rel_err(f64(st), str_) <= TOL["f16"]


@pytest.mark.parametrize("io", ["f32", "f16"])
def test_ragged_lengths_edges(io):
    """Row lengths on and around tile edges, a length-1 row, a full row, and clamped values."""
    L = 300
    prob = inputs.make_problem(7, 24, 16, L, io, seed=41)
    raw = torch.tensor([1, 64, 65, 128, L, 0, L + 50], dtype=torch.int32)
    prob["lengths"] = raw
    say("ragged edges io=%s" % io)
    y, last, _ = _run(prob)
    clamped = np.clip(raw.numpy(), 0, L)
    yr, lr = oracle.fwd(**oracle_args(prob), lengths=clamped)
    assert rel_err(f64(y), yr) <= TOL[io]
    assert rel_err(f64(last), lr) <= TOL[io]
    yh = f64(y)
    for b, ln in enumerate(clamped):
        assert np.all(yh[b, :, ln:] == 0.0)
    assert np.all(f64(last)[5] == 0.0)  # a zero-length row keeps the zero state


def test_checkpoints_match_oracle_states():
    for (Bsz, Dd, L, ragged) in [(2, 20, 200, False), (1, 16, 4096, False), (3, 40, 333, True)]:
        prob = inputs.make_problem(Bsz, Dd, 16, L, "f32", seed=51 + L, ragged=ragged)
        say("ckpt B=%d D=%d L=%d" % (Bsz, Dd, L))
        y, last, ck = _run(prob, ckpt=True)
        lens = None if prob["lengths"] is None else prob["lengths"].numpy()
        _, _, st = oracle.fwd(**oracle_args(prob), lengths=lens, states_every=64)
        assert rel_err(f64(ck), st) <= TOL["f32"]


def test_batch_permutation():
    """Permuting batch rows permutes outputs exactly (rows never read each other's data)."""
    prob = inputs.make_problem(4, 48, 16, 150, "f32", seed=61)
    y, last, _ = _run(prob)
    perm = [3, 1, 0, 2]
    prob2 = dict(prob)
    for k in ("u", "delta", "z", "Bm", "Cm"):
        prob2[k] = prob[k][perm].contiguous()
    y2, last2, _ = _run(prob2)
    assert torch.equal(y2, y[perm]) and torch.equal(last2, last[perm])


def test_chunked_equals_single_pass_shape():
    """A problem that splits time into chunks agrees with the oracle on every output,
    including the final state handed over between chunks."""
    prob = inputs.make_problem(1, 8, 16, 2500, "f32", seed=71, ragged=False)
    _check_full(prob)
    prob = inputs.make_problem(2, 8, 16, 2500, "f32", seed=72, ragged=True)
    _check_full(prob)


# --------------------------------------------------------------- decode step

@pytest.mark.parametrize("io", ["f32", "f16", "bf16"])
def test_step_batch_gt1_inplace(io):
    """B > 1 decode, in place and out of place, against the oracle step."""
    ss = _ss()
    Bsz, Dd, N = 4, 70, 16
    prob = inputs.make_problem(Bsz, Dd, N, 1, io, seed=81, decode_steps=3)
    g = to_dev(prob)
    rng = np.random.default_rng(82)
    st0 = torch.from_numpy(rng.standard_normal((Bsz, Dd, N))).float()
    st_dev = st0.to("cuda")
    st_ref = f64(st0)
    for k, tok in enumerate(prob["decode"]):
        gt = {key: v.to("cuda") for key, v in tok.items()}
        inplace = k % 2 == 0
        say("step io=%s k=%d inplace=%s" % (io, k, inplace))
        yt, st_new = ss.step(gt["u_t"], gt["delta_t"], g["A"], gt["B_t"], gt["C_t"], st_dev, D=g["D"],
                             z_t=gt["z_t"], delta_bias=g["bias"], state_out=st_dev if inplace else None)
        yr, st_ref = oracle.step(f64(tok["u_t"]), f64(tok["delta_t"]), f64(prob["A"]), f64(tok["B_t"]),
                                 f64(tok["C_t"]), st_ref, D=f64(prob["D"]), z_t=f64(tok["z_t"]),
                                 bias=f64(prob["bias"]))
        torch.cuda.synchronize()
        assert rel_err(f64(yt), yr) <= TOL[io]
        assert rel_err(f64(st_new), st_ref) <= TOL[io]
        st_dev = st_new


def test_forward_then_steps_equals_longer_forward():
    """concat(step) == forward: fwd over [0, L0) then single steps == fwd over [0, L)."""
    ss = _ss()
    prob = inputs.make_problem(2, 24, 16, 90, "f32", seed=91)
    g = to_dev(prob)
    L0 = 70
    sl = lambda t: t[..., :L0].contiguous()
    y0, st, _ = ss.fwd(sl(g["u"]), sl(g["delta"]), g["A"], sl(g["Bm"]), sl(g["Cm"]), D=g["D"], z=sl(g["z"]),
                       delta_bias=g["bias"])
    yfull, lastfull, _ = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"],
                                delta_bias=g["bias"])
    ys = []
    for t in range(L0, 90):
        yt, st = ss.step(g["u"][..., t].contiguous(), g["delta"][..., t].contiguous(), g["A"],
                         g["Bm"][..., t].contiguous(), g["Cm"][..., t].contiguous(), st, D=g["D"],
                         z_t=g["z"][..., t].contiguous(), delta_bias=g["bias"])
        ys.append(yt)
    torch.cuda.synchronize()
    ycat = torch.cat([y0, torch.stack(ys, dim=-1)], dim=-1)
    assert rel_err(f64(ycat), f64(yfull)) <= 1e-5
    assert rel_err(f64(st), f64(lastfull)) <= 1e-5


# --------------------------------------------------------------- prepared calls

def test_prepared_forward_call_matches_fwd():
    """FwdCall (validated once, replayed) gives the same bits as fwd on the same buffers,
    on the single-pass and on the time-chunked paths, over repeated launches."""
    ss = _ss()
    for Bsz, Dd, L, io in [(2, 40, 300, "f16"), (1, 16, 4096, "f32")]:
        prob = inputs.make_problem(Bsz, Dd, 16, L, io, seed=95)
        g = to_dev(prob)
        say("FwdCall B=%d D=%d L=%d io=%s" % (Bsz, Dd, L, io))
        y_ref, last_ref, _ = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"],
                                    delta_bias=g["bias"])
        y = torch.empty_like(y_ref)
        last = torch.empty_like(last_ref)
        call = ss.FwdCall(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"],
                          y=y, last_state=last)
        for _ in range(3):
            y.fill_(float("nan"))
            call()
            torch.cuda.synchronize()
            assert torch.equal(y, y_ref) and torch.equal(last, last_ref)


@pytest.mark.parametrize("io", ["f32", "f16"])
def test_prepared_step_call_matches_step(io):
    """StepCall updating the state in place over several steps == ss.step == the oracle."""
    ss = _ss()
    Bsz, Dd, N = 3, 50, 16
    prob = inputs.make_problem(Bsz, Dd, N, 1, io, seed=96, decode_steps=4)
    g = to_dev(prob)
    st0 = torch.from_numpy(np.random.default_rng(97).standard_normal((Bsz, Dd, N))).float()
    st_a = st0.to("cuda")
    st_b = st0.to("cuda")
    st_ref = f64(st0)
    ya = torch.empty((Bsz, Dd), dtype=g["u"].dtype, device="cuda")
    toks = [{k: v.to("cuda") for k, v in t.items()} for t in prob["decode"]]
    calls = [ss.StepCall(t["u_t"], t["delta_t"], g["A"], t["B_t"], t["C_t"], st_a, D=g["D"], z_t=t["z_t"],
                         delta_bias=g["bias"], y=ya) for t in toks]
    for k, (tok, call) in enumerate(zip(prob["decode"], calls)):
        say("StepCall io=%s k=%d" % (io, k))
        call()
        t = toks[k]
        yb, st_b = ss.step(t["u_t"], t["delta_t"], g["A"], t["B_t"], t["C_t"], st_b, D=g["D"], z_t=t["z_t"],
                           delta_bias=g["bias"])
        yr, st_ref = oracle.step(f64(tok["u_t"]), f64(tok["delta_t"]), f64(prob["A"]), f64(tok["B_t"]),
                                 f64(tok["C_t"]), st_ref, D=f64(prob["D"]), z_t=f64(tok["z_t"]),
                                 bias=f64(prob["bias"]))
        torch.cuda.synchronize()
        assert torch.equal(ya, yb) and torch.equal(st_a, st_b)
        assert rel_err(f64(ya), yr) <= TOL[io]
        assert rel_err(f64(st_a), st_ref) <= TOL[io]
