"""GPU parity of ss_bwd against the float64 oracle and finite differences (through the C ABI)."""
import itertools

import numpy as np
import pytest
import torch

import oracle
from _util import GRAD_TOL, TOL, f64, inputs, oracle_args, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

GRADS = ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "dbias")


def _ss():
    from mamba_selective_scan_fwd_amd import ss
    ss.load_library()
    return ss


def _gpu_grads(prob, softplus=True):
    ss = _ss()
    g = to_dev(prob)
    _, _, ck = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"],
                      delta_softplus=softplus, return_last_state=False, return_ckpt=True)
    out = ss.bwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], ck, g["dy"], D=g["D"], z=g["z"],
                 delta_bias=g["bias"], delta_softplus=softplus)
    torch.cuda.synchronize()
    return {k: f64(v) for k, v in out.items()}


def _check(prob, softplus=True, tol=None):
    say("bwd case B=%d D=%d N=%d L=%d io=%s" % (prob["batch"], prob["dim"], prob["dstate"], prob["seqlen"],
                                              prob["io"]))
    got = _gpu_grads(prob, softplus)
    ref = oracle.bwd(**oracle_args(prob), dy=f64(prob["dy"]), softplus=softplus)
    assert set(got) == set(ref), (sorted(got), sorted(ref))
    tol = tol or (GRAD_TOL if prob["io"] == "f32" else TOL[prob["io"]])
    errs = {k: rel_err(got[k], ref[k]) for k in ref}
    say("  errors " + " ".join("%s=%.2e" % kv for kv in sorted(errs.items())))
    for k, e in errs.items():
        assert e <= tol, (k, e)
    return got, ref


def test_config4_full():
    """Backward workload at full size (fp32, B=4, d_inner=1536, L=4097 -- not a multiple of 64)."""
    _check(inputs.make_config(4))


@pytest.mark.parametrize("over", [dict(seqlen=1), dict(dim=40)])
def test_config4_edges(over):
    """L = 1 and a channel count that leaves a partial workgroup."""
    _check(inputs.make_config(4, **over))


def test_finite_differences_slice():
    """First row, channels 0-3, steps 0-8 of the backward workload as its own problem:
    device gradients against central finite differences of the float64 forward."""
    prob = inputs.make_config(4, dim=8, seqlen=12)
    sl = dict(prob)
    for k in ("u", "delta", "z", "dy"):
        sl[k] = prob[k][:1, :4, :9].contiguous()
    for k in ("Bm", "Cm"):
        sl[k] = prob[k][:1, :, :9].contiguous()
    for k in ("A", "D", "bias"):
        sl[k] = prob[k][:4].contiguous()
    sl.update(batch=1, dim=4, seqlen=9)
    got = _gpu_grads(sl)
    base = {k: f64(sl[k]) for k in ("u", "delta", "z", "Bm", "Cm", "A", "D", "bias")}
    dy = f64(sl["dy"])

    def loss(**over):
        a = dict(base)
        a.update(over)
        y, _ = oracle.fwd(a["u"], a["delta"], a["A"], a["Bm"], a["Cm"], D=a["D"], z=a["z"], bias=a["bias"],
                          threads=1)
        return float(np.sum(dy * y))

    names = {"u": "du", "delta": "ddelta", "z": "dz", "Bm": "dB", "Cm": "dC", "A": "dA", "D": "dD", "bias": "dbias"}
    for name, gname in names.items():
        x = base[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            h = 1e-3 * max(1.0, abs(x[idx]))
            f = {}
            for kk in (-2, -1, 1, 2):
                q = x.copy()
                q[idx] += kk * h
                f[kk] = loss(**{name: q})
            fd[idx] = (8.0 * (f[1] - f[-1]) - (f[2] - f[-2])) / (12.0 * h)
        e = rel_err(got[gname], fd)
        say("  FD %s %.2e" % (gname, e))
        assert e <= GRAD_TOL, (gname, e)


@pytest.mark.parametrize("io", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("use_D,use_z,use_bias,softplus",
                         [(False, False, False, False), (True, False, True, True), (False, True, False, True),
                          (True, True, True, False), (True, True, True, True)])
def test_flag_matrix(io, use_D, use_z, use_bias, softplus):
    prob = inputs.make_problem(2, 40, 16, 200, io, seed=131, with_D=use_D, with_z=use_z, with_bias=use_bias,
                               with_dy=True)
    if not softplus:
        dl = prob["delta"].float().abs() * 0.05 + 0.01
        if use_bias:
            dl = dl - prob["bias"][None, :, None]
        prob["delta"] = dl.to(prob["delta"].dtype)
    _check(prob, softplus)


@pytest.mark.parametrize("Bsz,Dd,N,L", [(1, 1, 16, 1), (3, 17, 5, 63), (2, 33, 16, 64), (1, 16, 16, 65),
                                        (2, 20, 1, 130), (1, 64, 16, 1000)])
def test_edge_shapes(Bsz, Dd, N, L):
    _check(inputs.make_problem(Bsz, Dd, N, L, "f32", seed=7 * L + Dd, with_dy=True))


def test_max_seqlen():
    """The longest sequence the ABI accepts, L = 2^24, on one channel: 2^18 checkpoints,
    the reverse carry over 2^18 chunks and the dA/dD/dbias sums over all of them."""
    _check(inputs.make_problem(1, 1, 16, 1 << 24, "f32", seed=2425, with_dy=True))


def test_invariants_and_repeatability():
    """On device results: sum of ddelta over (b, t) equals dbias; u.du = dy.y per channel;
    two runs agree within the tolerance (channel sums use atomics)."""
    ss = _ss()
    prob = inputs.make_problem(3, 48, 16, 300, "f32", seed=141, with_dy=True)
    g1 = _gpu_grads(prob)
    g2 = _gpu_grads(prob)
    for k in g1:
        assert rel_err(g2[k], g1[k]) <= 1e-5, k
    assert np.allclose(g1["ddelta"].sum(axis=(0, 2)), g1["dbias"], rtol=1e-4, atol=1e-4 * np.abs(g1["dbias"]).max())
    g = to_dev(prob)
    y, _, _ = ss.fwd(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"])
    lhs = np.sum(f64(prob["u"]) * g1["du"], axis=2)
    rhs = np.sum(f64(prob["dy"]) * f64(y), axis=2)
    assert rel_err(lhs, rhs) <= 1e-4


def test_autograd_wrapper():
    """selective_scan_fn: forward through ss_fwd, backward through ss_bwd, against the oracle."""
    ss = _ss()
    prob = inputs.make_problem(2, 24, 16, 150, "f32", seed=151, with_dy=True)
    g = to_dev(prob)
    leaves = {k: g[k].clone().requires_grad_(True) for k in ("u", "delta", "A", "Bm", "Cm", "D", "z", "bias")}
    y = ss.selective_scan_fn(leaves["u"], leaves["delta"], leaves["A"], leaves["Bm"], leaves["Cm"], D=leaves["D"],
                             z=leaves["z"], delta_bias=leaves["bias"], delta_softplus=True)
    y.backward(g["dy"])
    ref = oracle.bwd(**oracle_args(prob), dy=f64(prob["dy"]))
    pairs = {"u": "du", "delta": "ddelta", "A": "dA", "Bm": "dB", "Cm": "dC", "D": "dD", "z": "dz", "bias": "dbias"}
    for leaf, gname in pairs.items():
        assert rel_err(f64(leaves[leaf].grad), ref[gname]) <= GRAD_TOL, gname
