"""Shared helpers for the tests (comparison metrics, device transfer)."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from mamba_selective_scan_fwd_amd import inputs  # noqa: E402

# sealed tolerances: max|err| / max|ref| over the tensor
TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
GRAD_TOL = 1e-4


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in the device result"
    den = np.max(np.abs(ref))
    num = np.max(np.abs(got - ref))
    return float(num / den) if den > 0 else float(num)


def f64(t):
    return inputs.to_f64(t)


def to_dev(prob, keys=("u", "delta", "z", "Bm", "Cm", "A", "D", "bias", "lengths", "dy")):
    out = {}
    for k in keys:
        v = prob.get(k)
        out[k] = None if v is None else v.to("cuda")
    return out


def oracle_args(prob):
    return dict(u=f64(prob["u"]), delta=f64(prob["delta"]), A=f64(prob["A"]), Bm=f64(prob["Bm"]),
                Cm=f64(prob["Cm"]), D=f64(prob["D"]), z=f64(prob["z"]), bias=f64(prob["bias"]))


def sample_rows(batch, dim, k, seed=0, must=()):
    """k distinct flat channel indices b*dim+d (always including `must`)."""
    rng = np.random.default_rng(1000 + seed)
    total = batch * dim
    pick = set(int(x) for x in must)
    extra = rng.choice(total, size=min(k, total), replace=False)
    for x in extra:
        if len(pick) >= k:
            break
        pick.add(int(x))
    return np.array(sorted(pick), dtype=np.int64)


def say(msg):
    print(msg, flush=True)


def oracle_rows(prob, rows, softplus=True, states_every=None):
    """Oracle forward of the selected flat channels only (grouped by batch row, widened
    row by row so that large problems never materialise in float64).  Returns
    (y (k, L), last (k, N)[, states (k, K, N)]) in the order of `rows`."""
    import oracle
    Bsz, Dd, L = prob["u"].shape
    rows = np.asarray(rows, dtype=np.int64)
    N = prob["A"].shape[1]
    y = np.empty((rows.size, L))
    last = np.empty((rows.size, N))
    st = None
    if states_every:
        st = np.empty((rows.size, -(-L // states_every), N))
    for b in np.unique(rows // Dd):
        idx = np.nonzero(rows // Dd == b)[0]
        ds = torch.from_numpy(rows[idx] % Dd)
        sel = lambda t: None if t is None else f64(t[b:b + 1].index_select(1, ds))
        A = f64(prob["A"].index_select(0, ds))
        D = None if prob["D"] is None else f64(prob["D"].index_select(0, ds))
        bias = None if prob["bias"] is None else f64(prob["bias"].index_select(0, ds))
        lens = None if prob.get("lengths") is None else [int(prob["lengths"][b])]
        out = oracle.fwd(sel(prob["u"]), sel(prob["delta"]), A, f64(prob["Bm"][b:b + 1]), f64(prob["Cm"][b:b + 1]),
                         D=D, z=sel(prob["z"]), bias=bias, softplus=softplus, lengths=lens,
                         states_every=states_every)
        y[idx] = out[0][0]
        last[idx] = out[1][0]
        if st is not None:
            st[idx] = out[2][0]
    if st is not None:
        return y, last, st
    return y, last


def gather_rows(t, rows):
    """(B, D, ...) device/host tensor -> float64 numpy (k, ...) of the selected flat channels."""
    Bsz, Dd = t.shape[0], t.shape[1]
    flat = t.reshape(Bsz * Dd, *t.shape[2:])
    idx = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=t.device)
    return f64(flat.index_select(0, idx))


def full_compare(prob, y, last, softplus=True):
    """max|err| / max|ref| over the WHOLE y and last_state tensors of a device forward, against
    the oracle run one batch row at a time (so that only one row is ever widened to float64).
    Also returns the oracle's final state (B, D, N) for continuing with decode steps."""
    import oracle
    Bsz, Dd, L = prob["u"].shape
    N = prob["A"].shape[1]
    lengths = prob.get("lengths")
    ey = ry = el = rl = 0.0
    last_ref = np.empty((Bsz, Dd, N))
    for b in range(Bsz):
        sl = lambda t: None if t is None else f64(t[b:b + 1])
        lens = None if lengths is None else [int(lengths[b])]
        yr, lr = oracle.fwd(sl(prob["u"]), sl(prob["delta"]), f64(prob["A"]), sl(prob["Bm"]), sl(prob["Cm"]),
                            D=None if prob["D"] is None else f64(prob["D"]), z=sl(prob["z"]),
                            bias=None if prob["bias"] is None else f64(prob["bias"]), softplus=softplus,
                            lengths=lens)
        yg, lg = f64(y[b:b + 1]), f64(last[b:b + 1])
        assert np.all(np.isfinite(yg)) and np.all(np.isfinite(lg)), "non-finite values in the device result"
        ey = max(ey, float(np.max(np.abs(yg - yr))))
        ry = max(ry, float(np.max(np.abs(yr))))
        el = max(el, float(np.max(np.abs(lg - lr))))
        rl = max(rl, float(np.max(np.abs(lr))))
        last_ref[b] = lr[0]
    return ey / ry, el / rl, last_ref
