"""Pins of the oracle's Mamba-2 SSD scan.

"Mamba" walkthrough, "Deep dive: Mamba-2 and state-space duality": A is a
scalar times the identity per head and heads share grouped B and C; the same
operator is both a linear recurrence and a masked quadratic attention.  The
recurrence in the oracle is checked against (a) the S6 oracle (a head of
headdim P is P channels with a shared Delta and A[d, n] = A_h), (b) the dual
quadratic form written out in numpy, (c) the packed-document identity and
prefill in pieces.  CPU only.
"""
import numpy as np
import pytest

import oracle
from mamba_selective_scan_fwd_amd import inputs


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _data(seed, Bsz=2, L=23, Hn=4, P=3, G=2, N=5):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((Bsz, L, Hn, P)), dt=rng.standard_normal((Bsz, L, Hn)),
                A=-rng.uniform(0.2, 2.0, Hn), Bm=rng.standard_normal((Bsz, L, G, N)),
                Cm=rng.standard_normal((Bsz, L, G, N)), D=rng.standard_normal(Hn),
                z=rng.standard_normal((Bsz, L, Hn, P)), dt_bias=rng.uniform(-2.0, 0.5, Hn))


@pytest.mark.parametrize("gate", [False, True])
def test_equals_s6_with_shared_delta_and_scalar_A(gate):
    q = _data(51)
    Bsz, L, Hn, P = q["x"].shape
    G, N = q["Bm"].shape[2], q["Bm"].shape[3]
    h0 = np.random.default_rng(52).standard_normal((Bsz, Hn, P, N))
    y, fin = oracle.ssd_fwd(q["x"], q["dt"], q["A"], q["Bm"], q["Cm"], D=q["D"], z=q["z"] if gate else None,
                            dt_bias=q["dt_bias"], h0=h0)
    hpg = Hn // G
    for g in range(G):
        heads = range(g * hpg, (g + 1) * hpg)
        # S6 channels d = (head, p) of this group
        u = np.stack([q["x"][:, :, h, p] for h in heads for p in range(P)], axis=1)       # (B, D, L)
        delta = np.stack([q["dt"][:, :, h] for h in heads for p in range(P)], axis=1)
        zz = np.stack([q["z"][:, :, h, p] for h in heads for p in range(P)], axis=1)
        A6 = np.array([[q["A"][h]] * N for h in heads for p in range(P)])
        D6 = np.array([q["D"][h] for h in heads for p in range(P)])
        b6 = np.array([q["dt_bias"][h] for h in heads for p in range(P)])
        h06 = np.stack([h0[:, h, p, :] for h in heads for p in range(P)], axis=1)         # (B, D, N)
        B6 = np.ascontiguousarray(q["Bm"][:, :, g, :].transpose(0, 2, 1))
        C6 = np.ascontiguousarray(q["Cm"][:, :, g, :].transpose(0, 2, 1))
        y6, last6 = oracle.fwd(u, delta, A6, B6, C6, D=D6, z=zz if gate else None, bias=b6, h0=h06, threads=1)
        k = 0
        for h in heads:
            for p in range(P):
                assert _rel(y[:, :, h, p], y6[:, k, :]) < 1e-13
                assert _rel(fin[:, h, p, :], last6[:, k, :]) < 1e-13
                k += 1


def test_equals_dual_quadratic_form():
    """y = (L o C B^T) (Delta x) + D x with L[t, s] = exp(A sum_{s<r<=t} Delta_r) for s <= t."""
    q = _data(53, L=17)
    Bsz, L, Hn, P = q["x"].shape
    G = q["Bm"].shape[2]
    y, _ = oracle.ssd_fwd(q["x"], q["dt"], q["A"], q["Bm"], q["Cm"], D=q["D"], dt_bias=q["dt_bias"])
    delta = np.logaddexp(0.0, q["dt"] + q["dt_bias"][None, None, :])     # softplus
    for b in range(Bsz):
        for h in range(Hn):
            g = h // (Hn // G)
            cs = np.cumsum(delta[b, :, h] * q["A"][h])
            CB = q["Cm"][b, :, g, :] @ q["Bm"][b, :, g, :].T                # (L, L)
            Lm = np.tril(np.exp(cs[:, None] - cs[None, :]))
            M = CB * Lm * delta[b, None, :, h]
            ref = M @ q["x"][b, :, h, :] + q["D"][h] * q["x"][b, :, h, :]
            assert _rel(y[b, :, h, :], ref) < 1e-12


@pytest.mark.parametrize("case", ["length1_docs", "tile_edges", "misaligned_rows", "many_short_docs"])
def test_packed_equals_documents(case):
    q = _data(54, L=140)
    seq = inputs.make_seq_idx(case, 2, 140, seed=55).numpy()
    y, fin = oracle.ssd_fwd(q["x"], q["dt"], q["A"], q["Bm"], q["Cm"], D=q["D"], z=q["z"], dt_bias=q["dt_bias"],
                            seq_idx=seq)
    for b in range(2):
        row = seq[b]
        cuts = [0] + [t for t in range(1, 140) if row[t] != row[t - 1]] + [140]
        for s0, s1 in zip(cuts[:-1], cuts[1:]):
            sl = lambda a: a[b:b + 1, s0:s1]
            yd, fd = oracle.ssd_fwd(sl(q["x"]), sl(q["dt"]), q["A"], sl(q["Bm"]), sl(q["Cm"]), D=q["D"],
                                    z=sl(q["z"]), dt_bias=q["dt_bias"])
            assert _rel(y[b:b + 1, s0:s1], yd) < 1e-13
        assert _rel(fin[b:b + 1], fd) < 1e-13


def test_prefill_in_pieces():
    q = _data(56, L=60)
    y, fin = oracle.ssd_fwd(q["x"], q["dt"], q["A"], q["Bm"], q["Cm"], D=q["D"], z=q["z"], dt_bias=q["dt_bias"])
    k = 37
    a = {n: (v[:, :k] if v.ndim > 1 and v.shape[1] == 60 else v) for n, v in q.items()}
    c = {n: (v[:, k:] if v.ndim > 1 and v.shape[1] == 60 else v) for n, v in q.items()}
    y1, f1 = oracle.ssd_fwd(a["x"], a["dt"], a["A"], a["Bm"], a["Cm"], D=a["D"], z=a["z"], dt_bias=a["dt_bias"])
    y2, f2 = oracle.ssd_fwd(c["x"], c["dt"], c["A"], c["Bm"], c["Cm"], D=c["D"], z=c["z"], dt_bias=c["dt_bias"],
                            h0=f1)
    assert _rel(np.concatenate([y1, y2], axis=1), y) < 1e-13
    assert _rel(f2, fin) < 1e-13
