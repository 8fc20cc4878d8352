"""Independent closed forms used to pin the oracle -- TEST INFRASTRUCTURE ONLY.

None of these share code with ``ss_oracle.c``; they compute the same
quantities from a different statement of the mathematics, so that a dropped
term, a wrong sign or an off-by-one in the recurrence shows up as a mismatch.
"""
import math

import numpy as np


def _softplus(x):
    # log(1 + e^x) for scalars, evaluated directly with the Python math library.
    return math.log1p(math.exp(x)) if x < 30 else x + math.log1p(math.exp(-x))


def unrolled_fwd(u, delta, A, Bm, Cm, D=None, z=None, bias=None, softplus=True, seq_idx=None, h0=None):
    """Unrolled (non-recursive) form of the selective scan, O(L^2 N) per channel.

    "Mamba" walkthrough, Part V "S6, and why selectivity forbids the
    convolution": the output at t is a weighted sum over all past inputs s,
    with weight C_t * Abar_t * ... * Abar_{s+1} * Bbar_s, where
    Abar_r = exp(Delta_r A) and Bbar_s = Delta_s B_s (Part IV Stage 4).
    An initial state h0 enters with weight C_t * Abar_t * ... * Abar_0.
    With document ids ("niverel-mamba" README, "seq_idx strict reset") a
    term reaches t only if no document starts in (s, t]: its weight is zero
    otherwise.  Pure-Python loops: tiny inputs only.
    """
    u = np.asarray(u, np.float64)
    Bsz, Dd, L = u.shape
    N = np.asarray(A).shape[1]
    y = np.zeros((Bsz, Dd, L))
    for b in range(Bsz):
        starts = set()
        if seq_idx is not None:
            starts = {r for r in range(1, L) if int(seq_idx[b][r]) != int(seq_idx[b][r - 1])}
        for d in range(Dd):
            dts = []
            for t in range(L):
                x = float(delta[b][d][t]) + (float(bias[d]) if bias is not None else 0.0)
                dts.append(_softplus(x) if softplus else x)
            for t in range(L):
                total = 0.0
                for n in range(N):
                    if h0 is not None and not any(r in starts for r in range(1, t + 1)):
                        w = float(Cm[b][n][t]) * float(h0[b][d][n])
                        for r in range(0, t + 1):
                            w *= math.exp(dts[r] * float(A[d][n]))
                        total += w
                    for s in range(t + 1):
                        if any(r in starts for r in range(s + 1, t + 1)):
                            continue
                        w = float(Cm[b][n][t])
                        for r in range(s + 1, t + 1):
                            w *= math.exp(dts[r] * float(A[d][n]))
                        w *= dts[s] * float(Bm[b][n][s])
                        total += w * float(u[b][d][s])
                if D is not None:
                    total += float(D[d]) * float(u[b][d][t])
                if z is not None:
                    zz = float(z[b][d][t])
                    total *= zz / (1.0 + math.exp(-zz))
                y[b, d, t] = total
    return y


def time_invariant_fwd(u, dt, A_d, B_vec, C_vec, D_d):
    """Time-invariant special case as a causal convolution (S4 view).

    "Mamba" walkthrough, Part V: with Delta, B and C fixed in time the map
    from u to y is a convolution with kernel K_k = C Abar^k Bbar (plus the
    skip D u).  One channel: u (L,), scalar dt, A_d/B_vec/C_vec (N,).
    Uses numpy's convolution, not a recurrence.
    """
    u = np.asarray(u, np.float64)
    L = u.shape[0]
    abar = np.exp(dt * np.asarray(A_d, np.float64))
    k = np.arange(L)[:, None]
    K = np.sum(np.asarray(C_vec)[None, :] * abar[None, :] ** k * dt * np.asarray(B_vec)[None, :], axis=1)
    return np.convolve(u, K)[:L] + D_d * u


def l1_closed_form(u, dt, A_d, B_vec, C_vec, D_d, z):
    """Single step from a zero state: h = Delta B u, y = (C.h + D u) SiLU(z)."""
    h = dt * np.asarray(B_vec, np.float64) * u
    y0 = float(np.dot(np.asarray(C_vec, np.float64), h)) + D_d * u
    return y0 * z / (1.0 + math.exp(-z)), h
