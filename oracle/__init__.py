"""Float64 CPU oracle for the Mamba selective scan (S6) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP product path never does, and
this package never imports the product.

The arithmetic lives in ``ss_oracle.c`` (plain sequential loops in double);
this module only marshals numpy float64 arrays into it.  ``brute.py`` holds
an independent O(L^2 N) unrolled form used to pin the oracle.

Every function takes the operands in the layouts of the problem statement
("Mamba" walkthrough, Part IV Stage 5): u, delta, z (B,D,L); A (D,N);
Bm, Cm (B,N,L); D, bias (D,).  Inputs must already be rounded to the I/O
precision the product sees; they are widened to float64 here.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        lib.sso_fwd.restype = ctypes.c_int
        lib.sso_fwd.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int,
                                _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _ip, _ip, _dp, _ip, _i64,
                                _dp, _dp, _dp, _i64, ctypes.c_int]
        lib.sso_step.restype = ctypes.c_int
        lib.sso_step.argtypes = [_i64, _i64, _i64, ctypes.c_int,
                                 _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.sso_bwd.restype = ctypes.c_int
        lib.sso_bwd.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int,
                                _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _ip, _ip, _dp, _dp, _dp,
                                _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int]
        lib.sso_conv1d_fwd.restype = ctypes.c_int
        lib.sso_conv1d_fwd.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, _dp, _dp, _dp, _ip, _dp, _dp, _dp]
        lib.sso_conv1d_step.restype = ctypes.c_int
        lib.sso_conv1d_step.argtypes = [_i64, _i64, _i64, ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.sso_ssd_fwd.restype = ctypes.c_int
        lib.sso_ssd_fwd.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                    _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _ip, _dp, _dp, _dp]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(x, shape=None):
    if x is None:
        return None
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError("oracle: expected shape %s, got %s" % (tuple(shape), a.shape))
    return a


def _ptr(a, typ=_dp):
    return None if a is None else a.ctypes.data_as(typ)


def _seq(seq_idx, Bsz, L):
    if seq_idx is None:
        return None
    a = np.ascontiguousarray(np.asarray(seq_idx, dtype=np.int64))
    if a.shape != (Bsz, L):
        raise ValueError("oracle: seq_idx must have shape %s" % ((Bsz, L),))
    return a


def fwd(u, delta, A, Bm, Cm, D=None, z=None, bias=None, softplus=True,
        lengths=None, h0=None, rows=None, states_every=None, threads=None, seq_idx=None):
    """Forward scan in float64.

    Returns ``(y, last_state)``, or ``(y, last_state, states)`` when
    ``states_every`` is given (states[b,d,k] = state after min(k*every, len_b)
    steps).  With ``rows`` (flat channel indices b*D+d) only those channels
    are computed; the other entries of y / last_state are NaN.  ``seq_idx``
    (B,L) integer document ids: the state restarts from zero wherever the id
    changes.
    """
    u = _f64(u)
    Bsz, Dd, L = u.shape
    A = _f64(A)
    N = A.shape[1]
    delta = _f64(delta, (Bsz, Dd, L))
    A = _f64(A, (Dd, N))
    Bm = _f64(Bm, (Bsz, N, L))
    Cm = _f64(Cm, (Bsz, N, L))
    D = _f64(D, (Dd,))
    z = _f64(z, (Bsz, Dd, L))
    bias = _f64(bias, (Dd,))
    h0 = _f64(h0, (Bsz, Dd, N))
    lens = None
    if lengths is not None:
        lens = np.ascontiguousarray(np.asarray(lengths, dtype=np.int64).reshape(Bsz))
    rws = None
    if rows is not None:
        rws = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
        if rws.size and (rws.min() < 0 or rws.max() >= Bsz * Dd):
            raise ValueError("oracle: row index out of range")
    y = np.full((Bsz, Dd, L), np.nan)
    last = np.full((Bsz, Dd, N), np.nan)
    states = None
    every = 0
    if states_every is not None:
        every = int(states_every)
        K = -(-L // every)
        states = np.full((Bsz, Dd, K, N), np.nan)
    seq = _seq(seq_idx, Bsz, L)
    rc = _load().sso_fwd(Bsz, Dd, N, L, int(bool(softplus)),
                         _ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(z),
                         _ptr(bias), _ptr(lens, _ip), _ptr(seq, _ip), _ptr(h0), _ptr(rws, _ip),
                         0 if rws is None else rws.size,
                         _ptr(y), _ptr(last), _ptr(states), every, threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle sso_fwd failed (%d)" % rc)
    if states is not None:
        return y, last, states
    return y, last


def step(u_t, delta_t, A, B_t, C_t, state_in, D=None, z_t=None, bias=None, softplus=True):
    """One decode step from ``state_in``; returns ``(y_t, state_out)``.

    u_t, delta_t, z_t: (B,D); B_t, C_t: (B,N); state_in: (B,D,N).
    """
    u_t = _f64(u_t)
    Bsz, Dd = u_t.shape
    A = _f64(A)
    N = A.shape[1]
    delta_t = _f64(delta_t, (Bsz, Dd))
    B_t = _f64(B_t, (Bsz, N))
    C_t = _f64(C_t, (Bsz, N))
    D = _f64(D, (Dd,))
    z_t = _f64(z_t, (Bsz, Dd))
    bias = _f64(bias, (Dd,))
    state_in = _f64(state_in, (Bsz, Dd, N))
    state_out = np.empty((Bsz, Dd, N))
    y_t = np.empty((Bsz, Dd))
    rc = _load().sso_step(Bsz, Dd, N, int(bool(softplus)), _ptr(u_t), _ptr(delta_t), _ptr(A),
                          _ptr(B_t), _ptr(C_t), _ptr(D), _ptr(z_t), _ptr(bias), _ptr(state_in),
                          _ptr(state_out), _ptr(y_t))
    if rc != 0:
        raise RuntimeError("oracle sso_step failed (%d)" % rc)
    return y_t, state_out


def bwd(u, delta, A, Bm, Cm, dy, D=None, z=None, bias=None, softplus=True,
        lengths=None, h0=None, threads=None, seq_idx=None, dlast=None, want_dh0=False):
    """Backward scan for the loss sum(dy * out) + sum(dlast * h_final), in float64.

    Returns a dict with du, ddelta, dA, dB, dC and, when the matching input
    is given, dz, dD, dbias; with ``want_dh0`` also dh0, the gradient w.r.t.
    the initial state (B,D,N).
    """
    u = _f64(u)
    Bsz, Dd, L = u.shape
    A = _f64(A)
    N = A.shape[1]
    delta = _f64(delta, (Bsz, Dd, L))
    A = _f64(A, (Dd, N))
    Bm = _f64(Bm, (Bsz, N, L))
    Cm = _f64(Cm, (Bsz, N, L))
    dy = _f64(dy, (Bsz, Dd, L))
    D = _f64(D, (Dd,))
    z = _f64(z, (Bsz, Dd, L))
    bias = _f64(bias, (Dd,))
    h0 = _f64(h0, (Bsz, Dd, N))
    lens = None
    if lengths is not None:
        lens = np.ascontiguousarray(np.asarray(lengths, dtype=np.int64).reshape(Bsz))
    out = {
        "du": np.empty((Bsz, Dd, L)), "ddelta": np.empty((Bsz, Dd, L)),
        "dA": np.empty((Dd, N)), "dB": np.empty((Bsz, N, L)), "dC": np.empty((Bsz, N, L)),
    }
    out["dz"] = np.empty((Bsz, Dd, L)) if z is not None else None
    out["dD"] = np.empty((Dd,)) if D is not None else None
    out["dbias"] = np.empty((Dd,)) if bias is not None else None
    out["dh0"] = np.empty((Bsz, Dd, N)) if want_dh0 else None
    seq = _seq(seq_idx, Bsz, L)
    dlast = _f64(dlast, (Bsz, Dd, N))
    rc = _load().sso_bwd(Bsz, Dd, N, L, int(bool(softplus)),
                         _ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(z),
                         _ptr(bias), _ptr(lens, _ip), _ptr(seq, _ip), _ptr(h0), _ptr(dy), _ptr(dlast),
                         _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dz"]), _ptr(out["dA"]),
                         _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dbias"]),
                         _ptr(out["dh0"]), threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle sso_bwd failed (%d)" % rc)
    return {k: v for k, v in out.items() if v is not None}


def conv1d_fwd(x, w, bias=None, silu=True, seq_idx=None, conv_init=None):
    """Depthwise causal conv1d (+ SiLU) in float64.  x (B,D,L), w (D,W), bias (D,),
    seq_idx (B,L), conv_init (B,D,W-1).  Returns (out (B,D,L), conv_final (B,D,W-1))."""
    x = _f64(x)
    Bsz, Dd, L = x.shape
    w = _f64(w)
    W = w.shape[1]
    w = _f64(w, (Dd, W))
    bias = _f64(bias, (Dd,))
    conv_init = _f64(conv_init, (Bsz, Dd, W - 1))
    seq = _seq(seq_idx, Bsz, L)
    out = np.empty((Bsz, Dd, L))
    fin = np.empty((Bsz, Dd, W - 1))
    rc = _load().sso_conv1d_fwd(Bsz, Dd, L, W, int(bool(silu)), _ptr(x), _ptr(w), _ptr(bias), _ptr(seq, _ip),
                                _ptr(conv_init), _ptr(out), _ptr(fin))
    if rc != 0:
        raise RuntimeError("oracle sso_conv1d_fwd failed (%d)" % rc)
    return out, fin


def conv1d_step(x_t, w, window, bias=None, silu=True):
    """One decode step of the convolution.  x_t (B,D), window (B,D,W-1).
    Returns (out_t (B,D), new window (B,D,W-1))."""
    x_t = _f64(x_t)
    Bsz, Dd = x_t.shape
    w = _f64(w)
    W = w.shape[1]
    window = _f64(window, (Bsz, Dd, W - 1))
    bias = _f64(bias, (Dd,))
    out = np.empty((Bsz, Dd))
    win = np.empty((Bsz, Dd, W - 1))
    rc = _load().sso_conv1d_step(Bsz, Dd, W, int(bool(silu)), _ptr(x_t), _ptr(w), _ptr(bias), _ptr(window),
                                 _ptr(win), _ptr(out))
    if rc != 0:
        raise RuntimeError("oracle sso_conv1d_step failed (%d)" % rc)
    return out, win


def ssd_fwd(x, dt, A, Bm, Cm, D=None, z=None, dt_bias=None, softplus=True, seq_idx=None, h0=None):
    """Mamba-2 SSD scan in float64 (plain recurrence).  x, z: (B,L,H,P); dt: (B,L,H);
    A, D, dt_bias: (H,); Bm, Cm: (B,L,G,N); seq_idx: (B,L); h0: (B,H,P,N).
    Returns (y (B,L,H,P), final_state (B,H,P,N))."""
    x = _f64(x)
    Bsz, L, Hn, P = x.shape
    Bm = _f64(Bm)
    G, N = Bm.shape[2], Bm.shape[3]
    dt = _f64(dt, (Bsz, L, Hn))
    A = _f64(A, (Hn,))
    Bm = _f64(Bm, (Bsz, L, G, N))
    Cm = _f64(Cm, (Bsz, L, G, N))
    D = _f64(D, (Hn,))
    z = _f64(z, (Bsz, L, Hn, P))
    dt_bias = _f64(dt_bias, (Hn,))
    h0 = _f64(h0, (Bsz, Hn, P, N))
    seq = _seq(seq_idx, Bsz, L)
    y = np.empty((Bsz, L, Hn, P))
    fin = np.empty((Bsz, Hn, P, N))
    rc = _load().sso_ssd_fwd(Bsz, L, Hn, P, G, N, int(bool(softplus)), _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm),
                             _ptr(Cm), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(seq, _ip), _ptr(h0), _ptr(y), _ptr(fin))
    if rc != 0:
        raise RuntimeError("oracle sso_ssd_fwd failed (%d)" % rc)
    return y, fin
