"""Host-side checks of the C ABI (no GPU): the library loads, exports every symbol
declared in include/ss.h, and rejects invalid arguments before any HIP call."""
import ctypes
import os
import re

import pytest

from mamba_selective_scan_fwd_amd import ss

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "ss.h")).read()
    return sorted(set(re.findall(r"^\s*(?:ss_status|size_t|const char \*)\s*(ss_\w+)\s*\(", text, re.M)))


def test_header_symbols_exported():
    lib = ss.load_library()
    names = _declared_symbols()
    assert set(names) >= {"ss_fwd", "ss_fwd_step", "ss_bwd", "ss_ckpt_count", "ss_status_str"}
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(ss.EXPORTS)


def _prob(**kw):
    d = dict(batch=2, dim=3, dstate=16, seqlen=10, io_dtype=0, delta_softplus=1)
    d.update(kw)
    return ss.ss_problem(d["batch"], d["dim"], d["dstate"], d["seqlen"], d["io_dtype"], d["delta_softplus"])


FAKE = 1 << 20  # aligned host-side stand-in address; never dereferenced (validation fails first)


def _fwd(p, **ptrs):
    lib = ss.load_library()
    args = dict(u=FAKE, delta=FAKE, A=FAKE, Bm=FAKE, Cm=FAKE, D=None, z=None, bias=None, lengths=None,
                seq_idx=None, h0=None, y=FAKE, last=None, ckpt=None, ws=None)
    args.update(ptrs)
    order = ["u", "delta", "A", "Bm", "Cm", "D", "z", "bias", "lengths", "seq_idx", "h0", "y", "last", "ckpt", "ws"]
    return lib.ss_fwd(ctypes.byref(p), *[args[k] for k in order], 0, None)


def test_status_strings():
    lib = ss.load_library()
    for code in range(7):
        assert lib.ss_status_str(code)
    assert b"unknown" in lib.ss_status_str(99)


def test_sizes():
    lib = ss.load_library()
    p = _prob(batch=8, dim=1536, seqlen=2048)
    assert lib.ss_ckpt_count(ctypes.byref(p)) == 8 * 1536 * 32 * 16
    assert lib.ss_fwd_workspace_min(ctypes.byref(p)) == 0    # enough channels: no time split
    # the optional work queue: control block, a flag per (row block, 2048-step unit), a state per
    # (channel, unit)
    q = 256 + ((8 * 96 * 1 * 4 + 255) // 256) * 256 + 8 * 1536 * 1 * 16 * 4
    assert lib.ss_fwd_workspace_size(ctypes.byref(p)) == q
    p1 = _prob(batch=1, dim=16, seqlen=32768)
    assert lib.ss_fwd_workspace_min(ctypes.byref(p1)) > 0    # few channels: time-chunked
    assert lib.ss_fwd_workspace_size(ctypes.byref(p1)) == lib.ss_fwd_workspace_min(ctypes.byref(p1))
    big = _prob(batch=257, dim=1536, seqlen=2048)                # too many rows for the queue
    assert lib.ss_fwd_workspace_size(ctypes.byref(big)) == 0
    p4 = _prob(batch=4, dim=1536, seqlen=4097)
    assert lib.ss_bwd_workspace_size(ctypes.byref(p4)) == 3 * 4 * 1536 * 65 * 16 * 4
    assert lib.ss_ckpt_count(ctypes.byref(_prob(seqlen=0))) == 0


def test_bwd_rejects_grids_beyond_the_dispatch_limit():
    """A backward whose per-chunk grid (batch x 64-step chunks x channel blocks) or carry grid
    (one workgroup per channel) would pass 2^23 workgroups is rejected on the host."""
    lib = ss.load_library()
    args = [FAKE] * 5 + [None, None, None] + [None, FAKE, FAKE, None] + [FAKE, FAKE, None] + [FAKE] * 3 + [None] * 3
    for p in (_prob(batch=1 << 20, dim=16, seqlen=1 << 14),      # 2^28 chunk workgroups
              _prob(batch=1 << 12, dim=1 << 12, seqlen=65)):      # 2^24 channels for the carry scan
        assert lib.ss_bwd_workspace_size(ctypes.byref(p)) == 0
        assert lib.ss_bwd(ctypes.byref(p), *args, FAKE, 1 << 30, None) == 2
    for ok in (_prob(batch=4, dim=1536, seqlen=4097), _prob(batch=1 << 12, dim=1 << 12, seqlen=64)):
        assert lib.ss_bwd_workspace_size(ctypes.byref(ok)) > 0

def test_channel_limit_is_exact():
    """batch * dim is bounded at 2^26 - 8 (one workgroup per 16 channels, twice over, within
    2^23 - 1 workgroups): the last accepted and the first rejected count, in both factors; the
    decode step's 32-bit channel indices rely on it."""
    lib = ss.load_library()
    lim = (1 << 26) - 8
    assert lib.ss_ckpt_count(ctypes.byref(_prob(batch=1, dim=lim, seqlen=1))) == lim * 16
    assert lib.ss_ckpt_count(ctypes.byref(_prob(batch=lim // 8, dim=8, seqlen=1))) == lim * 16
    assert lib.ss_ckpt_count(ctypes.byref(_prob(batch=1, dim=lim + 1, seqlen=1))) == 0
    assert lib.ss_ckpt_count(ctypes.byref(_prob(batch=(lim + 8) // 8, dim=8, seqlen=1))) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), 2), (dict(dim=-1), 2), (dict(seqlen=0), 2), (dict(seqlen=(1 << 24) + 1), 2),
    (dict(dstate=0), 2), (dict(dstate=17), 5), (dict(io_dtype=3), 3)])
def test_fwd_rejects_bad_problem(kw, code):
    assert _fwd(_prob(**kw)) == code


def test_fwd_rejects_null_and_misaligned():
    p = _prob()
    assert _fwd(p, u=None) == 1
    assert _fwd(p, y=None) == 1
    assert _fwd(p, Bm=FAKE + 4) == 4
    assert _fwd(p, D=FAKE + 8) == 4
    assert _fwd(p, seq_idx=FAKE + 4) == 4
    assert _fwd(p, h0=FAKE + 12) == 4
    # a time-chunked problem without its workspace
    assert _fwd(_prob(batch=1, dim=16, seqlen=32768)) == 5
    lib = ss.load_library()
    assert lib.ss_fwd(None, *([FAKE] * 14), None, 0, None) == 1


def test_step_and_bwd_validation():
    lib = ss.load_library()
    p = _prob()
    assert lib.ss_fwd_step(ctypes.byref(p), *([FAKE] * 5), None, None, None, None, FAKE, FAKE, None) == 1
    # partial overlap of state_in/state_out
    assert lib.ss_fwd_step(ctypes.byref(p), *([FAKE] * 5), None, None, None, FAKE, FAKE + 16, FAKE, None) == 5
    # argument order after the problem: u delta A Bm Cm | D z bias | seq_idx ckpt dy dlast |
    # du ddelta dz | dA dB dC dD dbias dh0
    # dz without z
    args = [FAKE] * 5 + [None, None, None] + [None, FAKE, FAKE, None] + [FAKE, FAKE, FAKE] + [FAKE] * 3 + [None] * 3
    assert lib.ss_bwd(ctypes.byref(p), *args, FAKE, 1 << 30, None) == 1
    # missing workspace
    args = [FAKE] * 5 + [None, None, None] + [None, FAKE, FAKE, None] + [FAKE, FAKE, None] + [FAKE] * 3 + [None] * 3
    assert lib.ss_bwd(ctypes.byref(p), *args, None, 0, None) == 5
    # misaligned document ids, final-state gradient, initial-state gradient
    for k in (8, 11, 20):
        bad = list(args)
        bad[k] = FAKE + 4
        assert lib.ss_bwd(ctypes.byref(p), *bad, FAKE, 1 << 30, None) == 4
    assert lib.ss_copy_probe(FAKE, FAKE, 15, None) == 2


def test_alu_probe_rejects_bad_arguments():
    lib = ss.load_library()
    assert lib.ss_alu_probe(0, 4, 16, 0, None, None) == 1          # no output
    assert lib.ss_alu_probe(0, 4, 16, 0, FAKE + 8, None) == 4      # misaligned output
    assert lib.ss_alu_probe(4, 4, 16, 0, FAKE, None) == 5          # unknown kind
    assert lib.ss_alu_probe(-1, 4, 16, 0, FAKE, None) == 5
    assert lib.ss_alu_probe(0, 0, 16, 0, FAKE, None) == 2          # empty grid
    assert lib.ss_alu_probe(0, (1 << 20) + 1, 16, 0, FAKE, None) == 2
    assert lib.ss_alu_probe(0, 4, 0, 0, FAKE, None) == 2           # no iterations
    assert lib.ss_alu_probe(0, 4, (1 << 20) + 1, 0, FAKE, None) == 2
    assert lib.ss_alu_probe(0, 4, 16, -1, FAKE, None) == 2         # LDS outside 0..65536
    assert lib.ss_alu_probe(0, 4, 16, 65537, FAKE, None) == 2


def _conv_prob(**kw):
    d = dict(batch=2, dim=3, seqlen=10, width=4, io_dtype=0, silu=1, reserved=0)
    d.update(kw)
    return ss.ss_conv_problem(d["batch"], d["dim"], d["seqlen"], d["width"], d["io_dtype"], d["silu"], d["reserved"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), 2), (dict(seqlen=0), 2), (dict(width=0), 5), (dict(width=5), 5), (dict(io_dtype=7), 3),
    (dict(reserved=1), 5)])
def test_conv_rejects_bad_problem(kw, code):
    lib = ss.load_library()
    assert lib.ss_conv1d_fwd(ctypes.byref(_conv_prob(**kw)), FAKE, FAKE, None, None, None, FAKE * 2, None,
                             None) == code


def test_conv_rejects_null_misaligned_and_overlap():
    lib = ss.load_library()
    p = _conv_prob()
    assert lib.ss_conv1d_fwd(ctypes.byref(p), None, FAKE, None, None, None, FAKE * 2, None, None) == 1
    assert lib.ss_conv1d_fwd(ctypes.byref(p), FAKE, FAKE + 4, None, None, None, FAKE * 2, None, None) == 4
    assert lib.ss_conv1d_fwd(ctypes.byref(p), FAKE, FAKE, None, FAKE + 8, None, FAKE * 2, None, None) == 4
    # out overlapping x (in place is a race between neighbouring taps)
    assert lib.ss_conv1d_fwd(ctypes.byref(p), FAKE, FAKE, None, None, None, FAKE + 16, None, None) == 5
    assert lib.ss_conv1d_step(ctypes.byref(p), FAKE, FAKE, None, None, FAKE, FAKE, None) == 1
    # partial overlap of the two windows
    assert lib.ss_conv1d_step(ctypes.byref(p), FAKE, FAKE, None, FAKE * 2, FAKE * 2 + 16, FAKE * 3, None) == 5


def _ssd_prob(**kw):
    d = dict(batch=2, seqlen=300, nheads=4, ngroups=2, headdim=64, dstate=64, io_dtype=2, dt_softplus=1)
    d.update(kw)
    return ss.ss_ssd_problem(d["batch"], d["seqlen"], d["nheads"], d["ngroups"], d["headdim"], d["dstate"],
                             d["io_dtype"], d["dt_softplus"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), 2), (dict(seqlen=0), 2), (dict(io_dtype=0), 3), (dict(headdim=32), 5), (dict(dstate=16), 5),
    (dict(dstate=80), 5), (dict(ngroups=3), 5)])
def test_ssd_rejects_bad_problem(kw, code):
    lib = ss.load_library()
    p = _ssd_prob(**kw)
    assert lib.ss_ssd_workspace_size(ctypes.byref(p)) == 0
    assert lib.ss_ssd_fwd(ctypes.byref(p), *([FAKE] * 5), None, None, None, None, None, FAKE, None, FAKE, 1 << 30,
                          None) == code


def test_ssd_workspace_and_validation():
    lib = ss.load_library()
    p = _ssd_prob()
    wsz = lib.ss_ssd_workspace_size(ctypes.byref(p))
    # 2 chunks of 256 steps x 2 rows x 4 heads: entry states (64 x 64) 16-bit;
    # 2 chunks x 2 rows x 2 groups: C B^T (256 x 256) bf16
    assert p.ngroups == 2
    assert wsz == 16 * 4096 * 2 + 8 * 256 * 256 * 2
    assert lib.ss_ssd_fwd(ctypes.byref(p), *([FAKE] * 5), None, None, None, None, None, FAKE, None, FAKE, wsz - 1,
                          None) == 5
    assert lib.ss_ssd_fwd(ctypes.byref(p), None, *([FAKE] * 4), None, None, None, None, None, FAKE, None, FAKE, wsz,
                          None) == 1
    assert lib.ss_ssd_fwd(ctypes.byref(p), *([FAKE] * 5), None, None, None, None, FAKE + 4, FAKE, None, FAKE, wsz,
                          None) == 4   # h0 misaligned
    assert lib.ss_ssd_fwd(ctypes.byref(p), *([FAKE] * 5), None, None, None, FAKE + 4, None, FAKE, None, FAKE, wsz,
                          None) == 4   # document ids misaligned
    long_row = _ssd_prob(batch=1, nheads=2, ngroups=2, seqlen=(1 << 29) + 1)
    wl = lib.ss_ssd_workspace_size(ctypes.byref(long_row))
    assert wl > 0
    assert lib.ss_ssd_fwd(ctypes.byref(long_row), *([FAKE] * 5), None, None, None, FAKE, None, FAKE, None, FAKE, wl,
                          None) == 5   # document ids on a row past 2^29 steps


def test_ssd_rejects_overlapping_buffers():
    """Outputs and workspace may not overlap other operands (y may only be x or z itself,
    final_state only h0 itself).  Every case returns before any HIP call."""
    lib = ss.load_library()
    p = _ssd_prob()
    wsz = lib.ss_ssd_workspace_size(ctypes.byref(p))
    G = 1 << 32                                   # far-apart, aligned fake device addresses
    x, dt, A, Bm, Cm, y, fin, ws, h0, seq = (G * k for k in range(1, 11))

    def call(**kw):
        a = dict(x=x, dt=dt, A=A, Bm=Bm, Cm=Cm, D=None, z=None, dt_bias=None, seq=seq, h0=h0, y=y, fin=fin, ws=ws)
        a.update(kw)
        return lib.ss_ssd_fwd(ctypes.byref(p), a["x"], a["dt"], a["A"], a["Bm"], a["Cm"], a["D"], a["z"],
                              a["dt_bias"], a["seq"], a["h0"], a["y"], a["fin"], a["ws"], wsz, None)

    assert call(y=Cm + 256) == 5          # y overlaps C
    assert call(y=Bm) == 5                # y is B
    assert call(y=x + 256) == 5           # y partly overlaps x
    assert call(fin=y + 4096) == 5        # final state inside y
    assert call(fin=dt) == 5              # final state is dt
    assert call(ws=x + 1024) == 5         # workspace overlaps x
    assert call(ws=h0) == 5               # workspace is h0
    assert call(h0=fin + 256) == 5        # h0 partly overlaps the final state
    assert call(y=seq) == 5               # y is the document ids
    assert call(ws=seq + 64) == 5         # workspace overlaps the document ids


def test_fwd_bwd_reject_overlapping_buffers():
    """ss_fwd: y may only be u, delta or z itself, other outputs overlap nothing; ss_bwd: no
    output or workspace overlaps any buffer.  Every case returns before any HIP call."""
    lib = ss.load_library()
    p = _prob(batch=2, dim=40, seqlen=300)
    G = 1 << 32
    u, dl, A, Bm, Cm, y, last, ck, h0 = (G * k for k in range(1, 10))
    assert _fwd(p, u=u, delta=dl, A=A, Bm=Bm, Cm=Cm, y=Bm) == 5              # y is B
    assert _fwd(p, u=u, delta=dl, A=A, Bm=Bm, Cm=Cm, y=u + 16) == 5          # y partly overlaps u
    assert _fwd(p, u=u, delta=dl, A=A, Bm=Bm, Cm=Cm, y=y, h0=h0, last=h0) == 5   # final state over h0
    assert _fwd(p, u=u, delta=dl, A=A, Bm=Bm, Cm=Cm, y=y, ckpt=y + 64) == 5  # checkpoints inside y
    wsz = lib.ss_bwd_workspace_size(ctypes.byref(p))
    names = ["u", "delta", "A", "Bm", "Cm", "D", "z", "bias", "seq_idx", "ckpt", "dy", "dlast", "du", "ddelta",
             "dz", "dA", "dB", "dC", "dD", "dbias", "dh0", "ws"]
    base = dict(zip(names, [G * (k + 1) for k in range(len(names))]))
    for opt in ("D", "z", "bias", "seq_idx", "dlast", "dz", "dD", "dbias", "dh0"):
        base[opt] = None

    def bwd(**kw):
        a = dict(base)
        a.update(kw)
        return lib.ss_bwd(ctypes.byref(p), *[a[k] for k in names], wsz, None)

    assert bwd(du=base["u"]) == 5                  # no in-place gradient
    assert bwd(dC=base["dB"] + 64) == 5            # dB and dC overlap
    assert bwd(ws=base["dy"] + 1024) == 5          # workspace overlaps dy
    assert bwd(dA=base["A"]) == 5                  # dA over A


def test_conv_rejects_overlapping_outputs():
    """The window going out may not be the window coming in, nor overlap x or out."""
    lib = ss.load_library()
    p = ss.ss_conv_problem(2, 40, 300, 4, 0, 1, 0)
    G = 1 << 32
    x, w, out, win_in, win_out = (G * k for k in range(1, 6))
    f = lambda **kw: lib.ss_conv1d_fwd(ctypes.byref(p), kw.get("x", x), w, None, None, kw.get("init", win_in),
                                       kw.get("out", out), kw.get("final", win_out), None)
    assert f(final=win_in) == 5          # in place: rejected (first and last time blocks race)
    assert f(final=out + 256) == 5       # final window inside out
    assert f(final=x) == 5               # final window over x
    assert f(out=x + 4096) == 5          # out partly over x

