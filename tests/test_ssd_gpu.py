"""GPU parity of ss_ssd_fwd (the Mamba-2 SSD chunked scan on the matrix cores) against
the float64 oracle's plain recurrence, through the C ABI.  16-bit data with fp32
accumulation: the fp16/bf16 tolerance (2e-2 of max|y|) applies."""
import numpy as np
import pytest
import torch

import oracle
from _util import TOL, f64, inputs, rel_err, say

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _ss():
    from mamba_selective_scan_fwd_amd import ss
    ss.load_library()
    return ss


def _data(Bsz, L, Hn, G, N, io, seed, P=64):
    rng = np.random.default_rng(seed)
    t = lambda a: torch.from_numpy(a).to(DT[io])
    dt0 = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), Hn))
    return dict(x=t(rng.standard_normal((Bsz, L, Hn, P))), dt=t(rng.standard_normal((Bsz, L, Hn)) * 0.5),
                A=torch.from_numpy(-np.exp(rng.uniform(0.0, np.log(16.0), Hn))).float(),
                Bm=t(rng.standard_normal((Bsz, L, G, N))), Cm=t(rng.standard_normal((Bsz, L, G, N))),
                D=torch.from_numpy(rng.standard_normal(Hn)).float(), z=t(rng.standard_normal((Bsz, L, Hn, P))),
                dt_bias=torch.from_numpy(np.log(np.expm1(dt0))).float(),
                h0=torch.from_numpy(rng.standard_normal((Bsz, Hn, P, N)) * 0.5).float())


def _run(q, use=("D", "z", "dt_bias", "h0")):
    ss = _ss()
    g = {k: v.cuda() for k, v in q.items()}
    y, fin = ss.ssd_fwd(g["x"], g["dt"], g["A"], g["Bm"], g["Cm"], D=g["D"] if "D" in use else None,
                        z=g["z"] if "z" in use else None, dt_bias=g["dt_bias"] if "dt_bias" in use else None,
                        h0=g["h0"] if "h0" in use else None, return_final_state=True)
    torch.cuda.synchronize()
    return y, fin


def _ref(q, use=("D", "z", "dt_bias", "h0"), heads=None):
    sel = (lambda a, ax: a) if heads is None else (lambda a, ax: a.index_select(ax, torch.as_tensor(heads)))
    return oracle.ssd_fwd(f64(sel(q["x"], 2)), f64(sel(q["dt"], 2)), f64(sel(q["A"], 0)), f64(q["Bm"]), f64(q["Cm"]),
                          D=f64(sel(q["D"], 0)) if "D" in use else None, z=f64(sel(q["z"], 2)) if "z" in use else None,
                          dt_bias=f64(sel(q["dt_bias"], 0)) if "dt_bias" in use else None,
                          h0=f64(sel(q["h0"], 1)) if "h0" in use else None)


@pytest.mark.parametrize("io", ["bf16", "f16"])
@pytest.mark.parametrize("N", [32, 64, 96, 128])
def test_state_sizes_and_dtypes(io, N):
    say("ssd io=%s N=%d" % (io, N))
    q = _data(2, 300, 4, 2, N, io, seed=N)
    y, fin = _run(q)
    yr, fr = _ref(q)
    ey, ef = rel_err(f64(y), yr), rel_err(f64(fin), fr)
    say("  errors y=%.2e final=%.2e" % (ey, ef))
    assert ey <= TOL[io] and ef <= TOL[io]


@pytest.mark.parametrize("L", [1, 2, 100, 255, 256, 257, 512, 777])
def test_lengths(L):
    q = _data(1, L, 2, 1, 64, "bf16", seed=L)
    y, fin = _run(q)
    yr, fr = _ref(q)
    assert rel_err(f64(y), yr) <= TOL["bf16"] and rel_err(f64(fin), fr) <= TOL["bf16"]


@pytest.mark.parametrize("use", [(), ("D",), ("z",), ("dt_bias",), ("h0",), ("D", "z", "dt_bias", "h0")])
def test_optional_operands(use):
    q = _data(2, 400, 4, 4, 64, "bf16", seed=7)
    y, fin = _run(q, use)
    yr, fr = _ref(q, use)
    assert rel_err(f64(y), yr) <= TOL["bf16"] and rel_err(f64(fin), fr) <= TOL["bf16"]


def test_softplus_off():
    ss = _ss()
    q = _data(1, 300, 2, 1, 64, "bf16", seed=8)
    q["dt"] = (q["dt"].float().abs() * 0.05 + 0.001).to(torch.bfloat16)   # a positive Delta, used as given
    g = {k: v.cuda() for k, v in q.items()}
    y = ss.ssd_fwd(g["x"], g["dt"], g["A"], g["Bm"], g["Cm"], D=g["D"], dt_softplus=False)
    torch.cuda.synchronize()
    yr, _ = oracle.ssd_fwd(f64(q["x"]), f64(q["dt"]), f64(q["A"]), f64(q["Bm"]), f64(q["Cm"]), D=f64(q["D"]),
                           softplus=False)
    assert rel_err(f64(y), yr) <= TOL["bf16"]


def test_prefill_in_pieces():
    """ssd(x[:k]) -> final state -> ssd(x[k:], h0=final) == ssd(x), on the device."""
    ss = _ss()
    q = _data(2, 900, 4, 2, 64, "bf16", seed=9)
    g = {k: v.cuda() for k, v in q.items()}
    y, fin = ss.ssd_fwd(g["x"], g["dt"], g["A"], g["Bm"], g["Cm"], D=g["D"], dt_bias=g["dt_bias"],
                        return_final_state=True)
    k = 300
    a = lambda t: t[:, :k].contiguous()
    c = lambda t: t[:, k:].contiguous()
    y1, f1 = ss.ssd_fwd(a(g["x"]), a(g["dt"]), g["A"], a(g["Bm"]), a(g["Cm"]), D=g["D"], dt_bias=g["dt_bias"],
                        return_final_state=True)
    y2, f2 = ss.ssd_fwd(c(g["x"]), c(g["dt"]), g["A"], c(g["Bm"]), c(g["Cm"]), D=g["D"], dt_bias=g["dt_bias"],
                        h0=f1, return_final_state=True)
    torch.cuda.synchronize()
    assert rel_err(f64(torch.cat([y1, y2], dim=1)), f64(y)) <= TOL["bf16"]
    assert rel_err(f64(f2), f64(fin)) <= TOL["bf16"]


def test_long_sequence_many_chunks():
    """64 chunks of 256 steps walked in order by the state kernel, with few waves per group
    (2 heads x 2 state slices), so the C B^T tiles are shared out in turns."""
    q = _data(1, 16384, 2, 1, 64, "bf16", seed=14)
    y, fin = _run(q)
    yr, fr = _ref(q)
    assert rel_err(f64(y), yr) <= TOL["bf16"] and rel_err(f64(fin), fr) <= TOL["bf16"]


def test_in_place_output():
    """y written over x (and, separately, over z) gives the out-of-place result bit for bit."""
    ss = _ss()
    q = _data(2, 600, 4, 2, 64, "bf16", seed=15)
    g = {k: v.cuda() for k, v in q.items()}
    kw = dict(D=g["D"], dt_bias=g["dt_bias"], h0=g["h0"])
    y = ss.ssd_fwd(g["x"], g["dt"], g["A"], g["Bm"], g["Cm"], z=g["z"], **kw)
    xi = g["x"].clone()
    ss.ssd_fwd(xi, g["dt"], g["A"], g["Bm"], g["Cm"], z=g["z"], y=xi, **kw)
    zi = g["z"].clone()
    ss.ssd_fwd(g["x"], g["dt"], g["A"], g["Bm"], g["Cm"], z=zi, y=zi, **kw)
    torch.cuda.synchronize()
    assert torch.equal(xi, y) and torch.equal(zi, y)


def test_workspace_contents_do_not_matter():
    """A workspace full of NaN (and one left dirty by a different problem) gives the same
    output bit for bit: nothing is read before it is written."""
    ss = _ss()
    q = _data(2, 700, 4, 2, 128, "bf16", seed=12)
    g = {k: v.cuda() for k, v in q.items()}
    call = lambda ws: ss.ssd_fwd(g["x"], g["dt"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"],
                                 dt_bias=g["dt_bias"], h0=g["h0"], workspace=ws, return_final_state=True)
    ws = torch.zeros(16 << 20, dtype=torch.float32, device="cuda")
    y0, f0 = call(ws)
    ws.fill_(float("nan"))
    y1, f1 = call(ws)
    q2 = _data(1, 300, 6, 3, 64, "f16", seed=13)
    g2 = {k: v.cuda() for k, v in q2.items()}
    ss.ssd_fwd(g2["x"], g2["dt"], g2["A"], g2["Bm"], g2["Cm"], workspace=ws)
    y2, f2 = call(ws)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(f0, f1) and torch.equal(y0, y2) and torch.equal(f0, f2)
    yr, fr = _ref(q)
    assert rel_err(f64(y1), yr) <= TOL["bf16"] and rel_err(f64(f1), fr) <= TOL["bf16"]


def test_mamba2_layer_shape_sampled_heads():
    """d_model 768, expand 2 -> 24 heads of 64, d_state 128, one group (the "niverel-mamba"
    README's V3 configuration) at the benchmarked size, B=8, L=2048, bf16: five heads
    against the oracle."""
    q = _data(8, 2048, 24, 1, 128, "bf16", seed=10)
    y, fin = _run(q)
    heads = [0, 5, 11, 17, 23]
    yr, fr = _ref(q, heads=heads)
    hi = torch.as_tensor(heads).cuda()
    assert rel_err(f64(y.index_select(2, hi)), yr) <= TOL["bf16"]
    assert rel_err(f64(fin.index_select(1, hi)), fr) <= TOL["bf16"]


# --------------------------------------------------------------- documents
# "niverel-mamba" README, "seq_idx strict reset": for Mamba-2 the SSM state
# resets to zero at every document boundary; h0 feeds a row's first document.

def _run_docs(q, seq, use=("D", "z", "dt_bias", "h0")):
    ss = _ss()
    g = {k: v.cuda() for k, v in q.items()}
    y, fin = ss.ssd_fwd(g["x"], g["dt"], g["A"], g["Bm"], g["Cm"], D=g["D"] if "D" in use else None,
                        z=g["z"] if "z" in use else None, dt_bias=g["dt_bias"] if "dt_bias" in use else None,
                        h0=g["h0"] if "h0" in use else None, seq_idx=seq.cuda(), return_final_state=True)
    torch.cuda.synchronize()
    return y, fin


def _ref_docs(q, seq, use=("D", "z", "dt_bias", "h0"), heads=None):
    sel = (lambda a, ax: a) if heads is None else (lambda a, ax: a.index_select(ax, torch.as_tensor(heads)))
    return oracle.ssd_fwd(f64(sel(q["x"], 2)), f64(sel(q["dt"], 2)), f64(sel(q["A"], 0)), f64(q["Bm"]), f64(q["Cm"]),
                          D=f64(sel(q["D"], 0)) if "D" in use else None, z=f64(sel(q["z"], 2)) if "z" in use else None,
                          dt_bias=f64(sel(q["dt_bias"], 0)) if "dt_bias" in use else None,
                          h0=f64(sel(q["h0"], 1)) if "h0" in use else None, seq_idx=seq.numpy())


@pytest.mark.parametrize("case", inputs.SEQ_CASES)
def test_documents_nine_cases(case):
    """The nine structural cases over three 256-step chunks (boundaries on chunk edges, inside
    chunks, at step 1, consecutive), with the initial state, every operand, two groups."""
    say("ssd documents case=%s" % case)
    q = _data(2, 700, 4, 2, 64, "bf16", seed=40)
    seq = inputs.make_seq_idx(case, 2, 700, seed=41)
    y, fin = _run_docs(q, seq)
    yr, fr = _ref_docs(q, seq)
    ey, ef = rel_err(f64(y), yr), rel_err(f64(fin), fr)
    say("  errors y=%.2e final=%.2e" % (ey, ef))
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"]


@pytest.mark.parametrize("L", [1, 2, 255, 256, 257, 513])
def test_documents_short_and_edge_lengths(L):
    """Document ids on rows that end at, just before or just past a chunk edge (a document
    starting at step 1 and at the chunk's last step included)."""
    q = _data(2, L, 2, 1, 64, "bf16", seed=47)
    ids = np.zeros((2, L), dtype=np.int32)
    for b, cut in enumerate([1, max(1, L - 1)]):
        ids[b, cut:] = 1
    seq = torch.from_numpy(ids)
    y, fin = _run_docs(q, seq)
    yr, fr = _ref_docs(q, seq)
    assert rel_err(f64(y), yr) <= TOL["bf16"] and rel_err(f64(fin), fr) <= TOL["bf16"]


@pytest.mark.parametrize("io,N", [("f16", 128), ("bf16", 32)])
def test_documents_long_rows(io, N):
    """L = 4096 (16 chunks) with documents of U[1, 700] steps, so most chunks hold a start and
    some documents span several chunks."""
    q = _data(2, 4096, 2, 1, N, io, seed=42)
    seq = inputs.packed_documents(4096, 2, 700, seed=43)
    say("ssd documents long rows io=%s N=%d" % (io, N))
    y, fin = _run_docs(q, seq)
    yr, fr = _ref_docs(q, seq)
    assert rel_err(f64(y), yr) <= TOL[io] and rel_err(f64(fin), fr) <= TOL[io]


def test_packed_row_equals_documents_on_device():
    """A row of three documents (300, 1 and 451 steps) gives, step for step, what the three run
    one by one give (h0 for the first only, zero for the others)."""
    ss = _ss()
    lens = [300, 1, 451]
    L = sum(lens)
    q = _data(1, L, 4, 2, 64, "bf16", seed=44)
    seq = torch.tensor(sum([[k] * n for k, n in enumerate(lens)], []), dtype=torch.int32).reshape(1, L)
    g = {k: v.cuda() for k, v in q.items()}
    y, fin = ss.ssd_fwd(g["x"], g["dt"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], dt_bias=g["dt_bias"],
                        h0=g["h0"], seq_idx=seq.cuda(), return_final_state=True)
    parts, t = [], 0
    for k, n in enumerate(lens):
        s = lambda a: a[:, t:t + n].contiguous()
        yk, fk = ss.ssd_fwd(s(g["x"]), s(g["dt"]), g["A"], s(g["Bm"]), s(g["Cm"]), D=g["D"], z=s(g["z"]),
                            dt_bias=g["dt_bias"], h0=g["h0"] if k == 0 else None, return_final_state=True)
        parts.append(yk)
        t += n
    torch.cuda.synchronize()
    assert rel_err(f64(y), f64(torch.cat(parts, dim=1))) <= TOL["bf16"]
    assert rel_err(f64(fin), f64(fk)) <= TOL["bf16"]


def test_documents_mamba2_layer_shape_sampled_heads():
    """The benchmarked layer (B=8, L=2048, 24 heads of 64, d_state 128, one group, bf16) packed
    with documents of U[1, 512] steps and an initial state: five heads against the oracle."""
    q = _data(8, 2048, 24, 1, 128, "bf16", seed=45)
    seq = inputs.packed_documents(2048, 8, 512, seed=46)
    y, fin = _run_docs(q, seq)
    heads = [0, 7, 12, 18, 23]
    yr, fr = _ref_docs(q, seq, heads=heads)
    hi = torch.as_tensor(heads).cuda()
    assert rel_err(f64(y.index_select(2, hi)), yr) <= TOL["bf16"]
    assert rel_err(f64(fin.index_select(1, hi)), fr) <= TOL["bf16"]
