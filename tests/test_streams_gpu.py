"""Every entry point enqueues on the caller's stream: the same calls made on a side stream
(default priority) give bit-identical results to the default stream's, and FwdCall /
StepCall / ConvStepCall honour an explicit stream."""
import pytest
import torch

from _util import say

pytestmark = pytest.mark.gpu


def _ss():
    from mamba_selective_scan_fwd_amd import ss
    ss.load_library()
    return ss


def _scan_inputs(seed=21, Bsz=2, Dd=40, N=16, L=700):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(s, generator=g)
    return dict(u=r(Bsz, Dd, L).cuda(), delta=(r(Bsz, Dd, L) * 0.5).cuda(), A=(-torch.rand(Dd, N, generator=g) * 4).cuda(),
                Bm=r(Bsz, N, L).cuda(), Cm=r(Bsz, N, L).cuda(), D=r(Dd).cuda(), z=r(Bsz, Dd, L).cuda(),
                bias=(r(Dd) * 0.1).cuda(), dy=r(Bsz, Dd, L).cuda())


def test_forward_backward_on_side_stream():
    ss = _ss()
    q = _scan_inputs()
    kw = dict(D=q["D"], z=q["z"], delta_bias=q["bias"])
    y0, l0, c0 = ss.fwd(q["u"], q["delta"], q["A"], q["Bm"], q["Cm"], return_ckpt=True, **kw)
    g0 = ss.bwd(q["u"], q["delta"], q["A"], q["Bm"], q["Cm"], c0, q["dy"], **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y1, l1, c1 = ss.fwd(q["u"], q["delta"], q["A"], q["Bm"], q["Cm"], return_ckpt=True, **kw)
        g1 = ss.bwd(q["u"], q["delta"], q["A"], q["Bm"], q["Cm"], c1, q["dy"], **kw)
    side.synchronize()
    say("side-stream forward/backward")
    assert torch.equal(y0, y1) and torch.equal(l0, l1) and torch.equal(c0, c1)
    for k in g0:
        assert torch.allclose(g0[k], g1[k], rtol=1e-5, atol=1e-6), k   # float atomics: order may differ


def test_prepared_calls_on_explicit_stream():
    ss = _ss()
    q = _scan_inputs(seed=22)
    side = torch.cuda.Stream()
    y0 = torch.empty_like(q["u"])
    y1 = torch.empty_like(q["u"])
    ss.FwdCall(q["u"], q["delta"], q["A"], q["Bm"], q["Cm"], D=q["D"], z=q["z"], delta_bias=q["bias"], y=y0)()
    torch.cuda.synchronize()
    call = ss.FwdCall(q["u"], q["delta"], q["A"], q["Bm"], q["Cm"], D=q["D"], z=q["z"], delta_bias=q["bias"], y=y1,
                      stream=side)
    call()
    side.synchronize()
    assert torch.equal(y0, y1)
    # decode step and conv step, prepared on the side stream
    Bsz, Dd, N = 2, 40, 16
    st_a = torch.randn(Bsz, Dd, N, device="cuda")
    st_b = st_a.clone()
    u_t, d_t, z_t = (q[k][..., 0].contiguous() for k in ("u", "delta", "z"))
    B_t, C_t = q["Bm"][..., 0].contiguous(), q["Cm"][..., 0].contiguous()
    ya, _ = ss.step(u_t, d_t, q["A"], B_t, C_t, st_a, D=q["D"], z_t=z_t, delta_bias=q["bias"], state_out=st_a)
    yb = torch.empty_like(u_t)
    torch.cuda.synchronize()
    ss.StepCall(u_t, d_t, q["A"], B_t, C_t, st_b, D=q["D"], z_t=z_t, delta_bias=q["bias"], y=yb, stream=side)()
    side.synchronize()
    assert torch.equal(ya, yb) and torch.equal(st_a, st_b)
    w = torch.randn(Dd, 4, device="cuda") * 0.5
    win_a = torch.randn(Bsz, Dd, 3, device="cuda")
    win_b = win_a.clone()
    oa, _ = ss.conv1d_step(u_t, w, win_a)
    ob = torch.empty_like(u_t)
    torch.cuda.synchronize()
    ss.ConvStepCall(u_t, w, win_b, ob, stream=side)()
    side.synchronize()
    assert torch.equal(oa, ob) and torch.equal(win_a, win_b)


def test_conv_and_ssd_on_side_stream():
    ss = _ss()
    g = torch.Generator().manual_seed(23)
    x = torch.randn(2, 40, 900, generator=g).half().cuda()
    w = (torch.randn(40, 4, generator=g) * 0.5).cuda()
    o0 = ss.conv1d(x, w)
    sx = torch.randn(1, 600, 4, 64, generator=g).bfloat16().cuda()
    sdt = (torch.randn(1, 600, 4, generator=g) * 0.5).bfloat16().cuda()
    sB = torch.randn(1, 600, 2, 64, generator=g).bfloat16().cuda()
    sC = torch.randn(1, 600, 2, 64, generator=g).bfloat16().cuda()
    sA = -torch.rand(4, generator=g).cuda() * 4
    s0 = ss.ssd_fwd(sx, sdt, sA, sB, sC)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        o1 = ss.conv1d(x, w)
        s1 = ss.ssd_fwd(sx, sdt, sA, sB, sC)
    side.synchronize()
    assert torch.equal(o0, o1) and torch.equal(s0, s1)


def test_graph_replays_match_eager():
    """Decode steps and a forward captured in a HIP graph (the serving pattern) and replayed
    three times, with eager work and a state reset between replays: every replay equals
    the eager results bit for bit (no memset node is ever recorded)."""
    ss = _ss()
    q = _scan_inputs(seed=24)
    Bsz, Dd, N = 2, 40, 16
    toks = [{k: q[k][..., t].contiguous() for k in ("u", "delta", "z")} for t in range(8)]
    for t, tok in enumerate(toks):
        tok["B"], tok["C"] = q["Bm"][..., t].contiguous(), q["Cm"][..., t].contiguous()
    st0 = torch.randn(Bsz, Dd, N, device="cuda")
    st_e = st0.clone()
    ys_e = []
    for tok in toks:
        y, _ = ss.step(tok["u"], tok["delta"], q["A"], tok["B"], tok["C"], st_e, D=q["D"], z_t=tok["z"],
                       delta_bias=q["bias"], state_out=st_e)
        ys_e.append(y.clone())
    yf_e = ss.fwd(q["u"], q["delta"], q["A"], q["Bm"], q["Cm"], D=q["D"], z=q["z"], delta_bias=q["bias"])[0]
    torch.cuda.synchronize()

    st = st0.clone()
    ys = [torch.empty_like(toks[0]["u"]) for _ in toks]
    yf = torch.empty_like(q["u"])

    def steps():
        for tok, y in zip(toks, ys):
            ss.step(tok["u"], tok["delta"], q["A"], tok["B"], tok["C"], st, D=q["D"], z_t=tok["z"],
                    delta_bias=q["bias"], state_out=st, y=y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        steps()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps()
        ss.FwdCall(q["u"], q["delta"], q["A"], q["Bm"], q["Cm"], D=q["D"], z=q["z"], delta_bias=q["bias"], y=yf,
                   stream=torch.cuda.current_stream())()
    for rep in range(3):
        st.copy_(st0)
        yf.zero_()
        junk = torch.randn(1 << 16, device="cuda").mul_(2.0).sum()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        say("graph replay %d" % rep)
        for y, ye in zip(ys, ys_e):
            assert torch.equal(y, ye)
        assert torch.equal(st, st_e) and torch.equal(yf, yf_e)


def test_graph_replays_conv_ssd_bwd():
    """The conv, the SSD layer and the backward captured in one HIP graph and replayed three
    times, with eager work between the replays: every replay equals the eager results (the
    backward's float atomics to within rounding, everything else bit for bit)."""
    ss = _ss()
    q = _scan_inputs(seed=25)
    kw = dict(D=q["D"], z=q["z"], delta_bias=q["bias"])
    g = torch.Generator().manual_seed(26)
    x = torch.randn(2, 40, 900, generator=g).half().cuda()
    w = (torch.randn(40, 4, generator=g) * 0.5).cuda()
    sx = torch.randn(1, 600, 4, 64, generator=g).bfloat16().cuda()
    sdt = (torch.randn(1, 600, 4, generator=g) * 0.5).bfloat16().cuda()
    sB = torch.randn(1, 600, 2, 64, generator=g).bfloat16().cuda()
    sC = torch.randn(1, 600, 2, 64, generator=g).bfloat16().cuda()
    sA = -torch.rand(4, generator=g).cuda() * 4
    _, _, ck = ss.fwd(q["u"], q["delta"], q["A"], q["Bm"], q["Cm"], return_ckpt=True, **kw)

    def work():
        o = ss.conv1d(x, w)
        s = ss.ssd_fwd(sx, sdt, sA, sB, sC, z=sx, D=sA)
        gr = ss.bwd(q["u"], q["delta"], q["A"], q["Bm"], q["Cm"], ck, q["dy"], **kw)
        return o, s, gr

    o_e, s_e, g_e = work()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        o_g, s_g, g_g = work()
    for rep in range(3):
        for t in (o_g, s_g, *g_g.values()):
            t.fill_(float("nan"))
        junk = torch.randn(1 << 16, device="cuda").mul_(3.0).sum()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        say("graph replay %d (conv, ssd, bwd)" % rep)
        assert torch.equal(o_g, o_e) and torch.equal(s_g, s_e)
        for k in g_e:
            if k in ("du", "ddelta", "dz"):
                assert torch.equal(g_g[k], g_e[k]), k
            else:
                assert torch.allclose(g_g[k], g_e[k], rtol=1e-5, atol=1e-6), k
