#!/usr/bin/env python3
"""Throughput of the selective-scan forward on one MI355X.

One step = one ss_fwd over the mamba-130m layer workload (B=8, d_inner=1536,
d_state=16, L=2048, fp16 I/O, fp32 state and arithmetic, softplus + bias,
D skip, SiLU gate, final state), inputs resident in HBM.  Three independent
input sets are rotated so that the 256 MB MALL cannot hold the working set
between steps.  Prints ONE JSON line.

Also measured (reported in "rows"): the long-sequence forward (B=1, D=16,
L=32768, fp32), the ragged mamba-2.8b layer forward (bf16), 64 decode steps
on the mamba-130m state, the backward (fp32, B=4, D=1536, L=4097), and a plain
device copy (achievable HBM bandwidth).  The float64 CPU oracle is timed on a
bounded sample of the same workload as "cpu_baseline".
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from mamba_selective_scan_fwd_amd import inputs, ss  # noqa: E402

PEAK_HBM_GBPS = 8000.0
# Algorithmic vector work of the forward, in lane-operations (one lane of one
# wave64 instruction), priced below at the issue rates the library's probe
# measures on the chip (not at a datasheet rate):
#   per (t, d, n): one exp (the decay) and four plain operations (the exp's
#                  argument Delta*A, Delta*u*B, the recurrence FMA, the readout FMA)
#   per (t, d):    four transcendentals (softplus: exp + log; SiLU: exp + rcp) and
#                  ten plain operations (softplus' other steps, Delta*u, skip, gate),
#                  plus four conversions when the I/O is 16-bit
TRANS_PER_TDN, PLAIN_PER_TDN = 1, 4
TRANS_PER_TD, PLAIN_PER_TD, CVT16_PER_TD = 4, 10, 4
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["mamba_selective_scan_fwd_amd/csrc/ss_fwd.hip", "mamba_selective_scan_fwd_amd/csrc/ss_device.h"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def fwd_alg_bytes(Bsz, Dd, N, L, s, lengths=None, ckpt=False):
    """Algorithmic bytes of one forward: inputs read once, y written once, weights, final state."""
    if lengths is None:
        lengths = [L] * Bsz
    valid = int(sum(lengths))
    byt = valid * (Dd * (3 * s + s) + 2 * N * s)       # u, delta, z read + y written; B, C read once
    byt += (L * Bsz - valid) * Dd * s                   # masked y written as zeros
    byt += 4 * (Dd * N + 2 * Dd)                        # A, D, bias
    byt += 4 * Bsz * Dd * N                             # final state
    if ckpt:
        byt += 4 * Bsz * Dd * ((L + 63) // 64) * N
    return byt


def fwd_alg_ops(Bsz, Dd, N, L, s, lengths=None):
    """(transcendental, plain) lane-operations of one forward."""
    td = (int(sum(lengths)) if lengths is not None else Bsz * L) * Dd
    trans = td * (TRANS_PER_TDN * N + TRANS_PER_TD)
    plain = td * (PLAIN_PER_TDN * N + PLAIN_PER_TD + (CVT16_PER_TD if s == 2 else 0))
    return trans, plain


def alu_floor_ms(ops, rates):
    """Shortest time the vector units can do `ops` in at the measured rates: every SIMD busy,
    each wave64 instruction costing its measured cycles, at the measured clock."""
    trans, plain = ops
    cycles = (trans * rates["exp"]["cycles_per_unit"] + plain * rates["fma"]["cycles_per_unit"]) / 64.0
    return cycles / rates["simds"] / (rates["clock_GHz"] * 1e9) * 1e3


def measure_alu_rates(waves_per_simd=3):
    """Issue rates of the scan's instructions on this chip at the headline's occupancy (three waves
    per SIMD), from the library's probe: cycles per wave64 instruction and the clock under load."""
    out = {}
    for kind in ("fma", "exp", "dpp_mul", "scan_step"):
        ss.alu_probe(kind, waves_per_simd, iters=256)        # warm
        out[kind] = ss.alu_probe(kind, waves_per_simd, iters=8192)
    props = torch.cuda.get_device_properties(0)
    out["simds"] = props.multi_processor_count * 4
    out["clock_GHz"] = out["scan_step"]["clock_GHz"]   # the mix closest to the kernel's
    return out


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the headline kernel from the committed counter summary,
    or None when it is missing or was taken on a different kernel source."""
    path = os.path.join(PROFILE_DIR, "ss_fwd_final_mamba130m_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def timed(fn, reps, stream, warm_s=0.12):
    """Average ms per call of fn() over reps calls, HIP events on the launch stream, after
    ~warm_s of untimed calls: the GPU needs ~100 ms of load to reach its working clock, and
    it idles while the host prepares the next workload."""
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while n < 2 or time.perf_counter() - t0 < warm_s:
        fn(n)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(reps):
        fn(i)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / reps


def dev_problem(prob):
    keys = ("u", "delta", "z", "Bm", "Cm", "A", "D", "bias", "lengths", "dy")
    return {k: (None if prob.get(k) is None else prob[k].to("cuda")) for k in keys}


def bench_headline(steps, warmup, stream, prewarm_s=0.3):
    sets = []
    for r in range(3):
        prob = inputs.make_config(2, seed=2 + 100 * r, decode_steps=0)
        sets.append(dev_problem(prob))
    Bsz, Dd, L = sets[0]["u"].shape
    N = sets[0]["A"].shape[1]
    ys = [torch.empty((Bsz, Dd, L), dtype=torch.float16, device="cuda") for _ in range(3)]
    lasts = [torch.empty((Bsz, Dd, N), dtype=torch.float32, device="cuda") for _ in range(3)]
    calls = [ss.FwdCall(g["u"], g["delta"], g["A"], g["Bm"], g["Cm"], D=g["D"], z=g["z"], delta_bias=g["bias"],
                        delta_softplus=True, y=ys[r], last_state=lasts[r], stream=stream)
             for r, g in enumerate(sets)]

    def step(i):
        calls[i % 3]()

    # untimed calls until the clock has settled (the GPU needs ~100 ms of load; a cold
    # clock reads 15-25% slow), then the requested warm-up steps
    torch.cuda.synchronize()
    t_pre, n_pre = time.perf_counter(), 0
    while time.perf_counter() - t_pre < prewarm_s:
        step(n_pre)
        n_pre += 1
        if n_pre % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    prewarm = {"prewarm_s": time.perf_counter() - t_pre, "prewarm_calls": n_pre}
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # the whole job: one event pair around the K steps on the launch stream
    # (events between launches would add their own gaps to it)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    # the spread of single launches: K more steps with an event pair around each
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        step(steps + i)
        stops[i].record(stream)
    torch.cuda.synchronize()
    per_launch = sorted(a.elapsed_time(b) for a, b in zip(starts, stops))
    # every step is one launch and the launches run back to back on one stream,
    # so the whole job's time per step is the kernel's duration; a pair of events
    # around a single launch adds its own overhead (~2 us) to what it measures
    kernel_ms = ms
    stats = {"per_launch_events_ms_mean": sum(per_launch) / steps, "per_launch_events_ms_median": per_launch[steps // 2],
             "per_launch_events_ms_min": per_launch[0], "per_launch_events_ms_max": per_launch[-1]}
    # warm figure, labelled as such: one input set called back to back, so the
    # MALL can hold part of it; never the reported value
    warm = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    reps = max(10, steps // 4)
    warm[0].record(stream)
    for _ in range(reps):
        calls[0]()
    warm[1].record(stream)
    torch.cuda.synchronize()
    stats["warm_single_set_kernel_ms"] = warm[0].elapsed_time(warm[1]) / reps
    stats.update(prewarm)
    return ms, kernel_ms, stats, wall, (Bsz, Dd, N, L), sets, ys


def bench_long(stream):
    """Long sequence, few channels (the time-chunked scan), fp32: B=1, D=16, L=32768."""
    p1 = dev_problem(inputs.make_config(1))
    y1 = torch.empty_like(p1["u"])
    s1 = torch.empty((1, 16, 16), dtype=torch.float32, device="cuda")
    c1 = ss.FwdCall(p1["u"], p1["delta"], p1["A"], p1["Bm"], p1["Cm"], D=p1["D"], z=p1["z"],
                    delta_bias=p1["bias"], y=y1, last_state=s1, stream=stream)
    f1 = lambda i: c1()
    f1(0)
    ms = timed(f1, 20, stream)
    tc = 1 * 16 * 32768
    return {"ms": ms, "token_channel_per_s": tc / (ms * 1e-3), "tokens_per_s": 32768 / (ms * 1e-3)}


def bench_rows(stream):
    rows = {}
    rows["fwd_long_B1_D16_L32768_f32"] = bench_long(stream)
    # ragged mamba-2.8b layer, bf16
    prob3 = inputs.make_config(3)
    lens = prob3["lengths"].tolist()
    p3 = dev_problem(prob3)
    del prob3
    y3 = torch.empty_like(p3["u"])
    s3 = torch.empty((4, 5120, 16), dtype=torch.float32, device="cuda")
    c3 = ss.FwdCall(p3["u"], p3["delta"], p3["A"], p3["Bm"], p3["Cm"], D=p3["D"], z=p3["z"],
                    delta_bias=p3["bias"], lengths=p3["lengths"], y=y3, last_state=s3, stream=stream)
    f3 = lambda i: c3()
    f3(0)
    ms = timed(f3, 10, stream)
    byt = fwd_alg_bytes(4, 5120, 16, 8192, 2, lengths=lens)
    rows["fwd_ragged_B4_D5120_L8192_bf16"] = {
        "ms": ms, "lengths": lens, "token_channel_per_s": sum(lens) * 5120 / (ms * 1e-3),
        "alg_GBps": byt / (ms * 1e-3) / 1e9, "hbm_frac": byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "alu_ops": fwd_alg_ops(4, 5120, 16, 8192, 2, lens)}
    del p3, c3, y3
    # packed documents (lengths U[1, 512]) and an initial state on the mamba-130m layer
    prob2p = inputs.make_config(2, decode_steps=0)
    g2p = dev_problem(prob2p)
    del prob2p
    seq = inputs.packed_documents(2048, 8, 512, seed=7).to("cuda")
    h0 = torch.randn((8, 1536, 16), dtype=torch.float32, device="cuda")
    y2p = torch.empty_like(g2p["u"])
    s2p = torch.empty((8, 1536, 16), dtype=torch.float32, device="cuda")
    c2p = ss.FwdCall(g2p["u"], g2p["delta"], g2p["A"], g2p["Bm"], g2p["Cm"], D=g2p["D"], z=g2p["z"],
                     delta_bias=g2p["bias"], y=y2p, last_state=s2p, stream=stream, seq_idx=seq, h0=h0)
    fp = lambda i: c2p()
    fp(0)
    ms = timed(fp, 20, stream)
    docs = int((seq[:, 1:] != seq[:, :-1]).sum().item()) + 8
    rows["fwd_packed_docs_h0_B8_D1536_L2048_f16"] = {
        "ms": ms, "documents": docs, "token_channel_per_s": 8 * 1536 * 2048 / (ms * 1e-3),
        "hbm_frac": fwd_alg_bytes(8, 1536, 16, 2048, 2) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    del g2p, c2p, y2p, s2p, seq, h0
    rows["conv1d_silu_B8_D1536_L2048_W4_f16"] = bench_conv(stream)
    # Mamba-2 SSD chunked scan on the matrix cores: d_model 768, expand 2 -> 24 heads of 64,
    # d_state 128, one group, chunk 256 (the "niverel-mamba" README's V3 configuration), B=8,
    # L=2048, bf16, with D, z gate and dt_bias; two rotated input sets
    rows["ssd_fwd_B8_L2048_H24_P64_N128_bf16"] = bench_ssd(stream)
    # decode: 64 single steps on the mamba-130m state
    prob2 = inputs.make_config(2, decode_steps=64)
    g2 = dev_problem(prob2)
    toks = [{k: v.to("cuda") for k, v in t.items()} for t in prob2["decode"]]
    state = torch.zeros((8, 1536, 16), dtype=torch.float32, device="cuda")
    yt = torch.empty((8, 1536), dtype=torch.float16, device="cuda")

    def fstep(i):
        t = toks[i % 64]
        ss.step(t["u_t"], t["delta_t"], g2["A"], t["B_t"], t["C_t"], state, D=g2["D"], z_t=t["z_t"],
                delta_bias=g2["bias"], state_out=state, y=yt)

    fstep(0)
    ms = timed(fstep, 64, stream)
    rows["decode_step_B8_D1536_f16"] = {"us_per_step_checked_call": ms * 1e3}
    # prepared calls: one C call per step (token buffers bound once)
    steps = [ss.StepCall(t["u_t"], t["delta_t"], g2["A"], t["B_t"], t["C_t"], state, D=g2["D"], z_t=t["z_t"],
                         delta_bias=g2["bias"], state_out=state, y=yt, stream=stream) for t in toks]
    fs = lambda i: steps[i % 64]()
    fs(0)
    ms = timed(fs, 64, stream)
    rows["decode_step_B8_D1536_f16"].update({"us_per_step": ms * 1e3,
                                             "state_GBps": 2 * 8 * 1536 * 16 * 4 / (ms * 1e-3) / 1e9})
    # graph-captured decode: 64 steps replayed as one graph
    try:
        g = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s2):
            fstep(0)
        torch.cuda.current_stream().wait_stream(s2)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(64):
                fstep(i)
        g.replay()
        torch.cuda.synchronize()
        ms = timed(lambda i: g.replay(), 10, stream)
        rows["decode_step_B8_D1536_f16"]["us_per_step_graph"] = ms * 1e3 / 64
    except Exception as e:  # graph capture is a measurement extra, never the headline
        rows["decode_step_B8_D1536_f16"]["graph_error"] = str(e)[:200]
    del g2, toks
    rows.update(bench_bwd(stream))
    torch.cuda.empty_cache()
    return rows


def bench_conv(stream):
    # the step before the scan: depthwise causal conv1d (width 4) + SiLU on the mamba-130m
    # layer's x branch (fp16), three rotated input sets (the 256 MB MALL cannot hold them)
    gcv = torch.Generator(device="cuda")
    gcv.manual_seed(9)
    xs = [torch.randn((8, 1536, 2048), device="cuda", generator=gcv).half() for _ in range(3)]
    outs = [torch.empty_like(xs[0]) for _ in range(3)]
    wcv = torch.randn((1536, 4), device="cuda", generator=gcv) * 0.5
    bcv = torch.randn((1536,), device="cuda", generator=gcv) * 0.1
    fc = lambda i: ss.conv1d(xs[i % 3], wcv, bcv, out=outs[i % 3])
    fc(0)
    ms = timed(fc, 30, stream)
    cbytes = 2 * 8 * 1536 * 2048 * 2 + 1536 * 5 * 4
    row = {
        "ms": ms, "alg_GBps": cbytes / (ms * 1e-3) / 1e9, "hbm_frac": cbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    win = torch.zeros((8, 1536, 3), dtype=torch.float32, device="cuda")
    fcs = lambda i: ss.conv1d_step(xs[0][..., i % 2048].contiguous(), wcv, win, bcv)
    fcs(0)
    ms = timed(fcs, 64, stream)
    row["decode_us_per_step_checked_call"] = ms * 1e3
    # the serving form: preallocated token, window and output buffers, one C call per step
    xt = xs[0][..., 0].contiguous()
    ot = torch.empty_like(xt)
    ccs = ss.ConvStepCall(xt, wcv, win, ot, bias=bcv, stream=stream)
    ccs()
    ms = timed(lambda i: ccs(), 256, stream)
    row["decode_us_per_step"] = ms * 1e3
    del xs, outs, win
    return row


def bench_bwd(stream):
    rows = {}
    # backward, fp32
    try:
        prob4 = inputs.make_config(4)
        p4 = dev_problem(prob4)
        del prob4
        _, _, ck = ss.fwd(p4["u"], p4["delta"], p4["A"], p4["Bm"], p4["Cm"], D=p4["D"], z=p4["z"],
                          delta_bias=p4["bias"], return_ckpt=True)
        fb = lambda i: ss.bwd(p4["u"], p4["delta"], p4["A"], p4["Bm"], p4["Cm"], ck, p4["dy"], D=p4["D"],
                              z=p4["z"], delta_bias=p4["bias"])
        fb(0)
        ms = timed(fb, 5, stream)
        Bsz, Dd, L, N = 4, 1536, 4097, 16
        byt = (Bsz * Dd * L * 4 * 7 + 2 * Bsz * N * L * 4 * 2 + ck.numel() * 4 + 4 * (Dd * N + 2 * Dd) * 2)
        rows["bwd_B4_D1536_L4097_f32"] = {"ms": ms, "token_channel_per_s": Bsz * Dd * L / (ms * 1e-3),
                                          "alg_GBps": byt / (ms * 1e-3) / 1e9}
        # the same with packed documents (lengths U[1, 600]), a final-state gradient and dh0
        seq = inputs.packed_documents(L, Bsz, 600, seed=8).to("cuda")
        dlast = torch.randn((Bsz, Dd, N), dtype=torch.float32, device="cuda")
        _, _, ck2 = ss.fwd(p4["u"], p4["delta"], p4["A"], p4["Bm"], p4["Cm"], D=p4["D"], z=p4["z"],
                           delta_bias=p4["bias"], return_ckpt=True, seq_idx=seq)
        fb2 = lambda i: ss.bwd(p4["u"], p4["delta"], p4["A"], p4["Bm"], p4["Cm"], ck2, p4["dy"], D=p4["D"],
                               z=p4["z"], delta_bias=p4["bias"], seq_idx=seq, dlast=dlast, want_dh0=True)
        fb2(0)
        ms = timed(fb2, 5, stream)
        rows["bwd_packed_docs_dlast_dh0_B4_D1536_L4097_f32"] = {
            "ms": ms, "token_channel_per_s": Bsz * Dd * L / (ms * 1e-3)}
        del p4, ck, ck2, seq, dlast
    except RuntimeError as e:
        rows["bwd_B4_D1536_L4097_f32"] = {"error": str(e)[:200]}
    return rows


def bench_ssd(stream):
    Bsz, L, Hn, P, G, N, Q = 8, 2048, 24, 64, 1, 128, 256
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    rnd = lambda *shape: torch.randn(shape, device="cuda", generator=gen)
    sets = []
    for _ in range(2):
        sets.append(dict(x=rnd(Bsz, L, Hn, P).bfloat16(), dt=(rnd(Bsz, L, Hn) * 0.5).bfloat16(),
                         Bm=rnd(Bsz, L, G, N).bfloat16(), Cm=rnd(Bsz, L, G, N).bfloat16(),
                         z=rnd(Bsz, L, Hn, P).bfloat16(), y=torch.empty((Bsz, L, Hn, P), dtype=torch.bfloat16,
                                                                       device="cuda")))
    A = -torch.exp(torch.rand(Hn, device="cuda", generator=gen) * 2.77)
    D = rnd(Hn)
    dt_bias = torch.log(torch.expm1(torch.exp(torch.rand(Hn, device="cuda", generator=gen) * 4.6 - 6.9)))
    ws = torch.empty(64 << 20, dtype=torch.float32, device="cuda")
    f = lambda i: ss.ssd_fwd(sets[i % 2]["x"], sets[i % 2]["dt"], A, sets[i % 2]["Bm"], sets[i % 2]["Cm"], D=D,
                             z=sets[i % 2]["z"], dt_bias=dt_bias, y=sets[i % 2]["y"], workspace=ws)
    for i in range(800):   # ~100 ms of load: the clock settles before the timed calls
        f(i)
    ms = timed(f, 50, stream)
    # the same layer packed with documents of U[1, 512] steps (the document-reset kernels)
    seq = inputs.packed_documents(L, Bsz, 512, seed=12).to("cuda")
    fd = lambda i: ss.ssd_fwd(sets[i % 2]["x"], sets[i % 2]["dt"], A, sets[i % 2]["Bm"], sets[i % 2]["Cm"], D=D,
                              z=sets[i % 2]["z"], dt_bias=dt_bias, y=sets[i % 2]["y"], workspace=ws, seq_idx=seq)
    ms_docs = timed(fd, 50, stream)
    nchunks = (L + Q - 1) // Q
    # dense work of the chunked algorithm per (row, chunk, head): C B^T and M x over the causal half,
    # the chunk state and the state readout
    flop = 2 * Bsz * nchunks * Hn * (Q * Q * N // 2 + Q * Q * P // 2 + 2 * Q * N * P)
    byt = Bsz * L * Hn * P * 2 * 3 + Bsz * L * Hn * 2 + 2 * Bsz * L * G * N * 2   # x, z, y, dt, B, C once
    del sets, ws
    return {"ms": ms, "ms_packed_documents": ms_docs, "token_channel_per_s": Bsz * L * Hn * P / (ms * 1e-3),
            "state_updates_per_s": Bsz * L * Hn * P * N / (ms * 1e-3),
            "mfma_TFLOPs": flop / (ms * 1e-3) / 1e12, "mfma_frac_of_bf16_peak": flop / (ms * 1e-3) / 2.5e15,
            "alg_GBps": byt / (ms * 1e-3) / 1e9, "hbm_frac": byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}


def copy_probe(stream):
    nbytes = 1 << 30
    src = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ss.copy_probe(src, dst)
    ms = timed(lambda i: ss.copy_probe(src, dst), 10, stream)
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def cpu_baseline(sets_cpu_seed=2, target_s=12.0):
    """The float64 oracle on a bounded sample of the headline workload: every batch row, a
    block of channels, the full sequence, sized to about target_s of wall time (when the whole
    workload takes less, whole passes over it are repeated); scaled to (token*channel)/s."""
    import oracle
    prob = inputs.make_config(2, seed=sets_cpu_seed, decode_steps=0)
    L = prob["seqlen"]
    threads = oracle.default_threads()

    def run(nd, reps=1):
        sel = lambda t: inputs.to_f64(t[:, :nd])
        args = dict(u=sel(prob["u"]), delta=sel(prob["delta"]), A=inputs.to_f64(prob["A"][:nd]),
                    Bm=inputs.to_f64(prob["Bm"]), Cm=inputs.to_f64(prob["Cm"]), D=inputs.to_f64(prob["D"][:nd]),
                    z=sel(prob["z"]), bias=inputs.to_f64(prob["bias"][:nd]))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.fwd(**args, threads=threads)
        return time.perf_counter() - t0
    # calibrate on a small block, then size the sample to ~target_s
    nd = 16
    t = run(nd)
    nd2 = int(min(1536, max(16, nd * target_s / max(t, 1e-3))))
    t1 = run(nd2)
    reps = max(1, int(round(target_s / max(t1, 1e-3)))) if nd2 == 1536 else 1
    t2 = run(nd2, reps) if reps > 1 else t1
    tc = 8 * nd2 * L * reps
    return {"value": tc / t2, "unit": "(token*channel)/s", "cores": threads, "kind": "oracle",
            "sample": "float64 oracle, all 8 batch rows x first %d of 1536 channels x L=%d of the mamba-130m "
                      "workload, %d pass(es) (%d token*channel), %.2f s wall" % (nd2, L, reps, tc, t2)}


def cpu_rows(rows, target_s=1.0):
    """The float64 oracle beside each other workload, on a bounded sample of it (the whole
    workload where it is small, else a block of channels or one head over the full sequence,
    drawn from the same distributions), scaled to the row's unit."""
    import oracle
    threads = oracle.default_threads()
    f64 = inputs.to_f64
    out = {}

    def per_call(fn):
        t0 = time.perf_counter()
        fn()
        t = time.perf_counter() - t0
        reps = max(1, int(target_s / max(t, 1e-4)))
        if reps > 1:
            t0 = time.perf_counter()
            for _ in range(reps):
                fn()
            t = (time.perf_counter() - t0) / reps
        return t, reps + 1

    def rec(value, unit, cores, sample):
        log("  oracle: %s" % sample)
        return {"value": value, "unit": unit, "cores": cores, "kind": "oracle", "sample": sample}

    def scan_args(p):
        return {k: f64(p[k]) for k in ("u", "delta", "A", "Bm", "Cm", "D", "z", "bias")}

    if "fwd_long_B1_D16_L32768_f32" in rows:
        a = scan_args(inputs.make_config(1))
        t, n = per_call(lambda: oracle.fwd(**a, threads=threads))
        out["fwd_long_B1_D16_L32768_f32"] = rec(16 * 32768 / t, "(token*channel)/s", min(threads, 16),
                                                "the whole workload, %d passes" % n)
        t1, n1 = per_call(lambda: oracle.fwd(**a, threads=1))
        out["fwd_long_B1_D16_L32768_f32"]["value_single_core"] = 16 * 32768 / t1
    lens = rows.get("fwd_ragged_B4_D5120_L8192_bf16", {}).get("lengths")
    if lens:
        nd = 64
        a = scan_args(inputs.make_problem(4, nd, 16, 8192, io="bf16", seed=3))
        ln = np.asarray(lens, dtype=np.int64)
        t, n = per_call(lambda: oracle.fwd(**a, lengths=ln, threads=threads))
        out["fwd_ragged_B4_D5120_L8192_bf16"] = rec(sum(lens) * nd / t, "(token*channel)/s", threads,
                                                    "%d of 5120 channels, the row's lengths %s, %d passes" % (nd, lens, n))
    if "fwd_packed_docs_h0_B8_D1536_L2048_f16" in rows:
        nd = 64
        a = scan_args(inputs.make_problem(8, nd, 16, 2048, io="f16", seed=2, A_mode="a_log"))
        seq = inputs.packed_documents(2048, 8, 512, seed=7).numpy()
        h0 = np.random.default_rng(7).standard_normal((8, nd, 16))
        t, n = per_call(lambda: oracle.fwd(**a, seq_idx=seq, h0=h0, threads=threads))
        out["fwd_packed_docs_h0_B8_D1536_L2048_f16"] = rec(8 * nd * 2048 / t, "(token*channel)/s", threads,
                                                           "%d of 1536 channels, the row's documents, %d passes" % (nd, n))
    if "conv1d_silu_B8_D1536_L2048_W4_f16" in rows:
        nd = 128
        rng = np.random.default_rng(9)
        x = f64(torch.from_numpy(rng.standard_normal((8, nd, 2048))).half())
        w = rng.standard_normal((nd, 4)) * 0.5
        bc = rng.standard_normal(nd) * 0.1
        t, n = per_call(lambda: oracle.conv1d_fwd(x, w, bc))
        out["conv1d_silu_B8_D1536_L2048_W4_f16"] = rec(8 * nd * 2048 / t, "(token*channel)/s", 1,
                                                       "%d of 1536 channels (single-threaded oracle), %d passes" % (nd, n))
    if "ssd_fwd_B8_L2048_H24_P64_N128_bf16" in rows:
        rng = np.random.default_rng(11)
        bf = lambda *sh: f64(torch.from_numpy(rng.standard_normal(sh)).bfloat16())
        x, z = bf(8, 2048, 1, 64), bf(8, 2048, 1, 64)
        dt = f64(torch.from_numpy(rng.standard_normal((8, 2048, 1)) * 0.5).bfloat16())
        Bm, Cm = bf(8, 2048, 1, 128), bf(8, 2048, 1, 128)
        A = -np.exp(rng.uniform(0, 2.77, 1))
        D = rng.standard_normal(1)
        db = np.log(np.expm1(np.exp(rng.uniform(-6.9, -2.3, 1))))
        t, n = per_call(lambda: oracle.ssd_fwd(x, dt, A, Bm, Cm, D=D, z=z, dt_bias=db))
        out["ssd_fwd_B8_L2048_H24_P64_N128_bf16"] = rec(8 * 2048 * 64 / t, "(token*channel)/s", 1,
                                                        "1 of 24 heads (single-threaded oracle), %d passes" % n)
    if "decode_step_B8_D1536_f16" in rows:
        p = inputs.make_problem(8, 1536, 16, 1, io="f16", seed=2, A_mode="a_log", decode_steps=1)
        tok = {k: f64(v) for k, v in p["decode"][0].items()}
        st = np.zeros((8, 1536, 16))
        a = {k: f64(p[k]) for k in ("A", "D", "bias")}
        t, n = per_call(lambda: oracle.step(tok["u_t"], tok["delta_t"], a["A"], tok["B_t"], tok["C_t"], st,
                                            D=a["D"], z_t=tok["z_t"], bias=a["bias"]))
        out["decode_step_B8_D1536_f16"] = rec(t * 1e6, "us/step", 1,
                                              "one step of the whole state (single-threaded oracle), %d steps" % n)
    if "bwd_B4_D1536_L4097_f32" in rows and "ms" in rows["bwd_B4_D1536_L4097_f32"]:
        nd = 32
        p = inputs.make_problem(4, nd, 16, 4097, io="f32", seed=4, with_dy=True)
        a = scan_args(p)
        dy = f64(p["dy"])
        t, n = per_call(lambda: oracle.bwd(a["u"], a["delta"], a["A"], a["Bm"], a["Cm"], dy, D=a["D"], z=a["z"],
                                           bias=a["bias"], threads=threads))
        out["bwd_B4_D1536_L4097_f32"] = rec(4 * nd * 4097 / t, "(token*channel)/s", threads,
                                            "%d of 1536 channels, %d passes" % (nd, n))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps first: the GPU needs ~100 ms of load to reach its working clock")
    ap.add_argument("--no-rows", action="store_true", help="headline only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--row", choices=["ssd", "conv", "bwd", "long"], help="time one secondary workload alone and print its JSON line "
                    "(for profiling it on its own); the headline is not run")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the scan shards by batch "
              "row or channel with no communication in the forward). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    torch.cuda.init()
    stream = torch.cuda.current_stream()
    if args.row:
        if args.row == "ssd":
            out = {"ssd_fwd_B8_L2048_H24_P64_N128_bf16": bench_ssd(stream)}
        elif args.row == "conv":
            out = {"conv1d_silu_B8_D1536_L2048_W4_f16": bench_conv(stream)}
        elif args.row == "long":
            out = {"fwd_long_B1_D16_L32768_f32": bench_long(stream)}
        else:
            out = bench_bwd(stream)
        out["copy_probe_GBps"] = copy_probe(stream)   # the counter calibration kernel, same process
        print(json.dumps(out), flush=True)
        return
    log("headline: %d warmup + %d timed steps" % (args.warmup, args.steps))
    ms, kernel_ms, stats, wall, (Bsz, Dd, N, L), sets, ys = bench_headline(args.steps, args.warmup, stream)
    del sets, ys
    torch.cuda.empty_cache()
    tc = Bsz * Dd * L
    value = tc / (ms * 1e-3)
    alg_bytes = fwd_alg_bytes(Bsz, Dd, N, L, 2)
    traffic = recorded_traffic()
    achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9
    result = {
        "metric": "selective-scan fwd (token*channel)/s and HBM GB/s as % of MI355X peak",
        "value": value,
        "unit": "(token*channel)/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "mamba-130m layer selective-scan forward: B=8, d_inner=1536, d_state=16, "
                               "L=2048, fp16 I/O, softplus+bias, D skip, SiLU gate, final state",
                   "io_dtype": "f16", "compute_dtype": "f32", "batch": Bsz, "d_inner": Dd, "d_state": N,
                   "seq_len": L, "input_sets_rotated": 3},
        # the HBM roofline of the one kernel of a step: algorithmic bytes per launch over the
        # launch's duration (HIP events around K back-to-back launches on the launch stream,
        # divided by K), against MI355X's 8 TB/s
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                     "kernel": "ss_fwd_chunk_kernel<f16, pairs, no documents, softplus+gate>",
                     "alg_bytes_per_launch": alg_bytes,
                     "kernel_ms_event_region": kernel_ms,
                     **stats},
        "wall_s_timed_region": wall,
    }
    # the vector-ALU ceiling, measured: the algorithm's instruction mix priced at the issue
    # rates the library's probe measures on this chip at the kernel's occupancy
    try:
        rates = measure_alu_rates(3)
        ops = fwd_alg_ops(Bsz, Dd, N, L, 2)
        floor = alu_floor_ms(ops, rates)
        step_cycles = rates["scan_step"]["cycles_per_unit"]
        # the scan core alone as this kernel maps it: one step per lane per (t, d, n), on
        # 16 lanes per channel
        core = tc * N / 64.0 * step_cycles / rates["simds"] / (rates["clock_GHz"] * 1e9) * 1e3
        result["alu"] = {
            "clock_GHz_under_load": rates["clock_GHz"],
            "cycles_per_wave64_instr": {k: rates[k]["cycles_per_unit"] for k in ("fma", "exp", "dpp_mul")},
            "cycles_per_scan_step": step_cycles,
            "alg_trans_lane_ops": ops[0], "alg_plain_lane_ops": ops[1],
            "floor_ms": floor, "frac": floor / kernel_ms,
            "scan_core_floor_ms": core, "scan_core_frac": core / kernel_ms,
            "probe": {k: rates[k] for k in ("fma", "exp", "dpp_mul", "scan_step")}}
    except Exception as e:
        rates = None
        result["alu_error"] = str(e)[:200]
    try:
        result["copy_probe_GBps"] = copy_probe(stream)
        result["roofline"]["frac_of_copy_probe"] = achieved / result["copy_probe_GBps"]
    except Exception as e:
        result["copy_probe_error"] = str(e)[:200]
    if not args.no_rows:
        log("other workloads")
        result["rows"] = bench_rows(stream)
        for row in result["rows"].values():
            if rates is not None and "alu_ops" in row:
                row["alu_floor_ms"] = alu_floor_ms(row["alu_ops"], rates)
                row["alu_frac"] = row["alu_floor_ms"] / row["ms"]
    if not args.no_cpu:
        log("cpu baseline (float64 oracle)")
        result["cpu_baseline"] = cpu_baseline()
        if "rows" in result:
            log("float64 oracle beside the other workloads")
            for k, v in cpu_rows(result["rows"]).items():
                result["rows"][k]["cpu_oracle"] = v
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
