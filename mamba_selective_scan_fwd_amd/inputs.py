"""Seeded synthetic inputs for the selective scan.

This module holds no arithmetic of the scan itself: it only draws random
operands in a fixed order and rounds them to the I/O precision.  It is the one
module that both the HIP path's tests/bench and the float64 oracle's callers
use, so that both sides see identical inputs.

Recipe (one ``numpy.random.default_rng(seed)`` per problem, draws in float64
in this order, then round-to-nearest-even to the I/O dtype):

1. u      ~ N(0,1)  (B, D, L)
2. delta  ~ N(0,1)  (B, D, L)
3. z      ~ N(0,1)  (B, D, L)
4. Bm     ~ N(0,1)  (B, N, L)
5. Cm     ~ N(0,1)  (B, N, L)
6. D      ~ N(0,1)  (D,), fp32
7. dt0    = exp(U(ln 1e-3, ln 1e-1)) (D,); bias = log(expm1(dt0)), fp32, so
   that softplus(bias) = dt0 (the usual dt initialisation of a Mamba layer)
8. lengths ~ integers U[1, L] (B,), only when ragged
9. dy     ~ N(0,1)  (B, D, L), only when a backward is wanted
10. decode tokens: per step u_t, delta_t, z_t (B, D) and B_t, C_t (B, N)

A is not drawn: A[d, n] = -(n+1) in fp32 ("neg_n1"), or for the A_log
parameterisation ("a_log") A = -exp(A_log) with A_log[d, n] = log(n+1),
evaluated in float64 and rounded to fp32.

Every tensor is returned on the CPU; callers move what they need to a device.
"""
from __future__ import annotations

import math

import numpy as np
import torch

IO_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _round(arr: np.ndarray, io: str) -> torch.Tensor:
    """Round float64 draws to the I/O dtype (round-to-nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(IO_DTYPES[io]).contiguous()


def make_A(dim: int, dstate: int, mode: str = "neg_n1") -> torch.Tensor:
    n1 = np.arange(1, dstate + 1, dtype=np.float64)
    if mode == "neg_n1":
        a = -np.broadcast_to(n1, (dim, dstate))
    elif mode == "a_log":
        a = -np.exp(np.broadcast_to(np.log(n1), (dim, dstate)))
    else:
        raise ValueError("unknown A mode %r" % mode)
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32)


def make_problem(batch: int, dim: int, dstate: int, seqlen: int, io: str = "f32", seed: int = 0, *,
                 A_mode: str = "neg_n1", ragged: bool = False, with_dy: bool = False,
                 decode_steps: int = 0, with_D: bool = True, with_z: bool = True,
                 with_bias: bool = True) -> dict:
    """Draw one problem.  Optional operands are always drawn (so the draw order
    never depends on the flags) and then dropped when not wanted."""
    if io not in IO_DTYPES:
        raise ValueError("io must be one of %s" % sorted(IO_DTYPES))
    rng = np.random.default_rng(seed)
    act = (batch, dim, seqlen)
    bc = (batch, dstate, seqlen)
    p = {"batch": batch, "dim": dim, "dstate": dstate, "seqlen": seqlen, "io": io, "seed": seed}
    p["u"] = _round(rng.standard_normal(act), io)
    p["delta"] = _round(rng.standard_normal(act), io)
    z = _round(rng.standard_normal(act), io)
    p["Bm"] = _round(rng.standard_normal(bc), io)
    p["Cm"] = _round(rng.standard_normal(bc), io)
    Dv = torch.from_numpy(rng.standard_normal(dim)).to(torch.float32)
    dt0 = np.exp(rng.uniform(math.log(1e-3), math.log(1e-1), size=dim))
    bias = torch.from_numpy(np.log(np.expm1(dt0))).to(torch.float32)
    lengths = None
    if ragged:
        lengths = torch.from_numpy(rng.integers(1, seqlen, size=batch, endpoint=True)).to(torch.int32)
    dy = _round(rng.standard_normal(act), io) if with_dy else None
    steps = []
    for _ in range(decode_steps):
        steps.append({
            "u_t": _round(rng.standard_normal((batch, dim)), io),
            "delta_t": _round(rng.standard_normal((batch, dim)), io),
            "z_t": _round(rng.standard_normal((batch, dim)), io),
            "B_t": _round(rng.standard_normal((batch, dstate)), io),
            "C_t": _round(rng.standard_normal((batch, dstate)), io),
        })
    p["z"] = z if with_z else None
    p["D"] = Dv if with_D else None
    p["bias"] = bias if with_bias else None
    p["A"] = make_A(dim, dstate, A_mode)
    p["lengths"] = lengths
    p["dy"] = dy
    p["decode"] = steps
    return p


# Packed-document layouts ("niverel-mamba" README, "seq_idx strict reset"
# names nine structural cases).  Each case gives, per batch row, the list of
# document lengths (summing to L); consecutive documents get distinct ids.
SEQ_CASES = ("single_document", "length1_docs", "consecutive_boundaries", "tile_edges", "inside_one_tile",
             "misaligned_rows", "terminal_padding", "nonzero_first_id", "many_short_docs")


def _doc_lengths(case: str, b: int, L: int, rng) -> list:
    def fill(first, total=L):
        out, tot = [], 0
        for x in first:
            x = min(x, total - tot)
            if x > 0:
                out.append(x)
                tot += x
        if tot < total:
            out.append(total - tot)
        return out
    if case == "single_document":      # the only boundary is position 0
        return [L]
    if case == "length1_docs":
        return fill([1, 3, 1, 1, 7, 1] * (L // 14 + 1))
    if case == "consecutive_boundaries":
        return fill([5, 1, 1, 1, 1, 9, 1, 1])
    if case == "tile_edges":           # boundaries on 16-step block and 64-step tile edges
        return fill([16, 48, 64, 128, 32, 16])
    if case == "inside_one_tile":      # a document strictly inside one 64-step tile
        return fill([70, 20, 40])
    if case == "misaligned_rows":      # every row cut elsewhere
        return fill([int(x) for x in rng.integers(1, max(2, L // 3), size=8)])
    if case == "terminal_padding":     # documents, then a padding segment (id -1)
        if L < 2:
            return [L]
        pad = max(1, L // 4)
        return fill([int(x) for x in rng.integers(1, max(2, L // 2), size=3)], L - pad) + [pad]
    if case == "nonzero_first_id":
        return fill([L // 3, L // 3])
    if case == "many_short_docs":
        return fill([int(x) for x in rng.integers(1, 9, size=L)])
    raise ValueError("unknown seq_idx case %r" % case)


def make_seq_idx(case: str, batch: int, seqlen: int, seed: int = 0) -> torch.Tensor:
    """Document ids (B, L) int32 for one of SEQ_CASES, from a seeded generator."""
    rng = np.random.default_rng(seed)
    out = np.empty((batch, seqlen), dtype=np.int32)
    for b in range(batch):
        lens = _doc_lengths(case, b, seqlen, rng)
        first = 7 + 3 * b if case == "nonzero_first_id" else 0
        t = 0
        for k, ln in enumerate(lens):
            pad = case == "terminal_padding" and k == len(lens) - 1 and len(lens) > 1
            out[b, t:t + ln] = -1 if pad else first + k
            t += ln
        assert t == seqlen
    return torch.from_numpy(out)


def packed_documents(seqlen: int, batch: int, max_len: int, seed: int) -> torch.Tensor:
    """Rows packed with documents of length U[1, max_len] (ids 0, 1, 2, ...), int32 (B, L)."""
    rng = np.random.default_rng(seed)
    out = np.empty((batch, seqlen), dtype=np.int32)
    for b in range(batch):
        t, k = 0, 0
        while t < seqlen:
            ln = int(rng.integers(1, max_len, endpoint=True))
            out[b, t:t + ln] = k
            t += ln
            k += 1
    return torch.from_numpy(out)


# The five synthetic workloads: shapes of the pages' long-sequence throughput
# run (B=1, D=16, N=16, L=32k) and of mamba-130m / mamba-2.8b layers.
CONFIGS = {
    0: dict(batch=1, dim=16, dstate=16, seqlen=2048, io="f32"),
    1: dict(batch=1, dim=16, dstate=16, seqlen=32768, io="f32"),
    2: dict(batch=8, dim=1536, dstate=16, seqlen=2048, io="f16", A_mode="a_log", decode_steps=64),
    3: dict(batch=4, dim=5120, dstate=16, seqlen=8192, io="bf16", ragged=True),
    4: dict(batch=4, dim=1536, dstate=16, seqlen=4097, io="f32", with_dy=True),
}

CONFIG_NAMES = {
    0: "fwd fp32 B=1 D=16 N=16 L=2048",
    1: "fwd fp32 B=1 D=16 N=16 L=32768",
    2: "fwd fp16 B=8 D=1536 N=16 L=2048 (mamba-130m layer) + 64 decode steps",
    3: "fwd bf16 B=4 D=5120 N=16 L=8192 ragged (mamba-2.8b layer)",
    4: "bwd fp32 B=4 D=1536 N=16 L=4097",
}


def make_config(k: int, **overrides) -> dict:
    """Problem for workload k with seed k (overrides change shape/flags)."""
    kw = dict(CONFIGS[k])
    kw.update(overrides)
    kw.setdefault("seed", k)
    return make_problem(**kw)


def to_f64(t):
    """Widen a (CPU or device) tensor to a float64 numpy array; None passes through."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
