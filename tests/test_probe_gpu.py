"""The measurement utilities on the GPU: the issue-rate probe returns a shader-clock count and
a constant-clock count for every wave that give a plausible clock and instruction cost, and the
copy probe copies."""
import pytest
import torch

from _util import say

pytestmark = pytest.mark.gpu


def _ss():
    from mamba_selective_scan_fwd_amd import ss
    ss.load_library()
    return ss


@pytest.mark.parametrize("kind", ["fma", "exp", "dpp_mul", "scan_step"])
def test_alu_probe_records(kind):
    ss = _ss()
    say("alu probe %s" % kind)
    r = ss.alu_probe(kind, waves_per_simd=2, iters=512)
    assert 0.3 < r["clock_GHz"] < 4.0, r
    # a wave64 instruction takes at least one cycle of its SIMD and far less than 100
    assert 1.0 <= r["cycles_per_unit"] < 100.0, r
    # every wave is counted on exactly one SIMD
    assert sum(k * v for k, v in r["waves_per_simd_hist"].items()) == r["workgroups"] * 4, r


def test_alu_probe_lds_limits_sharing():
    """With 41 KB of LDS per workgroup at most three workgroups fit a CU's 160 KB, so no SIMD
    holds more than three of their waves."""
    ss = _ss()
    r = ss.alu_probe("fma", waves_per_simd=3, iters=64, lds_bytes=41 * 1024)
    say("waves per SIMD with 41 KB of LDS per workgroup: %s" % r["waves_per_simd_hist"])
    assert max(r["waves_per_simd_hist"]) <= 3, r


def test_copy_probe_copies():
    ss = _ss()
    src = torch.arange(1 << 16, dtype=torch.float32, device="cuda")
    dst = torch.zeros_like(src)
    ss.copy_probe(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
