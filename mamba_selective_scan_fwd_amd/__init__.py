"""Mamba selective scan (S6) for AMD MI355X (gfx950): HIP kernels behind a C ABI.

``ss`` is the binding (fwd / step / bwd over libss.so); ``inputs`` draws the
seeded synthetic operands.
"""
from . import inputs  # noqa: F401
