"""Mamba selective scan (S6) for AMD MI355X (gfx950): HIP kernels behind a C ABI."""
