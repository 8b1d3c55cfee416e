"""Exact attention for AMD Instinct MI355X (gfx950): forward and backward.

The computation runs in hand-written HIP kernels behind a C ABI (libfa.so,
declared in include/fa.h). This package holds:
  capi      ctypes binding with the C ABI's names (fa_fwd, fa_fwd_ex, fa_bwd, ...)
  ops       tensor-level helpers that allocate outputs with PyTorch and call capi
  inputs    seeded synthetic inputs (bf16 bit patterns) for tests and benchmarks
  build     builds libfa.so in-tree for gfx950
"""
__all__ = ["capi", "ops", "inputs", "build"]
