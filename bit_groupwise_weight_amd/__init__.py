"""Groupwise weight-only low-bit linear layer for AMD MI355X (gfx950).

The computation lives in the HIP library liblowbit.so (C ABI in
include/lowbit.h); `lowbit` is its Python binding.  Importing this package does
not load the library; the first call through `lowbit` does, and raises if the
library is not built.
"""
__all__ = ["lowbit", "nn", "workloads"]
