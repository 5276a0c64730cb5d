"""Hierarchical adaptive sparse attention for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libdash.so`` built from ``csrc/``; the
Python functions in :mod:`adaptive_sparse_long_amd.api` only marshal torch
tensors (device memory) and the current HIP stream into it.
"""
