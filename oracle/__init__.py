"""CPU oracle for hierarchical adaptive sparse attention (test infrastructure).

This package is a plain, slow, float64 NumPy statement of what the GPU library
computes. It exists only to check the GPU library: the tests, the smoke check and
the CPU-baseline leg of the benchmark may import it; the product path never does.
It shares no code with the HIP library (no kernels, headers, helpers, tables or
pre/post-processing). Every function cites the passage of the pages it follows:

* "DashAttention: Differentiable and Adaptive Sparse Hierarchical Attention"
  (the DashAttention README page): "Usage", "How it works" items 1-3, "Core API".
* "AdaSplash: Adaptive Sparse Flash Attention" (the AdaSplash README page):
  "Usage" (Triton Entmax, AdaSplash with Block Masking), "Key Features".

The alpha-entmax mapping itself is named but not defined on the pages; the oracle
uses the published definition (Peters, Niculae & Martins, "Sparse
Sequence-to-Sequence Models", ACL 2019; Blondel, Martins & Niculae, "Learning
Classifiers with Fenchel-Young Losses", AISTATS 2019), which the AdaSplash paper
linked from its README builds on.
"""

from .entmax import (
    entmax_threshold,
    entmax,
    entmax_backward,
    entmax_threshold_bruteforce,
)
from .dash import (
    DashParams,
    chunk_summary,
    chunk_summary_backward,
    chunk_summaries,
    route_row,
    dash_rows,
    dash_prefill,
    dash_decode,
    dash_backward,
)
from .entmax_attention import entmax_attention, entmax_attention_rows, entmax_attention_backward

__all__ = [
    "entmax_threshold",
    "entmax",
    "entmax_backward",
    "entmax_threshold_bruteforce",
    "DashParams",
    "chunk_summary",
    "chunk_summary_backward",
    "chunk_summaries",
    "route_row",
    "dash_rows",
    "dash_prefill",
    "dash_decode",
    "dash_backward",
    "entmax_attention",
    "entmax_attention_rows",
    "entmax_attention_backward",
]
