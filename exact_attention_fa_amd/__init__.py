"""Exact attention for MI355X (gfx950): fused forward, backward by recomputation, and split-KV
decoding (contiguous, or over a paged KV cache with grouped query heads), as hand-written HIP
kernels behind a C ABI (include/fa.h).

    from exact_attention_fa_amd import fwd, bwd, decode, decode_paged
"""
from ._lib import (FaError, bwd, decode, decode_num_splits, decode_paged, decode_paged_num_splits,
                   fwd, load)

__all__ = ["FaError", "bwd", "decode", "decode_num_splits", "decode_paged",
           "decode_paged_num_splits", "fwd", "load"]
