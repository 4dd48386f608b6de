"""Exact attention for MI355X (gfx950): fused forward, backward by recomputation, and split-KV
decoding, as hand-written HIP kernels behind a C ABI (include/fa.h).

    from exact_attention_fa_amd import fwd, bwd, decode
"""
from ._lib import FaError, bwd, decode, decode_num_splits, fwd, load

__all__ = ["FaError", "bwd", "decode", "decode_num_splits", "fwd", "load"]
