"""Exact attention for MI355X (gfx950): fused forward, backward by recomputation, and split-KV
decoding (contiguous, with grouped query heads on a contiguous or a paged KV cache), also for batches of
different-length sequences, with grouped query heads, with an additive bias or mask, with
dropout on the probabilities, and an FP8 forward with incoherent processing, as hand-written HIP kernels behind a C ABI
(include/fa.h).

    from exact_attention_fa_amd import fwd, bwd, decode, decode_paged, fwd_varlen, bwd_varlen
"""
from ._lib import (FaError, bwd, bwd_bias, bwd_dropout, bwd_dv, bwd_gqa, bwd_gqa_workspace_bytes,
                   bwd_varlen, decode, decode_gqa, decode_gqa_num_splits,
                   decode_num_splits, decode_paged, decode_paged_num_splits, fwd, fwd_bias,
                   fwd_dropout, fwd_dv, fwd_fp8, fwd_gqa, fwd_varlen, load)

__all__ = ["FaError", "bwd", "bwd_bias", "bwd_dropout", "bwd_dv", "bwd_gqa", "bwd_gqa_workspace_bytes", "bwd_varlen",
           "decode", "decode_gqa", "decode_gqa_num_splits", "decode_num_splits", "decode_paged", "decode_paged_num_splits", "fwd",
           "fwd_bias", "fwd_dropout", "fwd_dv", "fwd_fp8", "fwd_gqa", "fwd_varlen", "load"]
