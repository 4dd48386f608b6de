"""CPU fp64 oracle for exact attention. Test infrastructure: only tests, the smoke check and the
benchmark's CPU-baseline leg may use it; the product path never does."""
from .attention import (backward, backward_bias, backward_gqa, backward_head, backward_varlen,
                        decode, decode_paged, forward, forward_bias, forward_gqa, forward_head,
                        forward_varlen, gather_paged, kv_head_of, scores, softmax_rows, visible,
                        visible_varlen)
from .dropout import backward_dropout, dropout_keep, forward_dropout, keep_threshold, philox
from .fp8 import (e4m3_decode, e4m3_encode, e4m3_round, forward_fp8, hadamard_signs,
                  prepare_head, rotate, sylvester_hadamard)

__all__ = ["backward", "backward_bias", "backward_gqa", "forward_bias", "forward_gqa", "kv_head_of", "backward_head", "backward_varlen", "decode", "decode_paged", "forward",
           "forward_head", "forward_varlen", "gather_paged", "scores", "softmax_rows", "visible",
           "visible_varlen", "backward_dropout", "dropout_keep", "forward_dropout",
           "keep_threshold", "philox", "e4m3_decode", "e4m3_encode", "e4m3_round",
           "forward_fp8", "hadamard_signs", "prepare_head", "rotate", "sylvester_hadamard"]
