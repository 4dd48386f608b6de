"""CPU fp64 oracle for exact attention. Test infrastructure: only tests, the smoke check and the
benchmark's CPU-baseline leg may use it; the product path never does."""
from .attention import (backward, backward_head, decode, decode_paged, forward, forward_head,
                        gather_paged, scores, softmax_rows, visible)

__all__ = ["backward", "backward_head", "decode", "decode_paged", "forward", "forward_head",
           "gather_paged", "scores", "softmax_rows", "visible"]
