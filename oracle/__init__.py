"""CPU fp64 oracle for exact attention. Test infrastructure: only tests, the smoke check and the
benchmark's CPU-baseline leg may use it; the product path never does."""
from .attention import (backward, backward_head, decode, forward, forward_head, scores,
                        softmax_rows, visible)

__all__ = ["backward", "backward_head", "decode", "forward", "forward_head", "scores",
           "softmax_rows", "visible"]
