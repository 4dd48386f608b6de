"""fa_decode_noalloc (the decode with its partials in the library's own device array) through the
C ABI against fa_decode (workspace given by the caller) on the same inputs: bitwise equal at the
same split count, and within the parity bars of the oracle. Two calls in a row, the second
smaller, so that the second reads nothing the first left in the array; no allocation on the
call path when outputs are given."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from exact_attention_fa_amd import inputs
from tests.helpers import assert_fwd_close, default_scale, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _one(fa, seed, B, H, Nk, d, splits):
    import torch
    q16, k16, v16 = inputs.qkv_bf16(seed, B, H, 1, Nk, d)
    q, k, v = to_dev(q16), to_dev(k16), to_dev(v16)
    scale = default_scale(d)
    o_ref_t, l_ref_t = fa.decode(q, k, v, scale=scale, num_splits=splits)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, 1), float("nan"), dtype=torch.float32, device=q.device)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    fa.decode_noalloc(q, k, v, scale=scale, num_splits=splits, out=(o, lse))
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(o, o_ref_t) and torch.equal(lse, l_ref_t), "differs from fa_decode"
    f = inputs.bf16_to_f64
    o_or, l_or = oracle.decode(f(q16), f(k16), f(v16), scale)
    assert_fwd_close(from_dev(o), lse.cpu().numpy().astype(np.float64), o_or, l_or,
                     f"noalloc B{B} H{H} Nk{Nk} d{d} C{splits}")


def test_noalloc_matches_decode_twice_then_smaller(gpu):
    _one(gpu, 501, 4, 16, 9000, 128, 0)    # automatic split count (64 splits)
    _one(gpu, 502, 1, 3, 700, 64, 5)       # smaller: fewer heads, keys and splits


def test_noalloc_largest_and_refused(gpu):
    """The largest split count that fits the array at B8 H32 d128, and one that does not."""
    B, H, d = 8, 32, 128
    per = gpu.decode_workspace_bytes(B, H, 4096, d, 1)
    c = min(1024, gpu.DECODE_NOALLOC_SCRATCH_BYTES // per)
    while gpu.decode_workspace_bytes(B, H, 4096, d, c) > gpu.DECODE_NOALLOC_SCRATCH_BYTES:
        c -= 1
    _one(gpu, 503, B, H, 4096, d, c)
    q16, k16, v16 = inputs.qkv_bf16(504, B, H, 1, 4096, d)
    with pytest.raises(gpu.FaError) as e:
        gpu.decode_noalloc(to_dev(q16), to_dev(k16), to_dev(v16), num_splits=c + 1)
    assert e.value.status == 6  # FA_ERR_WORKSPACE
