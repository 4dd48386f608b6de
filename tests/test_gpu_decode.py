"""Decode (split-KV) parity against the fp64 oracle, split-count invariance, and agreement with
the forward kernel at one query row."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from exact_attention_fa_amd import inputs
from tests.helpers import assert_fwd_close, default_scale, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _decode(fa, q16, k16, v16, splits=0, scale=None):
    import torch
    d = q16.shape[-1]
    o, lse = fa.decode(to_dev(q16), to_dev(k16), to_dev(v16), scale=scale or default_scale(d),
                       num_splits=splits)
    torch.cuda.synchronize()
    return from_dev(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nk", [1, 7, 64, 1000, 4097, 20000])
@pytest.mark.parametrize("splits", [0, 1, 2, 7, 16, 64])
def test_decode_parity(gpu, d, nk, splits):
    B, H = 2, 3
    q16, k16, v16 = inputs.qkv_bf16(50 + nk, B, H, 1, nk, d)
    if splits > nk:  # more splits than keys: rejected before any launch
        with pytest.raises(gpu.FaError) as e:
            _decode(gpu, q16, k16, v16, splits)
        assert e.value.status == 8  # FA_ERR_ARG
        return
    o, lse = _decode(gpu, q16, k16, v16, splits)
    f = inputs.bf16_to_f64
    o_ref, l_ref = oracle.decode(f(q16), f(k16), f(v16), default_scale(d))
    assert_fwd_close(o, lse, o_ref, l_ref, f"decode d{d} nk{nk} C{splits}")


def test_decode_split_invariance_and_fwd_agreement(gpu):
    import torch
    B, H, nk, d = 4, 8, 9000, 128
    q16, k16, v16 = inputs.qkv_bf16(61, B, H, 1, nk, d)
    res = [_decode(gpu, q16, k16, v16, c) for c in (1, 3, 16, 100)]
    for o, l in res[1:]:
        assert np.max(np.abs(o - res[0][0])) <= 2 ** -7  # one bf16 ulp at |o| < 2
        assert np.max(np.abs(l - res[0][1])) <= 1e-5
    o_f, l_f = gpu.fwd(to_dev(q16), to_dev(k16), to_dev(v16), causal=True)
    torch.cuda.synchronize()
    assert np.max(np.abs(from_dev(o_f) - res[0][0])) <= 2 ** -7
    assert np.max(np.abs(l_f.cpu().numpy() - res[0][1])) <= 1e-5
    a = _decode(gpu, q16, k16, v16, 16)
    assert np.array_equal(a[0], res[2][0]) and np.array_equal(a[1], res[2][1])


@pytest.mark.slow
def test_c5_full_size(gpu):
    """B8 H32, one query, KV length 65536, d128: every (b, h) against the oracle, one head slice
    at a time (K and V are 2^31 elements each)."""
    import torch
    B, H, nk, d = 8, 32, 65536, 128
    scale = default_scale(d)
    q16 = inputs.tensor_bf16(5, "q", B, H, 1, d)
    k16 = inputs.tensor_bf16(5, "k", B, H, nk, d)
    v16 = inputs.tensor_bf16(5, "v", B, H, nk, d)
    k, v = to_dev(k16), to_dev(v16)
    o_t, l_t = gpu.decode(to_dev(q16), k, v, scale=scale)
    torch.cuda.synchronize()
    o, lse = from_dev(o_t), l_t.cpu().numpy().astype(np.float64)
    f = inputs.bf16_to_f64
    o_ref = np.empty_like(o)
    l_ref = np.empty_like(lse)
    for b in range(B):
        for h in range(H):
            o_ref[b, h], l_ref[b, h] = oracle.forward_head(f(q16[b, h]), f(k16[b, h]), f(v16[b, h]),
                                                           scale, False)
    assert_fwd_close(o, lse, o_ref, l_ref, "C5 decode")
