"""Forward parity: the HIP kernel (through the C ABI) against the fp64 oracle on the same seeded
bf16 inputs, plus full-size checks that need no oracle."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from exact_attention_fa_amd import inputs
from tests.helpers import assert_fwd_close, default_scale, from_dev, to_dev

pytestmark = pytest.mark.gpu


def run_fwd(fa, q16, k16, v16, causal, scale):
    import torch
    q, k, v = to_dev(q16), to_dev(k16), to_dev(v16)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return from_dev(o), lse.cpu().numpy().astype(np.float64)


def full_parity(fa, seed, B, H, Nq, Nk, d, causal, scale=None):
    scale = default_scale(d) if scale is None else scale
    q16, k16, v16 = inputs.qkv_bf16(seed, B, H, Nq, Nk, d)
    o, lse = run_fwd(fa, q16, k16, v16, causal, scale)
    f = inputs.bf16_to_f64
    o_ref, l_ref = oracle.forward(f(q16), f(k16), f(v16), scale, causal)
    assert_fwd_close(o, lse, o_ref, l_ref, f"B{B} H{H} Nq{Nq} Nk{Nk} d{d} causal{causal}")


def test_c1_small(gpu):
    """B1 H1 N256 d64, non-causal, scale 1/8."""
    full_parity(gpu, 1, 1, 1, 256, 256, 64, False)


@pytest.mark.parametrize("causal", [False, True])
def test_c2(gpu, causal):
    """B4 H16 N2048 d128, non-causal and causal: every element against the oracle."""
    full_parity(gpu, 2, 4, 16, 2048, 2048, 128, causal)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 17, 64, 255, 257, 300])
def test_ragged_square(gpu, n, causal, d):
    full_parity(gpu, 100 + n, 2, 3, n, n, d, causal)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq,nk,causal", [(1, 300, True), (5, 77, True), (130, 1000, True),
                                          (200, 333, False), (333, 200, False), (1, 1, True),
                                          (129, 129, True), (64, 4097, True)])
def test_rectangular(gpu, nq, nk, causal, d):
    full_parity(gpu, 7, 1, 2, nq, nk, d, causal)


def test_scale_not_default(gpu):
    full_parity(gpu, 8, 1, 2, 200, 200, 64, True, scale=0.3)


def sampled_parity(fa, seed, B, H, N, d, causal, heads, rows):
    """Full-size launch; oracle on sampled (b, h, rows) only (rows are independent)."""
    import torch
    scale = default_scale(d)
    q16, k16, v16 = inputs.qkv_bf16(seed, B, H, N, N, d)
    q, k, v = to_dev(q16), to_dev(k16), to_dev(v16)
    o_t, lse_t = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    f = inputs.bf16_to_f64
    for b, h in heads:
        o = from_dev(o_t[b, h, rows])
        lse = lse_t[b, h, rows].cpu().numpy().astype(np.float64)
        o_ref, l_ref = oracle.forward_head(f(q16[b, h]), f(k16[b, h]), f(v16[b, h]), scale, causal,
                                           rows=rows)
        assert_fwd_close(o, lse, o_ref, l_ref, f"B{B} H{H} N{N} d{d} head ({b},{h})")
    return q, k, v, o_t, lse_t


def _rows(N, rng):
    r = np.unique(np.concatenate([[0, 1, 127, 128, N // 2, N - 129, N - 2, N - 1],
                                  rng.integers(0, N, 40)]))
    return r


@pytest.mark.slow
def test_c3_fwd_sampled(gpu):
    """B2 H16 N8192 d128 causal, at full size; sampled rows of four heads against the oracle."""
    rng = np.random.default_rng(3)
    sampled_parity(gpu, 3, 2, 16, 8192, 128, True, [(0, 0), (0, 9), (1, 7), (1, 15)], _rows(8192, rng))


@pytest.mark.slow
@pytest.mark.parametrize("H,d", [(32, 128), (64, 64)])
def test_c4_long_context_sampled(gpu, H, d):
    """B1 N32768 causal (H32 d128, and H64 d64), full size; sampled rows against the oracle."""
    rng = np.random.default_rng(4)
    sampled_parity(gpu, 4, 1, H, 32768, d, True, [(0, 0), (0, H - 1)], _rows(32768, rng))


def test_full_size_invariants(gpu):
    """No oracle needed: all V rows equal => every O row equals that row; Q = 0 => O is the
    running mean of V (causal) and L = ln(i + 1); bitwise repeatability."""
    import torch
    B, H, N, d = 2, 4, 4096, 128
    q16, k16, v16 = inputs.qkv_bf16(21, B, H, N, N, d)
    q, k = to_dev(q16), to_dev(k16)
    vrow = np.repeat(v16[:, :, :1], N, axis=2)
    o, _ = gpu.fwd(q, k, to_dev(vrow), causal=True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(from_dev(o), np.repeat(inputs.bf16_to_f64(v16[:, :, :1]), N, axis=2),
                               rtol=0, atol=1e-2)
    zq = torch.zeros_like(q)
    v = to_dev(v16)
    o, lse = gpu.fwd(zq, k, v, causal=True)
    torch.cuda.synchronize()
    vf = inputs.bf16_to_f64(v16)
    mean = np.cumsum(vf, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert np.max(np.abs(from_dev(o) - mean)) <= 1e-2
    np.testing.assert_allclose(lse.cpu().numpy(), np.log(np.arange(1, N + 1))[None, None, :].repeat(H, 1).repeat(B, 0),
                               rtol=1e-3, atol=1e-3)
    o1, l1 = gpu.fwd(q, k, v, causal=False)
    o2, l2 = gpu.fwd(q, k, v, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_causal_prefix_invariance(gpu):
    """Redrawing the second half of K/V leaves the first-half rows of O and L bitwise equal."""
    import torch
    B, H, N, d = 1, 4, 2048, 64
    q16, k16, v16 = inputs.qkv_bf16(22, B, H, N, N, d)
    k2, v2 = k16.copy(), v16.copy()
    k2[:, :, N // 2:] = inputs.tensor_bf16(99, "k", B, H, N - N // 2, d)
    v2[:, :, N // 2:] = inputs.tensor_bf16(99, "v", B, H, N - N // 2, d)
    q = to_dev(q16)
    o1, l1 = gpu.fwd(q, to_dev(k16), to_dev(v16), causal=True)
    o2, l2 = gpu.fwd(q, to_dev(k2), to_dev(v2), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, : N // 2], o2[:, :, : N // 2])
    assert torch.equal(l1[:, :, : N // 2], l2[:, :, : N // 2])
    assert not torch.equal(o1[:, :, N // 2:], o2[:, :, N // 2:])


def test_bad_arguments_raise(gpu):
    import torch
    q = torch.zeros((1, 1, 8, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu.FaError) as e:
        gpu.fwd(q, q, q)
    assert e.value.status == 3
