"""Additive bias / masks on the scores: fwd_bias / bwd_bias through the C ABI against the fp64
oracle (oracle.forward_bias / backward_bias) on the same seeded bf16 inputs, for full,
broadcast and per-key biases, -inf masks (including rows masked entirely) and the causal mask on
top."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from exact_attention_fa_amd import inputs
from tests.helpers import GRAD_REL_FRO, assert_fwd_close, default_scale, from_dev, rel_fro, to_dev

pytestmark = pytest.mark.gpu

NEG_INF_BF16 = 0xFF80


def make_bias(seed, shape, mask_frac=0.0, masked_rows=()):
    """bf16 bias of `shape`: 2 N(0, 1), a fraction of entries set to -inf, and whole rows
    (index tuples into the leading dims + row) set to -inf."""
    g = np.random.default_rng(seed)
    u = inputs.bf16_round((2 * g.standard_normal(shape)).astype(np.float32))
    if mask_frac:
        u[g.random(shape) < mask_frac] = NEG_INF_BF16
    for idx in masked_rows:
        u[idx] = NEG_INF_BF16
    return u


def run(fa, q16, k16, v16, do16, b16, causal):
    import torch
    scale = default_scale(q16.shape[3])
    q, k, v, do = to_dev(q16), to_dev(k16), to_dev(v16), to_dev(do16)
    bias = to_dev(b16)
    o, lse = fa.fwd_bias(q, k, v, bias, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd_bias(q, k, v, o, lse, do, bias, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return (from_dev(o), lse.cpu().numpy().astype(np.float64),
            [from_dev(t) for t in (dq, dk, dv)], scale)


def check(fa, seed, B, H, Nq, Nk, d, causal, bshape, mask_frac=0.0, masked_rows=()):
    q16, k16, v16, do16 = inputs.qkv_bf16(seed, B, H, Nq, Nk, d, with_do=True)
    b16 = make_bias(seed, bshape, mask_frac, masked_rows)
    o, lse, grads, scale = run(fa, q16, k16, v16, do16, b16, causal)
    f = inputs.bf16_to_f64
    bias = f(b16)
    o_ref, l_ref = oracle.forward_bias(f(q16), f(k16), f(v16), bias, scale, causal)
    what = f"B{B} H{H} {Nq}x{Nk} d{d} causal{causal} bias{bshape}"
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: masked rows differ"
    assert np.all(o[empty] == 0.0), f"{what}: masked rows not zero"
    assert_fwd_close(o[~empty], lse[~empty], o_ref[~empty], l_ref[~empty], what)
    ref = oracle.backward_bias(f(q16), f(k16), f(v16), f(do16), bias, scale, causal)
    for name, g, r in zip(("dQ", "dK", "dV"), grads, ref):
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        e = rel_fro(g, r)
        assert e <= GRAD_REL_FRO, f"{what}: {name} relative Frobenius error {e:.3e}"
    if np.any(empty):
        assert np.all(grads[0][empty] == 0.0), f"{what}: dQ of masked rows not zero"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [17, 64, 255, 300])
def test_bias_full(gpu, n, causal, d):
    check(gpu, 80 + n, 2, 2, n, n, d, causal, (2, 2, n, n))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bias_broadcast_and_masks(gpu, causal, d):
    # one [Nq, Nk] bias for all batches and heads, 30 % masked, two rows masked entirely
    check(gpu, 90, 2, 3, 200, 333 if not causal else 333, d, causal, (200, 333), 0.3,
          masked_rows=[(5,), (150,)])
    # per-key bias (a key padding mask) for each batch: [B, 1, 1, Nk]
    check(gpu, 91, 2, 3, 130, 1000, d, causal, (2, 1, 1, 1000), 0.2)
    # per-head bias [1, H, Nq, Nk]
    check(gpu, 92, 2, 3, 257, 257, d, causal, (1, 3, 257, 257))


def test_bias_as_causal_mask(gpu):
    """A -inf bias above the diagonal, without the causal flag, gives the causal results."""
    import torch
    B, H, N, d = 1, 2, 300, 128
    q16, k16, v16, do16 = inputs.qkv_bf16(93, B, H, N, N, d, with_do=True)
    tri = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], NEG_INF_BF16, 0).astype(np.uint16)
    q, k, v, do = to_dev(q16), to_dev(k16), to_dev(v16), to_dev(do16)
    o1, l1 = gpu.fwd(q, k, v, causal=True)
    g1 = gpu.bwd(q, k, v, o1, l1, do, causal=True)
    o2, l2 = gpu.fwd_bias(q, k, v, to_dev(tri), causal=False)
    g2 = gpu.bwd_bias(q, k, v, o2, l2, do, to_dev(tri), causal=False)
    torch.cuda.synchronize()
    assert float((o1.float() - o2.float()).abs().max()) <= 1e-2
    assert float((l1 - l2).abs().max()) <= 1e-3 * max(1.0, float(l1.abs().max()))
    for a, b in zip(g1, g2):
        assert rel_fro(from_dev(b), from_dev(a)) <= GRAD_REL_FRO


def test_bias_b2_h8_n2048(gpu):
    check(gpu, 94, 2, 8, 2048, 2048, 128, True, (1, 8, 2048, 2048))
