"""Backward parity: dQ, dK, dV from the HIP kernels (fed with the GPU forward's O and LSE, as a
training step would) against the fp64 oracle's textbook chain rule, plus full-size invariants."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from exact_attention_fa_amd import inputs
from tests.helpers import GRAD_REL_FRO, default_scale, from_dev, rel_fro, to_dev

pytestmark = pytest.mark.gpu


def gpu_fwd_bwd(fa, q16, k16, v16, do16, causal, scale):
    import torch
    q, k, v, do = to_dev(q16), to_dev(k16), to_dev(v16), to_dev(do16)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_grads(got, ref, what):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        e = rel_fro(g, r)
        assert e <= GRAD_REL_FRO, f"{what}: {name} relative Frobenius error {e:.3e} > {GRAD_REL_FRO}"


def full_parity(fa, seed, B, H, Nq, Nk, d, causal, scale=None):
    scale = default_scale(d) if scale is None else scale
    q16, k16, v16 = inputs.qkv_bf16(seed, B, H, Nq, Nk, d)
    do16 = inputs.tensor_bf16(seed, "do", B, H, Nq, d)
    got = [from_dev(t) for t in gpu_fwd_bwd(fa, q16, k16, v16, do16, causal, scale)]
    f = inputs.bf16_to_f64
    ref = oracle.backward(f(q16), f(k16), f(v16), f(do16), scale, causal)
    check_grads(got, ref, f"B{B} H{H} Nq{Nq} Nk{Nk} d{d} causal{causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 17, 64, 255, 257, 300])
def test_bwd_ragged_square(gpu, n, causal, d):
    full_parity(gpu, 200 + n, 1, 2, n, n, d, causal)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq,nk,causal", [(1, 300, True), (5, 77, True), (130, 1000, True),
                                          (200, 333, False), (333, 200, False), (129, 129, True),
                                          (64, 4097, True)])
def test_bwd_rectangular(gpu, nq, nk, causal, d):
    full_parity(gpu, 9, 1, 2, nq, nk, d, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_c2_shape(gpu, causal):
    """B4 H16 N2048 d128 (the C2 shape) with gradients, every element against the oracle."""
    full_parity(gpu, 2, 4, 16, 2048, 2048, 128, causal)


@pytest.mark.slow
def test_c3_fwd_bwd_sampled_heads(gpu):
    """B2 H16 N8192 d128 causal at full size; whole gradients of three heads against the oracle,
    and gradient sum rules on every head."""
    import torch
    B, H, N, d = 2, 16, 8192, 128
    scale = default_scale(d)
    q16, k16, v16 = inputs.qkv_bf16(3, B, H, N, N, d)
    do16 = inputs.tensor_bf16(3, "do", B, H, N, d)
    dq, dk, dv = gpu_fwd_bwd(gpu, q16, k16, v16, do16, True, scale)
    f = inputs.bf16_to_f64
    for b, h in [(0, 0), (1, 5), (1, 15)]:
        ref = oracle.backward_head(f(q16[b, h]), f(k16[b, h]), f(v16[b, h]), f(do16[b, h]), scale, True)
        got = [from_dev(t[b, h]) for t in (dq, dk, dv)]
        check_grads(got, ref, f"C3 head ({b},{h})")
    # sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i on every head (fp32 sums of the bf16 outputs)
    dk_sum = dk.float().sum(dim=2)
    dv_sum = dv.float().sum(dim=2)
    do_sum = to_dev(do16).float().sum(dim=2)
    dk_scale = dk.float().abs().sum(dim=2)
    assert torch.all(dk_sum.abs() <= 2e-2 * dk_scale + 1e-3)
    assert torch.all((dv_sum - do_sum).abs() <= 2e-2 * dv.float().abs().sum(dim=2) + 1e-2)


def test_bwd_zero_dout_and_determinism(gpu):
    import torch
    B, H, N, d = 2, 4, 1000, 128
    q16, k16, v16 = inputs.qkv_bf16(31, B, H, N, N, d)
    do16 = inputs.tensor_bf16(31, "do", B, H, N, d)
    zeros = np.zeros_like(do16)
    g0 = gpu_fwd_bwd(gpu, q16, k16, v16, zeros, True, default_scale(d))
    assert all(int(torch.count_nonzero(t)) == 0 for t in g0)
    g1 = gpu_fwd_bwd(gpu, q16, k16, v16, do16, True, default_scale(d))
    g2 = gpu_fwd_bwd(gpu, q16, k16, v16, do16, True, default_scale(d))
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))


def test_bwd_bad_workspace_raises(gpu):
    import torch
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(gpu.FaError) as e:
        gpu.bwd(q, q, q, q, lse, q, workspace=ws)
    assert e.value.status == 6
