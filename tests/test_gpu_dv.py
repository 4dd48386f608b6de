"""V with its own head dimension (d_v != d): fwd_dv / bwd_dv through the C ABI against the fp64
oracle (whose forward and backward take V's width from V) on the same seeded bf16 inputs."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from exact_attention_fa_amd import inputs
from tests.helpers import GRAD_REL_FRO, assert_fwd_close, default_scale, from_dev, rel_fro, to_dev

pytestmark = pytest.mark.gpu


def check(fa, seed, B, H, Nq, Nk, d, d_v, causal):
    import torch
    scale = default_scale(d)
    q16 = inputs.tensor_bf16(seed, "q", B, H, Nq, d)
    k16 = inputs.tensor_bf16(seed, "k", B, H, Nk, d)
    v16 = inputs.tensor_bf16(seed, "v", B, H, Nk, d_v)
    do16 = inputs.tensor_bf16(seed, "do", B, H, Nq, d_v)
    q, k, v, do = to_dev(q16), to_dev(k16), to_dev(v16), to_dev(do16)
    o, lse = fa.fwd_dv(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd_dv(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    f = inputs.bf16_to_f64
    what = f"B{B} H{H} {Nq}x{Nk} d{d} d_v{d_v} causal{causal}"
    o_ref, l_ref = oracle.forward(f(q16), f(k16), f(v16), scale, causal)
    assert_fwd_close(from_dev(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, what)
    ref = oracle.backward(f(q16), f(k16), f(v16), f(do16), scale, causal)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        e = rel_fro(from_dev(g), r)
        assert e <= GRAD_REL_FRO, f"{what}: {name} relative Frobenius error {e:.3e}"


@pytest.mark.parametrize("d,d_v", [(128, 64), (64, 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 17, 64, 255, 300])
def test_dv_ragged(gpu, n, causal, d, d_v):
    check(gpu, 110 + n, 2, 2, n, n, d, d_v, causal)


@pytest.mark.parametrize("d,d_v", [(128, 64), (64, 128)])
@pytest.mark.parametrize("nq,nk,causal", [(5, 77, True), (130, 1000, True), (333, 200, False)])
def test_dv_rectangular(gpu, nq, nk, causal, d, d_v):
    check(gpu, 111, 1, 2, nq, nk, d, d_v, causal)


@pytest.mark.parametrize("d,d_v", [(128, 64), (64, 128), (128, 128)])
def test_dv_b4_h16_n2048(gpu, d, d_v):
    check(gpu, 112, 4, 16, 2048, 2048, d, d_v, True)
