"""Grouped query heads in the forward and backward passes: fwd_gqa / bwd_gqa through the C ABI
against the fp64 oracle (oracle.forward_gqa / backward_gqa) on the same seeded bf16 inputs;
H_kv = H against the plain entry points; and a long-sequence case with the K/V heads spread over
the eight XCDs (the grouped workgroup order)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from exact_attention_fa_amd import inputs
from tests.helpers import GRAD_REL_FRO, assert_fwd_close, default_scale, from_dev, rel_fro, to_dev

pytestmark = pytest.mark.gpu


def _inputs(seed, B, H, H_kv, Nq, Nk, d):
    return (inputs.tensor_bf16(seed, "q", B, H, Nq, d), inputs.tensor_bf16(seed, "k", B, H_kv, Nk, d),
            inputs.tensor_bf16(seed, "v", B, H_kv, Nk, d), inputs.tensor_bf16(seed, "do", B, H, Nq, d))


def check(fa, seed, B, H, H_kv, Nq, Nk, d, causal):
    import torch
    scale = default_scale(d)
    q16, k16, v16, do16 = _inputs(seed, B, H, H_kv, Nq, Nk, d)
    q, k, v, do = to_dev(q16), to_dev(k16), to_dev(v16), to_dev(do16)
    o, lse = fa.fwd_gqa(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd_gqa(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    f = inputs.bf16_to_f64
    what = f"B{B} H{H} H_kv{H_kv} {Nq}x{Nk} d{d} causal{causal}"
    o_ref, l_ref = oracle.forward_gqa(f(q16), f(k16), f(v16), scale, causal)
    assert_fwd_close(from_dev(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, what)
    ref = oracle.backward_gqa(f(q16), f(k16), f(v16), f(do16), scale, causal)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        e = rel_fro(from_dev(g), r)
        assert e <= GRAD_REL_FRO, f"{what}: {name} relative Frobenius error {e:.3e}"


CASES = [  # (B, H, H_kv, Nq, Nk, d, causal)
    (1, 4, 2, 200, 200, 64, True),       # 2 query heads per K/V head, ragged length
    (2, 8, 2, 333, 333, 128, False),     # 4 per K/V head
    (1, 8, 1, 129, 300, 128, True),      # MQA, N_q < N_k (bottom-right causal)
    (2, 6, 3, 64, 64, 64, True),         # 2 per K/V head, one tile
    (1, 16, 8, 512, 512, 128, True),     # 8 K/V heads: the grouped XCD order
    (2, 16, 4, 300, 300, 64, False),     # 8 K/V heads over the batch, 4 query heads each
    (1, 3, 1, 1, 1, 128, False),         # one query, one key
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}Hkv{}_{}x{}_d{}_c{}".format(*c))
def test_gqa_parity(gpu, case):
    B, H, H_kv, Nq, Nk, d, causal = case
    check(gpu, 120 + H + Nq, B, H, H_kv, Nq, Nk, d, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_with_one_query_head_per_kv_head_is_plain(gpu, causal):
    """H_kv = H: the same kernels with groups of one, bitwise equal to fwd / bwd."""
    import torch
    q16, k16, v16, do16 = _inputs(130, 2, 4, 4, 257, 257, 128)
    q, k, v, do = to_dev(q16), to_dev(k16), to_dev(v16), to_dev(do16)
    a = gpu.fwd_gqa(q, k, v, causal=causal)
    b = gpu.fwd(q, k, v, causal=causal)
    ga = gpu.bwd_gqa(q, k, v, a[0], a[1], do, causal=causal)
    gb = gpu.bwd(q, k, v, b[0], b[1], do, causal=causal)
    torch.cuda.synchronize()
    for x, y in zip(a + ga, b + gb):
        assert torch.equal(x, y)


def test_gqa_long_sequence_grouped_order(gpu):
    """B1 H16 H_kv8, N 2048, d128, causal: 8 K/V heads, so the workgroups of each K/V head's two
    query heads go to one XCD; every head against the oracle."""
    check(gpu, 131, 1, 16, 8, 2048, 2048, 128, True)


def test_gqa_determinism(gpu):
    import torch
    q16, k16, v16, do16 = _inputs(132, 1, 8, 2, 700, 700, 128)
    q, k, v, do = to_dev(q16), to_dev(k16), to_dev(v16), to_dev(do16)
    o, lse = gpu.fwd_gqa(q, k, v, causal=True)
    g1 = gpu.bwd_gqa(q, k, v, o, lse, do, causal=True)
    g2 = gpu.bwd_gqa(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(g1, g2))


def test_gqa_bad_arguments_raise(gpu):
    import torch
    from exact_attention_fa_amd import FaError
    q = torch.zeros(1, 6, 64, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 4, 64, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(FaError):
        gpu.fwd_gqa(q, k, k)


def test_gqa_in_workgroup_sums(gpu):
    """B8 H16 H_kv8, N 4096, d128, causal: 8 x 8 K/V heads x 32 key tiles = 2048 workgroups, so
    the dK/dV pass sums each group in its workgroup (no partial rows: the workspace is the plain
    one). Checked on the first K/V head of the first sequence and its two query heads."""
    import torch
    B, H, H_kv, N, d = 8, 16, 8, 4096, 128
    assert gpu.bwd_gqa_workspace_bytes(B, H, H_kv, N, N, d) == gpu.bwd_workspace_bytes(B, H, N, N, d)
    scale = default_scale(d)
    q16, k16, v16, do16 = _inputs(133, B, H, H_kv, N, N, d)
    q, k, v, do = to_dev(q16), to_dev(k16), to_dev(v16), to_dev(do16)
    o, lse = gpu.fwd_gqa(q, k, v, causal=True, scale=scale)
    dq, dk, dv = gpu.bwd_gqa(q, k, v, o, lse, do, causal=True, scale=scale)
    torch.cuda.synchronize()
    f = inputs.bf16_to_f64
    sl_q, sl_kv = (slice(0, 1), slice(0, 2)), (slice(0, 1), slice(0, 1))
    o_ref, l_ref = oracle.forward_gqa(f(q16[sl_q]), f(k16[sl_kv]), f(v16[sl_kv]), scale, True)
    assert_fwd_close(from_dev(o[sl_q]), lse[sl_q].cpu().numpy().astype(np.float64), o_ref, l_ref,
                     "B8 H16 H_kv8 N4096, first group")
    ref = oracle.backward_gqa(f(q16[sl_q]), f(k16[sl_kv]), f(v16[sl_kv]), f(do16[sl_q]), scale, True)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq[sl_q], dk[sl_kv], dv[sl_kv]), ref):
        e = rel_fro(from_dev(g), r)
        assert e <= GRAD_REL_FRO, f"first group: {name} relative Frobenius error {e:.3e}"
