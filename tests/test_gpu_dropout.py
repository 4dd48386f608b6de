"""Dropout on P: fwd_dropout / bwd_dropout through the C ABI against the fp64 oracle
(oracle.forward_dropout / backward_dropout, whose mask comes from the oracle's own Philox-4x32-10),
on the same seeded inputs. With V the identity (N_k = d) the forward's output is P Z / (1 - p)
itself, so the GPU's keep mask is compared bit for bit with the oracle's.

Tolerances: for p <= 0.5 the O bar (max abs 1e-2) is applied to O itself. At p = 0.9 it is
applied to (1 - p) O, the output before the inverted-dropout scale: that scale multiplies O, and
with it the bf16 step of every output element, by ten, so O's own rounding alone can exceed the
bar. The LSE and gradient bars (relative) are unchanged."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from exact_attention_fa_amd import inputs
from tests.helpers import GRAD_REL_FRO, assert_fwd_close, default_scale, from_dev, rel_fro, to_dev

pytestmark = pytest.mark.gpu

SEEDS = [(7, 0), (2**40 + 12345, 3), (0xFFFFFFFFFFFFFFFF, 2**32 - 1)]


def o_factor(p: float) -> float:
    """The factor O is compared under: 1 (O itself) for p <= 0.5, 1 - p above."""
    return 1.0 if p <= 0.5 else 1.0 - p


def _identity_v(B, H, n, d):
    v = np.zeros((B, H, n, d), dtype=np.uint16)
    idx = np.arange(n)
    v[:, :, idx, idx] = 0x3F80  # bf16 1.0
    return v


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
@pytest.mark.parametrize("si", range(len(SEEDS)))
def test_dropout_mask_bitwise(gpu, si, p, causal, d):
    import torch
    seed, offset = SEEDS[si]
    B, H = 2, 3
    Nk = d
    Nq = d if causal else 300
    q16 = inputs.tensor_bf16(30 + si, "q", B, H, Nq, d)
    k16 = inputs.tensor_bf16(30 + si, "k", B, H, Nk, d)
    v16 = _identity_v(B, H, Nk, d)
    o, lse = gpu.fwd_dropout(to_dev(q16), to_dev(k16), to_dev(v16), p, seed, offset, causal=causal)
    torch.cuda.synchronize()
    o = from_dev(o)
    scale = default_scale(d)
    f = inputs.bf16_to_f64
    for b in range(B):
        for h in range(H):
            z = oracle.dropout_keep(seed, offset, b * H + h, Nq, Nk, p)
            vis = oracle.visible(Nq, Nk, causal)
            got = o[b, h] != 0.0
            assert np.array_equal(got, z & vis), (b, h, int(np.sum(got != (z & vis))))
    o_ref, l_ref = oracle.forward_dropout(f(q16), f(k16), f(v16), scale, causal, p, seed, offset)
    fo = o_factor(p)
    assert_fwd_close(o * fo, lse.cpu().numpy().astype(np.float64), o_ref * fo, l_ref,
                     f"p{p} seed{si}")


def run(fa, seed_in, B, H, Nq, Nk, d, causal, p, seed, offset):
    import torch
    scale = default_scale(d)
    q16, k16, v16, do16 = inputs.qkv_bf16(seed_in, B, H, Nq, Nk, d, with_do=True)
    q, k, v, do = to_dev(q16), to_dev(k16), to_dev(v16), to_dev(do16)
    o, lse = fa.fwd_dropout(q, k, v, p, seed, offset, causal=causal)
    dq, dk, dv = fa.bwd_dropout(q, k, v, o, lse, do, p, seed, offset, causal=causal)
    torch.cuda.synchronize()
    got = [from_dev(o), lse.cpu().numpy().astype(np.float64)] + [from_dev(t) for t in (dq, dk, dv)]
    return got, (q16, k16, v16, do16), scale


def check_all(got, ins, scale, causal, p, seed, offset, what):
    f = inputs.bf16_to_f64
    q, k, v, do = (f(x) for x in ins)
    o_ref, l_ref = oracle.forward_dropout(q, k, v, scale, causal, p, seed, offset)
    assert_fwd_close(got[0] * o_factor(p), got[1], o_ref * o_factor(p), l_ref, what)
    ref = oracle.backward_dropout(q, k, v, do, scale, causal, p, seed, offset)
    for name, g, r in zip(("dQ", "dK", "dV"), got[2:], ref):
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        e = rel_fro(g, r)
        assert e <= GRAD_REL_FRO, f"{what}: {name} relative Frobenius error {e:.3e}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 17, 255, 300])
def test_dropout_ragged(gpu, n, causal, d):
    got, ins, scale = run(gpu, 60 + n, 2, 2, n, n, d, causal, 0.2, 99, 5)
    check_all(got, ins, scale, causal, 0.2, 99, 5, f"n{n} d{d} causal{causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq,nk,causal,p", [(5, 77, True, 0.3), (130, 1000, True, 0.1),
                                            (200, 333, False, 0.5), (333, 200, False, 0.1),
                                            (64, 4097, True, 0.3)])
def test_dropout_rectangular(gpu, nq, nk, causal, p, d):
    got, ins, scale = run(gpu, 61, 1, 2, nq, nk, d, causal, p, 2**33 + 5, 11)
    check_all(got, ins, scale, causal, p, 2**33 + 5, 11, f"{nq}x{nk} d{d} causal{causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_b2_h4_n2048(gpu, causal):
    got, ins, scale = run(gpu, 62, 2, 4, 2048, 2048, 128, causal, 0.1, 1234, 0)
    check_all(got, ins, scale, causal, 0.1, 1234, 0, f"B2 H4 N2048 causal{causal}")


def test_dropout_p0_is_plain_and_determinism(gpu):
    """p = 0 gives fa_fwd / fa_bwd bit for bit; a repeated call is bitwise identical; another
    seed or offset gives another mask."""
    import torch
    B, H, N, d = 1, 2, 300, 128
    q16, k16, v16, do16 = inputs.qkv_bf16(63, B, H, N, N, d, with_do=True)
    q, k, v, do = to_dev(q16), to_dev(k16), to_dev(v16), to_dev(do16)
    o0, l0 = gpu.fwd(q, k, v, causal=True)
    g0 = gpu.bwd(q, k, v, o0, l0, do, causal=True)
    o1, l1 = gpu.fwd_dropout(q, k, v, 0.0, 5, 0, causal=True)
    g1 = gpu.bwd_dropout(q, k, v, o1, l1, do, 0.0, 5, 0, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert all(torch.equal(a, b) for a, b in zip(g0, g1))
    oa, la = gpu.fwd_dropout(q, k, v, 0.3, 5, 1, causal=True)
    ga = gpu.bwd_dropout(q, k, v, oa, la, do, 0.3, 5, 1, causal=True)
    ob, lb = gpu.fwd_dropout(q, k, v, 0.3, 5, 1, causal=True)
    gb = gpu.bwd_dropout(q, k, v, ob, lb, do, 0.3, 5, 1, causal=True)
    oc, _ = gpu.fwd_dropout(q, k, v, 0.3, 6, 1, causal=True)
    od, _ = gpu.fwd_dropout(q, k, v, 0.3, 5, 2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(la, lb) and torch.equal(la, l0)
    assert all(torch.equal(a, b) for a, b in zip(ga, gb))
    assert not torch.equal(oa, oc) and not torch.equal(oa, od)


@pytest.mark.slow
def test_dropout_full_size_head(gpu):
    """B2 H16 N8192 d128 causal, p = 0.1, launched whole; one whole head's O, L and gradients
    against the oracle."""
    import torch
    B, H, N, d = 2, 16, 8192, 128
    p, seed, offset = 0.1, 77, 9
    scale = default_scale(d)
    q16, k16, v16, do16 = inputs.qkv_bf16(3, B, H, N, N, d, with_do=True)
    q, k, v, do = to_dev(q16), to_dev(k16), to_dev(v16), to_dev(do16)
    o, lse = gpu.fwd_dropout(q, k, v, p, seed, offset, causal=True)
    dq, dk, dv = gpu.bwd_dropout(q, k, v, o, lse, do, p, seed, offset, causal=True)
    torch.cuda.synchronize()
    b, h = 1, 7
    f = inputs.bf16_to_f64
    sl = [f(x[b:b + 1, h:h + 1]) for x in (q16, k16, v16, do16)]
    ids = np.array([[b * H + h]])
    o_ref, l_ref = oracle.forward_dropout(*sl[:3], scale, True, p, seed, offset, head_ids=ids)
    assert_fwd_close(from_dev(o[b:b + 1, h:h + 1]) * o_factor(p),
                     lse[b:b + 1, h:h + 1].cpu().numpy().astype(np.float64), o_ref * o_factor(p),
                     l_ref, "full-size head")
    ref = oracle.backward_dropout(*sl, scale, True, p, seed, offset, head_ids=ids)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        e = rel_fro(from_dev(g[b:b + 1, h:h + 1]), r)
        assert e <= GRAD_REL_FRO, f"{name} relative Frobenius error {e:.3e}"
