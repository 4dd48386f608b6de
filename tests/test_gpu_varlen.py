"""Variable-length batches: fwd_varlen / bwd_varlen through the C ABI against the fp64 oracle's
forward_varlen / backward_varlen on the same seeded inputs. Padding rows and keys of every input
hold NaN, so any read of them would show; output buffers start as NaN, so every padding row must
be written (o = 0, lse = -inf, zero gradients)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from exact_attention_fa_amd import inputs
from tests.helpers import GRAD_REL_FRO, assert_fwd_close, default_scale, from_dev, rel_fro, to_dev

pytestmark = pytest.mark.gpu


def _lens_dev(x):
    import torch
    return torch.as_tensor(np.asarray(x, dtype=np.int32)).cuda()


def run_varlen(fa, seed, B, H, Nq, Nk, d, lens_q, lens_k, causal, with_bwd=True, scale=None):
    import torch
    scale = default_scale(d) if scale is None else scale
    q16, k16, v16, do16 = inputs.qkv_bf16(seed, B, H, Nq, Nk, d, with_do=True)
    clamp_q = np.clip(lens_q, 0, Nq)
    clamp_k = np.clip(lens_k, 0, Nk)
    q16 = inputs.fill_padding(q16, clamp_q)
    do16 = inputs.fill_padding(do16, clamp_q)
    k16 = inputs.fill_padding(k16, clamp_k)
    v16 = inputs.fill_padding(v16, clamp_k)
    q, k, v, do = to_dev(q16), to_dev(k16), to_dev(v16), to_dev(do16)
    lq, lk = _lens_dev(lens_q), _lens_dev(lens_k)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=q.device)
    fa.fwd_varlen(q, k, v, lq, lk, causal=causal, scale=scale, out=(o, lse))
    grads = None
    if with_bwd:
        outs = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
        grads = fa.bwd_varlen(q, k, v, o, lse, do, lq, lk, causal=causal, scale=scale, out=outs)
    torch.cuda.synchronize()
    f = inputs.bf16_to_f64
    ref = oracle.forward_varlen(f(q16), f(k16), f(v16), lens_q, lens_k, scale, causal)
    ref_g = (oracle.backward_varlen(f(q16), f(k16), f(v16), f(do16), lens_q, lens_k, scale, causal)
             if with_bwd else None)
    got = (from_dev(o), lse.cpu().numpy().astype(np.float64))
    got_g = tuple(from_dev(t) for t in grads) if with_bwd else None
    return got, ref, got_g, ref_g


def check(got, ref, got_g, ref_g, lens_q, lens_k, what):
    (o, lse), (o_ref, l_ref) = got, ref
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: rows with lse = -inf differ"
    assert np.all(o[empty] == 0.0), f"{what}: empty rows not zero"
    live = ~empty
    if np.any(live):
        assert_fwd_close(o[live], lse[live], o_ref[live], l_ref[live], what)
    if got_g is None:
        return
    # exact zeros: dQ of rows with no softmax (padding, or no visible key); dK, dV of keys past
    # the sequence's key length, and of every key of a sequence with no query
    n_k = got_g[1].shape[2]
    dead_keys = np.zeros(got_g[1].shape[:3], dtype=bool)
    for b in range(len(lens_k)):
        lk = min(max(int(lens_k[b]), 0), n_k)
        dead_keys[b, :, lk:] = True
        if min(max(int(lens_q[b]), 0), o.shape[2]) == 0:
            dead_keys[b] = True
    for name, g, r, dead in zip(("dQ", "dK", "dV"), got_g, ref_g, (empty, dead_keys, dead_keys)):
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        assert np.all(g[dead] == 0.0), f"{what}: {name} of padding not zero"
        e = rel_fro(g, r)
        assert e <= GRAD_REL_FRO, f"{what}: {name} relative Frobenius error {e:.3e}"


CASES = [  # (B, H, Nq, Nk, lens_q, lens_k)
    (5, 2, 300, 300, [300, 1, 0, 257, 64], [300, 1, 0, 257, 64]),
    (6, 2, 200, 333, [200, 17, 130, 0, 5, 150], [333, 300, 129, 40, 0, 77]),
    (3, 2, 300, 100, [300, 50, 129], [100, 100, 128]),   # padded N_q > N_k
    (2, 3, 129, 129, [129, 129], [129, 129]),           # full lengths
    (3, 1, 64, 64, [0, 0, 0], [0, 0, 0]),               # nothing valid
    (3, 2, 70, 70, [90, -4, 70], [-1, 70, 200]),        # lengths clamped to [0, N]
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_varlen_parity(gpu, case, causal, d):
    B, H, Nq, Nk, lens_q, lens_k = CASES[case]
    got, ref, got_g, ref_g = run_varlen(gpu, 40 + case, B, H, Nq, Nk, d, np.array(lens_q),
                                        np.array(lens_k), causal)
    check(got, ref, got_g, ref_g, lens_q, lens_k, f"case {case} d{d} causal{causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_mixed_lengths_b4_h16_n2048(gpu, causal):
    """B4 H16 padded to 2048, d128, lengths drawn on [1, 2048]: every element against the
    oracle."""
    lens = inputs.varlen_lengths(5, 4, 1, 2048)
    got, ref, got_g, ref_g = run_varlen(gpu, 6, 4, 16, 2048, 2048, 128, lens, lens, causal)
    check(got, ref, got_g, ref_g, lens, lens, f"mixed {lens.tolist()} causal{causal}")


def test_varlen_full_lengths_match_dense(gpu):
    """With every length equal to N the variable-length entry points and fwd/bwd agree to the
    parity bar (both against the oracle) on a causal ragged shape."""
    import torch
    B, H, N, d = 2, 2, 257, 128
    q16, k16, v16, do16 = inputs.qkv_bf16(3, B, H, N, N, d, with_do=True)
    q, k, v, do = to_dev(q16), to_dev(k16), to_dev(v16), to_dev(do16)
    lens = _lens_dev([N] * B)
    o1, l1 = gpu.fwd(q, k, v, causal=True)
    o2, l2 = gpu.fwd_varlen(q, k, v, lens, lens, causal=True)
    g1 = gpu.bwd(q, k, v, o1, l1, do, causal=True)
    g2 = gpu.bwd_varlen(q, k, v, o2, l2, do, lens, lens, causal=True)
    torch.cuda.synchronize()
    assert float((o1.float() - o2.float()).abs().max()) <= 1e-2
    assert float((l1 - l2).abs().max()) <= 1e-3 * max(1.0, float(l1.abs().max()))
    for a, b in zip(g1, g2):
        e = rel_fro(from_dev(b), from_dev(a))
        assert e <= GRAD_REL_FRO
