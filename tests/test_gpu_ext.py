"""Variable lengths, grouped K/V heads and dropout in one call: fwd_ext / bwd_ext through the C
ABI against the fp64 oracle's forward_combined / backward_combined on the same seeded inputs.
Padding rows and keys of every input hold NaN and every output buffer starts as NaN, so a read of
padding or an unwritten row would show; padding rows must be exactly o = 0, lse = -inf, and
padding gradients exactly zero. With one option (or none) the call must give the dedicated entry
point's results bit for bit."""
from __future__ import annotations

import numpy as np
import pytest

import oracle.combined as OC
from exact_attention_fa_amd import inputs
from tests.helpers import GRAD_REL_FRO, assert_fwd_close, default_scale, from_dev, rel_fro, to_dev

pytestmark = pytest.mark.gpu


def _lens_dev(x):
    import torch
    return torch.as_tensor(np.asarray(x, dtype=np.int32)).cuda()


def run(fa, seed, B, H, H_kv, Nq, Nk, d, lens_q, lens_k, causal, p, dseed, offset):
    import torch
    scale = default_scale(d)
    q16 = inputs.tensor_bf16(seed, "q", B, H, Nq, d)
    do16 = inputs.tensor_bf16(seed, "do", B, H, Nq, d)
    k16 = inputs.tensor_bf16(seed, "k", B, H_kv, Nk, d)
    v16 = inputs.tensor_bf16(seed, "v", B, H_kv, Nk, d)
    if lens_q is not None:
        cq, ck = np.clip(lens_q, 0, Nq), np.clip(lens_k, 0, Nk)
        q16, do16 = inputs.fill_padding(q16, cq), inputs.fill_padding(do16, cq)
        k16, v16 = inputs.fill_padding(k16, ck), inputs.fill_padding(v16, ck)
    q, k, v, do = to_dev(q16), to_dev(k16), to_dev(v16), to_dev(do16)
    lq = _lens_dev(lens_q) if lens_q is not None else None
    lk = _lens_dev(lens_k) if lens_k is not None else None
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=q.device)
    fa.fwd_ext(q, k, v, lq, lk, p, dseed, offset, causal=causal, scale=scale, out=(o, lse))
    outs = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
    grads = fa.bwd_ext(q, k, v, o, lse, do, lq, lk, p, dseed, offset, causal=causal,
                       scale=scale, out=outs)
    torch.cuda.synchronize()
    f = inputs.bf16_to_f64
    args = (lens_q, lens_k, scale, causal, p, dseed, offset)
    ref = OC.forward_combined(f(q16), f(k16), f(v16), *args)
    ref_g = OC.backward_combined(f(q16), f(k16), f(v16), f(do16), *args)
    got = (from_dev(o), lse.cpu().numpy().astype(np.float64))
    return got, ref, tuple(from_dev(t) for t in grads), ref_g


def o_factor(p: float) -> float:
    # as in the dropout tests: O itself for p <= 0.5, (1 - p) O above
    return 1.0 if p <= 0.5 else 1.0 - p


def check(got, ref, got_g, ref_g, p, what, lens_q=None, lens_k=None):
    (o, lse), (o_ref, l_ref) = got, ref
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: rows with lse = -inf differ"
    assert np.all(o[empty] == 0.0), f"{what}: empty rows not zero"
    live = ~empty
    if np.any(live):
        assert_fwd_close(o[live] * o_factor(p), lse[live], o_ref[live] * o_factor(p), l_ref[live],
                         what)
    for name, g, r in zip(("dQ", "dK", "dV"), got_g, ref_g):
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        if lens_q is not None:  # rows past l_q (dQ), keys past l_k (dK, dV): exactly zero
            lens, n = (lens_q, g.shape[2]) if name == "dQ" else (lens_k, g.shape[2])
            for b, l_ in enumerate(lens):
                assert np.all(g[b, :, min(max(int(l_), 0), n):] == 0), f"{what}: {name} padding"
        e = rel_fro(g, r)
        assert e <= GRAD_REL_FRO, f"{what}: {name} relative Frobenius error {e:.3e}"


CASES = [  # (B, H, H_kv, N_q, N_k, lens_q, lens_k)
    (3, 4, 2, 300, 300, [300, 1, 177], [300, 0, 200]),    # l_q > l_k, an empty sequence
    (2, 6, 3, 257, 400, [257, 64], [400, 64]),
    (2, 4, 1, 130, 130, [129, 130], [130, 65]),           # multi-query
    (2, 2, 2, 200, 333, [200, 17], [333, 333]),           # one K/V head per query head
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.3])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}Hkv{}q{}k{}".format(*c[:5]))
def test_ext_ragged(gpu, case, p, causal, d):
    B, H, H_kv, Nq, Nk, lq, lk = case
    got, ref, got_g, ref_g = run(gpu, 600 + Nq, B, H, H_kv, Nq, Nk, d, lq, lk, causal, p,
                                 2**35 + 3, 9)
    check(got, ref, got_g, ref_g, p, f"{case} p{p} causal{causal} d{d}", lq, lk)


def test_ext_b4_h16_hkv4_n2048_lengths(gpu):
    """B4 H16 with 4 K/V heads, padded to 2048, lengths drawn on [1, 2048], causal, dropout
    p = 0.1: every element of O, LSE, dQ, dK, dV against the oracle."""
    lens = inputs.varlen_lengths(61, 4, 1, 2048)
    got, ref, got_g, ref_g = run(gpu, 61, 4, 16, 4, 2048, 2048, 128, lens, lens, True, 0.1,
                                 0xD00D, 4)
    check(got, ref, got_g, ref_g, 0.1, f"B4 H16 H_kv4 N2048 lengths {lens.tolist()}", lens,
          lens)


def test_ext_single_options_match_dedicated_entries(gpu):
    """One option at a time (or none) gives the dedicated entry point's results bit for bit."""
    import torch
    B, H, N, d = 2, 4, 300, 128
    q16, k16, v16, do16 = inputs.qkv_bf16(620, B, H, N, N, d, with_do=True)
    q, k, v, do = to_dev(q16), to_dev(k16), to_dev(v16), to_dev(do16)
    lens = _lens_dev([300, 123])

    def same(a, b):
        return all(torch.equal(x, y) for x, y in zip(a, b))
    o0 = gpu.fwd(q, k, v, causal=True)
    e0 = gpu.fwd_ext(q, k, v, causal=True)
    assert same(o0, e0)
    assert same(gpu.bwd(q, k, v, *o0, do, causal=True), gpu.bwd_ext(q, k, v, *e0, do, causal=True))
    o1 = gpu.fwd_varlen(q, k, v, lens, lens, causal=True)
    e1 = gpu.fwd_ext(q, k, v, lens, lens, causal=True)
    assert same(o1, e1)
    assert same(gpu.bwd_varlen(q, k, v, *o1, do, lens, lens, causal=True),
                gpu.bwd_ext(q, k, v, *e1, do, lens, lens, causal=True))
    o2 = gpu.fwd_dropout(q, k, v, 0.2, 77, 5, causal=True)
    e2 = gpu.fwd_ext(q, k, v, p_drop=0.2, seed=77, offset=5, causal=True)
    assert same(o2, e2)
    assert same(gpu.bwd_dropout(q, k, v, *o2, do, 0.2, 77, 5, causal=True),
                gpu.bwd_ext(q, k, v, *e2, do, p_drop=0.2, seed=77, offset=5, causal=True))
    kg, vg = k[:, :2].contiguous(), v[:, :2].contiguous()
    o3 = gpu.fwd_gqa(q, kg, vg, causal=True)
    e3 = gpu.fwd_ext(q, kg, vg, causal=True)
    assert same(o3, e3)
    assert same(gpu.bwd_gqa(q, kg, vg, *o3, do, causal=True),
                gpu.bwd_ext(q, kg, vg, *e3, do, causal=True))
    torch.cuda.synchronize()


def test_ext_rejects_one_length_array(gpu):
    B, H, N, d = 1, 2, 64, 64
    q16, k16, v16 = inputs.qkv_bf16(621, B, H, N, N, d)
    q, k, v = to_dev(q16), to_dev(k16), to_dev(v16)
    with pytest.raises(ValueError):
        gpu.fwd_ext(q, k, v, _lens_dev([64]), None)
