"""One head at the largest extent the library accepts: K and V of B = H = 1 with N_k = 2^23 - 64
keys at d = 128, i.e. 2^31 - 2^14 bytes each, just under the per-head limit of 2^31 bytes that
the host checks (the kernels address a head's rows through 32-bit offsets). The split-KV decode
and the forward with four query rows, causal and not, against the fp64 oracle at the parity
bars, so that every key tile up to the last one is read from where it lies.

The grouped-query decodes address whole caches through 64-bit offsets: a contiguous cache whose
last K/V head starts past byte 2^31 of K and V, and a paged cache of more than 2^32 bytes whose
block table points at its last blocks, against the oracle on the heads and blocks that hold data
(the rest of each cache is zero)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from exact_attention_fa_amd import inputs
from tests.helpers import assert_fwd_close, default_scale, from_dev, to_dev

pytestmark = pytest.mark.gpu

D = 128
NK = (1 << 31) // (2 * D) - 64  # rows of one head: 2^31 - 2^14 bytes


@pytest.fixture(scope="module")
def big_kv():
    k16 = inputs.long_head_bf16(71, "k", NK, D)
    v16 = inputs.long_head_bf16(71, "v", NK, D)
    assert k16.nbytes < (1 << 31) and k16.nbytes > (1 << 31) - (1 << 15)
    f = inputs.bf16_to_f64
    return k16, v16, to_dev(k16), to_dev(v16), f(k16), f(v16)


@pytest.mark.parametrize("splits", [0, 1024])
def test_decode_largest_head(gpu, big_kv, splits):
    import torch
    _, _, k, v, kf, vf = big_kv
    q16 = inputs.tensor_bf16(71, "q", 1, 1, 1, D)
    o, lse = gpu.decode(to_dev(q16), k, v, scale=default_scale(D), num_splits=splits)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode(inputs.bf16_to_f64(q16), kf, vf, default_scale(D))
    assert_fwd_close(from_dev(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref,
                     f"decode N_k {NK} C {splits}")


@pytest.mark.parametrize("causal", [False, True])
def test_forward_largest_head(gpu, big_kv, causal):
    import torch
    _, _, k, v, kf, vf = big_kv
    q16 = inputs.tensor_bf16(72, "q", 1, 1, 4, D)
    o, lse = gpu.fwd(to_dev(q16), k, v, causal=causal, scale=default_scale(D))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.forward(inputs.bf16_to_f64(q16), kf, vf, default_scale(D), causal)
    assert_fwd_close(from_dev(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref,
                     f"forward N_q 4 N_k {NK} causal {causal}")


def test_backward_largest_head(gpu, big_kv):
    """Gradients of four query rows over the largest head: every dK/dV workgroup and the dQ
    pass's last key tiles sit near the end of the 2^31-byte range."""
    import torch
    from tests.helpers import GRAD_REL_FRO, rel_fro
    _, _, k, v, kf, vf = big_kv
    q16 = inputs.tensor_bf16(73, "q", 1, 1, 4, D)
    do16 = inputs.tensor_bf16(73, "do", 1, 1, 4, D)
    q, do = to_dev(q16), to_dev(do16)
    o, lse = gpu.fwd(q, k, v, causal=False, scale=default_scale(D))
    grads = gpu.bwd(q, k, v, o, lse, do, causal=False, scale=default_scale(D))
    torch.cuda.synchronize()
    f = inputs.bf16_to_f64
    ref = oracle.backward(f(q16), kf, vf, f(do16), default_scale(D), False)
    for name, g, r in zip(("dQ", "dK", "dV"), grads, ref):
        e = rel_fro(from_dev(g), r)
        assert e <= GRAD_REL_FRO, f"{name} relative Frobenius error {e:.3e} at N_k {NK}"


HKV_G, NK_G = 5, (1 << 21) + 77  # K/V head 4 starts 4 * NK_G * 256 bytes = 2^31 + 78848 bytes in


@pytest.mark.parametrize("splits", [0, 1])
def test_decode_gqa_head_past_2gib(gpu, splits):
    """fa_decode_gqa, 4 query heads per K/V head, over K and V [1, 5, 2^21 + 77, 128] (2.5 GiB
    each) with random data in the last K/V head only: its four query heads against the oracle;
    the others see all-zero keys and values, whose decode is exact (uniform weights over the
    N_k positions: O = 0, LSE = ln N_k)."""
    import torch
    G, d = 4, 128
    H = HKV_G * G
    assert (HKV_G - 1) * NK_G * d * 2 > (1 << 31)
    k16 = inputs.long_head_bf16(81, "k", NK_G, d)
    v16 = inputs.long_head_bf16(81, "v", NK_G, d)
    q16 = inputs.tensor_bf16(81, "q", 1, H, 1, d)
    k = torch.zeros((1, HKV_G, NK_G, d), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    k[0, HKV_G - 1] = to_dev(k16)[0, 0]
    v[0, HKV_G - 1] = to_dev(v16)[0, 0]
    o, lse = gpu.decode_gqa(to_dev(q16), k, v, scale=default_scale(d), num_splits=splits)
    torch.cuda.synchronize()
    o_h, l_h = from_dev(o), lse.cpu().numpy().astype(np.float64)
    del k, v
    f = inputs.bf16_to_f64
    kf, vf = f(k16), f(v16)
    h0 = (HKV_G - 1) * G
    for h in range(h0, H):
        o_ref, l_ref = oracle.decode(f(q16[:, h:h + 1]), kf, vf, default_scale(d))
        assert_fwd_close(o_h[:, h:h + 1], l_h[:, h:h + 1], o_ref, l_ref,
                         f"decode_gqa C {splits} query head {h} (K/V head {HKV_G - 1})")
    assert_fwd_close(o_h[:, :h0], l_h[:, :h0], np.zeros_like(o_h[:, :h0]),
                     np.full_like(l_h[:, :h0], np.log(NK_G)), f"decode_gqa C {splits} zero heads")


NB_P, HKV_P, BS_P = (1 << 19) + 100, 2, 16  # 8 KiB per block: the cache spans 2^32 + 800 KiB


@pytest.mark.parametrize("splits", [0, 1])
def test_decode_paged_blocks_past_4gib(gpu, splits):
    """fa_decode_paged over caches of 2^19 + 100 blocks (2 K/V heads, 16 positions, d = 128;
    more than 2^32 bytes each): sequence 0 reads the last 63 blocks of the cache in reverse
    order, sequence 1 blocks drawn from the whole cache; only those blocks hold data. Against
    the oracle on a compact copy of the same blocks under the same table."""
    import torch
    G, d, max_blocks = 4, 128, 64
    H = HKV_P * G
    assert NB_P * HKV_P * BS_P * d * 2 > (1 << 32)
    lens = np.array([1000, 1021], dtype=np.int32)
    table = np.zeros((2, max_blocks), dtype=np.int32)
    table[0, :63] = np.arange(NB_P - 1, NB_P - 64, -1)
    table[1] = np.random.default_rng(82).choice(NB_P, size=max_blocks, replace=False)
    used = np.unique(table)
    compact = np.searchsorted(used, table).astype(np.int32)  # the table over the compact copy
    kb16 = inputs.tensor_bf16(82, "k", len(used), HKV_P, BS_P, d)
    vb16 = inputs.tensor_bf16(82, "v", len(used), HKV_P, BS_P, d)
    q16 = inputs.tensor_bf16(82, "q", 2, H, 1, d)[:, :, 0, :].copy()
    idx = torch.from_numpy(used.astype(np.int64)).cuda()
    kc = torch.zeros((NB_P, HKV_P, BS_P, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kc[idx] = to_dev(kb16)
    vc[idx] = to_dev(vb16)
    o, lse = gpu.decode_paged(to_dev(q16), kc, vc, torch.from_numpy(table).cuda(),
                              torch.from_numpy(lens).cuda(), scale=default_scale(d),
                              num_splits=splits)
    torch.cuda.synchronize()
    o_h, l_h = from_dev(o), lse.cpu().numpy().astype(np.float64)
    del kc, vc
    f = inputs.bf16_to_f64
    o_ref, l_ref = oracle.decode_paged(f(q16), f(kb16), f(vb16), compact, lens, default_scale(d))
    assert_fwd_close(o_h, l_h, o_ref, l_ref, f"decode_paged C {splits} over {NB_P} blocks")

