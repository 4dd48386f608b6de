"""Decode over a paged KV cache with grouped query heads: parity against the fp64 oracle
(oracle.decode_paged), split-count invariance, the documented edge cases (empty sequence, block
ids out of range), and agreement with the contiguous decode when the cache is not paged."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from exact_attention_fa_amd import inputs
from tests.helpers import assert_fwd_close, default_scale, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _run(fa, q16, kc16, vc16, table, lens, splits=0, scale=None):
    import torch
    d = q16.shape[-1]
    o, lse = fa.decode_paged(to_dev(q16), to_dev(kc16), to_dev(vc16),
                             torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).cuda(),
                             torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).cuda(),
                             scale=scale or default_scale(d), num_splits=splits)
    torch.cuda.synchronize()
    return from_dev(o), lse.cpu().numpy().astype(np.float64)


def _case(seed, B, H, H_kv, d, bs, lens, max_blocks=None):
    max_blocks = max_blocks or max(1, -(-max(lens) // bs))
    q16 = inputs.tensor_bf16(seed, "q", B, H, 1, d)[:, :, 0, :].copy()
    kc, vc, table, sl = inputs.paged_kv_bf16(seed, B, H_kv, lens, d, bs, max_blocks)
    return q16, kc, vc, table, sl


def _oracle(q16, kc, vc, table, lens, scale):
    f = inputs.bf16_to_f64
    return oracle.decode_paged(f(q16), f(kc), f(vc), table, lens, scale)


CASES = [  # (B, H, H_kv, d, block_size, seq_lens)
    (3, 8, 8, 128, 16, [1, 37, 300]),        # multi-head, ragged lengths
    (2, 32, 8, 128, 16, [1000, 4097]),       # GQA, 4 query heads per K/V head
    (2, 16, 1, 64, 32, [513, 64]),           # MQA, 16 query heads on one K/V head
    (1, 12, 4, 64, 1, [77]),                 # block size 1, 3 heads per group
    (2, 6, 2, 128, 64, [5000, 1]),           # 3 heads per group, long and single position
    (2, 4, 2, 64, 128, [129, 255]),          # positions straddling large blocks
    # groups of 8 or more query heads run on the matrix cores
    (2, 64, 8, 128, 16, [1000, 4097]),       # 8 query heads per K/V head
    (2, 32, 1, 128, 16, [33, 2000]),         # MQA, one full block of 32 query heads
    (1, 40, 1, 64, 8, [300]),                # 40 heads: a full block and a block of 8
    (2, 16, 2, 64, 1, [77, 31]),             # block size 1, 8 heads per group
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}Hkv{}d{}bs{}".format(*c[:5]))
@pytest.mark.parametrize("splits", [0, 1, 5, 64])
def test_decode_paged_parity(gpu, case, splits):
    B, H, H_kv, d, bs, lens = case
    q16, kc, vc, table, sl = _case(70 + H + bs, B, H, H_kv, d, bs, lens)
    if splits > table.shape[1] * bs:  # more splits than positions: rejected before any launch
        with pytest.raises(gpu.FaError) as e:
            _run(gpu, q16, kc, vc, table, sl, splits)
        assert e.value.status == 8  # FA_ERR_ARG
        return
    o, lse = _run(gpu, q16, kc, vc, table, sl, splits)
    o_ref, l_ref = _oracle(q16, kc, vc, table, sl, default_scale(d))
    assert_fwd_close(o, lse, o_ref, l_ref, f"paged {case} C{splits}")


@pytest.mark.parametrize("heads", [(32, 8), (64, 4)], ids=["group4", "group16"])
def test_decode_paged_split_invariance(gpu, heads):
    H, H_kv = heads
    q16, kc, vc, table, sl = _case(81, 4, H, H_kv, 128, 16, [9000, 17, 4096, 2500])
    res = [_run(gpu, q16, kc, vc, table, sl, c) for c in (1, 3, 16, 100)]
    for o, l in res[1:]:
        assert np.max(np.abs(o - res[0][0])) <= 2 ** -7  # one bf16 ulp at |o| < 2
        assert np.max(np.abs(l - res[0][1])) <= 1e-5
    a = _run(gpu, q16, kc, vc, table, sl, 16)
    assert np.array_equal(a[0], res[2][0]) and np.array_equal(a[1], res[2][1])


def test_decode_paged_matches_contiguous_decode(gpu):
    """H_kv = H with the cache in sequence order (block i of sequence b = block b*max_blocks+i):
    the same numbers as the contiguous decode kernel to within a bf16 ulp."""
    import torch
    B, H, n, d, bs = 2, 4, 3000, 128, 16
    q16, k16, v16 = inputs.qkv_bf16(91, B, H, 1, n, d)
    mb = -(-n // bs)
    kc = np.zeros((B * mb, H, bs, d), dtype=np.uint16)
    vc = np.zeros_like(kc)
    pad = mb * bs - n
    kpad = np.concatenate([k16, np.zeros((B, H, pad, d), np.uint16)], axis=2)
    vpad = np.concatenate([v16, np.zeros((B, H, pad, d), np.uint16)], axis=2)
    kc[:] = kpad.reshape(B, H, mb, bs, d).transpose(0, 2, 1, 3, 4).reshape(B * mb, H, bs, d)
    vc[:] = vpad.reshape(B, H, mb, bs, d).transpose(0, 2, 1, 3, 4).reshape(B * mb, H, bs, d)
    table = np.arange(B * mb, dtype=np.int32).reshape(B, mb)
    o_p, l_p = _run(gpu, q16[:, :, 0, :].copy(), kc, vc, table, np.full(B, n, np.int32), 8)
    o_c, l_c = gpu.decode(to_dev(q16), to_dev(k16), to_dev(v16), num_splits=8)
    torch.cuda.synchronize()
    assert np.max(np.abs(o_p - from_dev(o_c)[:, :, 0, :])) <= 2 ** -7
    assert np.max(np.abs(l_p - l_c.cpu().numpy()[:, :, 0])) <= 1e-5


@pytest.mark.parametrize("heads", [(4, 2), (16, 2)], ids=["group2", "group8"])
def test_decode_paged_edge_cases(gpu, heads):
    """A sequence with no position gives o = 0, lse = -inf; a block id outside [0, num_blocks)
    reads as zero rows (its positions score 0 and contribute v = 0)."""
    B, (H, H_kv), d, bs = 3, heads, 128, 16
    q16, kc, vc, table, sl = _case(93, B, H, H_kv, d, bs, [40, 40, 40])
    sl = sl.copy()
    sl[1] = 0
    table = table.copy()
    bad = int(table[2, 1])
    table[2, 1] = kc.shape[0] + 5                     # out of range
    o, lse = _run(gpu, q16, kc, vc, table, sl)
    assert np.all(o[1] == 0.0) and np.all(np.isneginf(lse[1]))
    kc_ref, vc_ref = kc.copy(), vc.copy()
    zero = np.zeros((1,) + kc.shape[1:], np.uint16)  # the reading: that block is all zero
    kc_ref = np.concatenate([kc_ref, zero])
    vc_ref = np.concatenate([vc_ref, zero])
    table_ref = table.copy()
    table_ref[2, 1] = kc.shape[0]
    o_ref, l_ref = _oracle(q16, kc_ref, vc_ref, table_ref, sl, default_scale(d))
    keep = [0, 2]
    assert_fwd_close(o[keep], lse[keep], o_ref[keep], l_ref[keep], "paged edge cases")
    assert bad >= 0


@pytest.mark.parametrize("heads", [(32, 8), (64, 8)], ids=["group4", "group8"])
def test_decode_paged_serving_size(gpu, heads):
    """B8, 32768 positions per sequence (block size 16), d128, 4 or 8 query heads per K/V head:
    every (b, h) against the oracle."""
    B, (H, H_kv), d, bs, n = 8, heads, 128, 16, 32768
    q16, kc, vc, table, sl = _case(95, B, H, H_kv, d, bs, [n] * B)
    o, lse = _run(gpu, q16, kc, vc, table, sl)
    o_ref, l_ref = _oracle(q16, kc, vc, table, sl, default_scale(d))
    assert_fwd_close(o, lse, o_ref, l_ref, "paged serving size")
