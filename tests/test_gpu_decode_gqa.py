"""Decode with grouped query heads over a contiguous cache (fa_decode_gqa): parity against the
fp64 oracle (oracle.forward_gqa with one query row), split-count invariance, agreement with the
paged decode over the same positions, and a full-size launch checked on sampled heads."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from exact_attention_fa_amd import inputs
from tests.helpers import assert_fwd_close, default_scale, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _run(fa, q16, k16, v16, splits=0):
    import torch
    o, lse = fa.decode_gqa(to_dev(q16), to_dev(k16), to_dev(v16), num_splits=splits)
    torch.cuda.synchronize()
    return from_dev(o), lse.cpu().numpy().astype(np.float64)


def _case(seed, B, H, H_kv, Nk, d):
    q16 = inputs.tensor_bf16(seed, "q", B, H, 1, d)
    k16 = inputs.tensor_bf16(seed, "k", B, H_kv, Nk, d)
    v16 = inputs.tensor_bf16(seed, "v", B, H_kv, Nk, d)
    return q16, k16, v16


def _oracle(q16, k16, v16):
    f = inputs.bf16_to_f64
    return oracle.forward_gqa(f(q16), f(k16), f(v16), default_scale(q16.shape[-1]), False)


CASES = [  # (B, H, H_kv, N_k, d)
    (2, 8, 2, 1000, 128),     # 4 query heads per K/V head
    (1, 32, 1, 777, 64),      # multi-query: 32 heads, one full block of the instruction
    (2, 40, 1, 300, 128),     # 40 heads on one K/V head: a block of 32 and a block of 8
    (3, 12, 4, 31, 64),       # fewer positions than one 32-position tile
    (2, 6, 3, 4097, 128),     # 2 heads per group, a ragged last tile
    (2, 4, 4, 513, 64),       # H_kv = H: the multi-head decode
    (1, 16, 2, 1, 128),       # a single position
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}Hkv{}N{}d{}".format(*c))
@pytest.mark.parametrize("splits", [0, 1, 7, 64])
def test_decode_gqa_parity(gpu, case, splits):
    B, H, H_kv, Nk, d = case
    q16, k16, v16 = _case(90 + H + Nk, B, H, H_kv, Nk, d)
    if splits > Nk:  # more splits than positions: rejected before any launch
        with pytest.raises(gpu.FaError) as e:
            _run(gpu, q16, k16, v16, splits)
        assert e.value.status == 8  # FA_ERR_ARG
        return
    o, lse = _run(gpu, q16, k16, v16, splits)
    o_ref, l_ref = _oracle(q16, k16, v16)
    assert_fwd_close(o, lse, o_ref, l_ref, f"decode_gqa {case} splits {splits}")


def test_decode_gqa_split_invariance(gpu):
    """Every split count gives the same result within fp32 rounding of the combine."""
    q16, k16, v16 = _case(95, 2, 16, 2, 3000, 128)
    base_o, base_l = _run(gpu, q16, k16, v16, 1)
    for c in (2, 5, 16, 100, 1024):
        o, lse = _run(gpu, q16, k16, v16, c)
        assert np.max(np.abs(o - base_o)) <= 2 ** -7, f"splits {c}"
        assert np.max(np.abs(lse - base_l)) <= 1e-5, f"splits {c}"


def test_decode_gqa_matches_paged(gpu):
    """The contiguous cache laid out as blocks of 16 positions (block j of sequence b at block id
    b * blocks_per_seq + j) through fa_decode_paged gives the same outputs."""
    import torch
    B, H, H_kv, Nk, d, bs = 2, 16, 4, 1024, 128, 16
    q16, k16, v16 = _case(96, B, H, H_kv, Nk, d)
    o, lse = _run(gpu, q16, k16, v16, 16)
    nb = Nk // bs
    def paged(x):  # [B, H_kv, Nk, d] -> [B * nb, H_kv, bs, d]
        return np.ascontiguousarray(
            x.reshape(B, H_kv, nb, bs, d).transpose(0, 2, 1, 3, 4).reshape(B * nb, H_kv, bs, d))
    table = np.arange(B * nb, dtype=np.int32).reshape(B, nb)
    lens = np.full(B, Nk, dtype=np.int32)
    po, pl = gpu.decode_paged(to_dev(q16[:, :, 0, :].copy()), to_dev(paged(k16)), to_dev(paged(v16)),
                              torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(),
                              num_splits=16)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(po), o[:, :, 0, :])
    assert np.array_equal(pl.cpu().numpy().astype(np.float64), lse[:, :, 0])


def test_decode_gqa_serving_size(gpu):
    """B8 H32 with 8 K/V heads over 65536 positions (d128), launched whole with the automatic
    split count; sampled query heads checked against the oracle."""
    B, H, H_kv, Nk, d = 8, 32, 8, 65536, 128
    q16, k16, v16 = _case(97, B, H, H_kv, Nk, d)
    o, lse = _run(gpu, q16, k16, v16, 0)
    f = inputs.bf16_to_f64
    G = H // H_kv
    for b, h in [(0, 0), (3, 13), (7, 31)]:
        kv = h // G
        o_ref, l_ref = oracle.forward_gqa(f(q16[b:b + 1, h:h + 1]), f(k16[b:b + 1, kv:kv + 1]),
                                          f(v16[b:b + 1, kv:kv + 1]), default_scale(d), False)
        assert_fwd_close(o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], o_ref, l_ref,
                         f"serving size head ({b},{h})")
