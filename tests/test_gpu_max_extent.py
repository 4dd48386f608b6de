"""One head at the largest extent the library accepts: K and V of B = H = 1 with N_k = 2^23 - 64
keys at d = 128, i.e. 2^31 - 2^14 bytes each, just under the per-head limit of 2^31 bytes that
the host checks (the kernels address a head's rows through 32-bit offsets). The split-KV decode
and the forward with four query rows, causal and not, against the fp64 oracle at the parity
bars, so that every key tile up to the last one is read from where it lies."""
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
