"""The online softmax's rescaling under scores whose running maximum moves ([MW] "Online
Softmax": when a block raises a row's maximum, the running sum and output are multiplied by
exp(m_old - m_new)). iid N(0, 1) inputs at scale 1/sqrt(d) move the maximum almost only in the
first key block, so these cases force it:

* rising keys (inputs.rising_keys): Q's column 0 is 3 and K's column 0 grows linearly with the key
  index, so every query's scores grow along the keys and its maximum rises on every 64-key block,
  by 3 or by 12 in log2 units per block. The forward moves its reference when a lane's
  probabilities of a block sum past 2^8 (or, in the forms that take the maximum first, when the
  maximum passes the reference by 8): with 3 per block that happens every second or third block,
  before any single probability reaches 2^8, with 12 on every block;
* a peaked softmax: iid inputs at scale 1 with d = 128 (score standard deviation about 11, in
  log2 units about 16), where the maximum jumps by large, irregular amounts. O is then close to
  single V rows, so V is scaled by 1/4 (exactly, in bf16): at |O| >= 2.5 the bf16 step of O alone
  would exceed the O bar. V plays no part in the row maximum.

Forward, backward, decode and paged decode against the fp64 oracle at the parity bars, with one
derived exception. A key ramp steep enough to move the maximum on every block puts a large common
offset on K's column 0 (hundreds), while dQ_i = scale sum_j dS_ij K_j is a small difference
around that offset (the rows of dS sum to zero). Two roundings that any bf16 backward makes are
amplified by the offset: O is stored in bf16, so D = rowsum(dO * O) misses rowsum(P * dP) by a
bf16 step, and dS enters the dS K product as a bf16 matrix operand. On the rising-key cases dQ is
therefore held to max(2e-2, 1.5 x the error of the exact chain rule with just those two roundings)
(dq_floor below; about 6e-2 for 12 per block over 1000 keys), dK and dV to the plain bar."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from exact_attention_fa_amd import inputs
from tests.helpers import GRAD_REL_FRO, assert_fwd_close, default_scale, from_dev, rel_fro, to_dev

pytestmark = pytest.mark.gpu

LOG2E = 1.0 / math.log(2.0)


def per_key_for(rise_per_block: float, scale: float, q_value: float = 3.0,
                block: int = 64) -> float:
    """K column-0 step per key that raises every score by `rise_per_block` log2 units per block."""
    return rise_per_block / (q_value * block * scale * LOG2E)


def quarter(u16):
    """bf16 values divided by 4 (exact: only the exponent changes for these magnitudes)."""
    return inputs.bf16_round((inputs.bf16_to_f32(u16) * np.float32(0.25)).astype(np.float32))


def make_case(kind, seed, B, H, n_q, n_k, d):
    q16, k16, v16, do16 = inputs.qkv_bf16(seed, B, H, n_q, n_k, d, with_do=True)
    if kind == "peaked":
        return (q16, k16, quarter(v16), do16), 1.0
    scale = default_scale(d)
    rise = {"rise3": 3.0, "rise12": 12.0}[kind]
    q16, k16 = inputs.rising_keys(q16, k16, per_key_for(rise, scale))
    return (q16, k16, v16, do16), scale


CASES = [("rise3", 1, 2, 1000, 1000, 128, True), ("rise3", 1, 2, 300, 700, 64, False),
         ("rise12", 1, 2, 1000, 1000, 128, True), ("rise12", 2, 1, 513, 513, 64, True),
         ("rise12", 1, 2, 257, 1100, 128, False), ("peaked", 1, 2, 1000, 1000, 128, True),
         ("peaked", 2, 2, 300, 300, 128, False), ("peaked", 1, 2, 700, 700, 64, True)]


def _bf16(x):
    return inputs.bf16_to_f64(inputs.bf16_round(np.asarray(x, dtype=np.float32)))


def dq_floor(q, k, v, do, scale, causal, dq_ref):
    """Relative Frobenius error of dQ from the exact chain rule (fp64, oracle.scores for S and the
    mask) with D taken from the bf16-rounded O and dS rounded to bf16 before the dS K product."""
    num = den = 0.0
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            s = oracle.scores(q[b, h], k[b, h], scale, causal)
            p = np.exp(s - np.max(s, axis=1, keepdims=True))
            p /= np.sum(p, axis=1, keepdims=True)
            o = p @ v[b, h]
            dp = do[b, h] @ v[b, h].T
            ds = p * (dp - np.sum(do[b, h] * _bf16(o), axis=1, keepdims=True))
            dq = scale * (_bf16(ds) @ k[b, h])
            num += float(np.sum((dq - dq_ref[b, h]) ** 2))
            den += float(np.sum(dq_ref[b, h] ** 2))
    return math.sqrt(num / den)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "{}-B{}H{}q{}k{}d{}c{}".format(*c))
def test_rescale_fwd_bwd(gpu, case):
    import torch
    kind, B, H, n_q, n_k, d, causal = case
    (q16, k16, v16, do16), scale = make_case(kind, 400 + n_q + d, B, H, n_q, n_k, d)
    q, k, v, do = (to_dev(x) for x in (q16, k16, v16, do16))
    o, lse = gpu.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = gpu.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    f = inputs.bf16_to_f64
    o_ref, l_ref = oracle.forward(f(q16), f(k16), f(v16), scale, causal)
    assert_fwd_close(from_dev(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref,
                     f"{case} forward")
    ref = oracle.backward(f(q16), f(k16), f(v16), f(do16), scale, causal)
    bars = {"dQ": GRAD_REL_FRO, "dK": GRAD_REL_FRO, "dV": GRAD_REL_FRO}
    if kind != "peaked":
        floor = dq_floor(f(q16), f(k16), f(v16), f(do16), scale, causal, ref[0])
        bars["dQ"] = max(GRAD_REL_FRO, 1.5 * floor)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        g = from_dev(g)
        assert np.all(np.isfinite(g)), f"{case}: non-finite {name}"
        e = rel_fro(g, r)
        print(f"{case} {name} relative Frobenius error {e:.3e} (bar {bars[name]:.3e})")
        assert e <= bars[name], f"{case}: {name} relative Frobenius error {e:.3e}"


@pytest.mark.parametrize("kind", ["rise3", "rise12", "peaked"])
@pytest.mark.parametrize("splits", [0, 1, 7])
def test_rescale_decode(gpu, kind, splits):
    import torch
    B, H, n_k, d = 2, 3, 5000, 128
    (q16, k16, v16, _), scale = make_case(kind, 450, B, H, 1, n_k, d)
    o, lse = gpu.decode(to_dev(q16), to_dev(k16), to_dev(v16), scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    f = inputs.bf16_to_f64
    o_ref, l_ref = oracle.decode(f(q16), f(k16), f(v16), scale)
    assert_fwd_close(from_dev(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref,
                     f"decode {kind} C{splits}")


@pytest.mark.parametrize("kind", ["rise3", "rise12", "peaked"])
@pytest.mark.parametrize("heads", [(8, 2), (32, 1)], ids=["group4", "mqa32"])
def test_rescale_decode_paged(gpu, kind, heads):
    import torch
    H, H_kv = heads
    B, d, bs, lens = 2, 128, 16, [3000, 777]
    q16 = inputs.tensor_bf16(460, "q", B, H, 1, d)[:, :, 0, :].copy()
    kc, vc, table, sl = inputs.paged_kv_bf16(460, B, H_kv, lens, d, bs, -(-max(lens) // bs))
    scale = 1.0 if kind == "peaked" else default_scale(d)
    if kind == "peaked":
        vc = quarter(vc)
    else:
        # the paged kernel's tiles hold 32 positions: rise 3 or 12 per 64 positions
        q16, kc = inputs.rising_keys_paged(q16, kc, table, sl,
                                           per_key_for({"rise3": 3.0, "rise12": 12.0}[kind],
                                                       scale))
    o, lse = gpu.decode_paged(to_dev(q16), to_dev(kc), to_dev(vc),
                              torch.from_numpy(table).cuda(), torch.from_numpy(sl).cuda(),
                              scale=scale)
    torch.cuda.synchronize()
    f = inputs.bf16_to_f64
    o_ref, l_ref = oracle.decode_paged(f(q16), f(kc), f(vc), table, sl, scale)
    assert_fwd_close(from_dev(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref,
                     f"paged decode {kind} H{H} H_kv{H_kv}")


@pytest.mark.parametrize("kind", ["rise3", "rise12", "peaked"])
@pytest.mark.parametrize("d", [64, 128])
def test_rescale_fwd_ext(gpu, kind, d):
    """The same moving maxima through fwd_ext with per-sequence lengths, 2 query heads per K/V
    head and dropout p = 0.2 (the lengths-with-dropout form of the forward), causal, against
    the oracle's forward_combined; padding rows and keys hold NaN. On the rising keys O is
    close to the last keys' V rows times 1/(1 - p) = 1.25, up to |O| = 4.6, where one bf16 step
    of O (2^-5) exceeds the O bar, so V is quartered there too (exactly, and V plays no part in
    the row maximum)."""
    import torch
    import oracle.combined as OC
    B, H, H_kv, n = 2, 4, 2, 700
    lens = np.array([700, 450], dtype=np.int32)
    (q16, k16, v16, _), scale = make_case(kind, 470 + d, B, H, n, n, d)
    k16, v16 = k16[:, :H_kv].copy(), v16[:, :H_kv].copy()
    if kind != "peaked":  # (make_case quarters V of the peaked case already)
        v16 = quarter(v16)
    q16 = inputs.fill_padding(q16, lens)
    k16, v16 = inputs.fill_padding(k16, lens), inputs.fill_padding(v16, lens)
    lq = torch.from_numpy(lens).cuda()
    o, lse = gpu.fwd_ext(to_dev(q16), to_dev(k16), to_dev(v16), lq, lq, 0.2, 0xACE, 3,
                         causal=True, scale=scale)
    torch.cuda.synchronize()
    f = inputs.bf16_to_f64
    o_ref, l_ref = OC.forward_combined(f(q16), f(k16), f(v16), lens, lens, scale, True, 0.2,
                                       0xACE, 3)
    o_h, l_h = from_dev(o), lse.cpu().numpy().astype(np.float64)
    live = ~np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l_h), ~live), f"{kind} d{d}: rows with lse = -inf differ"
    assert np.all(o_h[~live] == 0.0), f"{kind} d{d}: empty rows not zero"
    assert_fwd_close(o_h[live], l_h[live], o_ref[live], l_ref[live], f"fwd_ext {kind} d{d}")


@pytest.mark.parametrize("kind", ["rise3", "rise12", "peaked"])
@pytest.mark.parametrize("causal", [False, True])
def test_rescale_bias(gpu, kind, causal):
    """The bias form of the forward (the one that takes the row maximum first and moves the
    reference when a row passes it by more than 8) under moving maxima: on iid inputs a bias that
    rises along the keys by 3 or 12 log2 units per 64-key block, and a peaked softmax (scale 1,
    d = 128, V quartered) under an iid 2 N(0, 1) bias; forward and gradients against the oracle
    (K is not ramped here, so dQ keeps the plain bar)."""
    import torch
    B, H, n_q, n_k, d = 1, 2, 500, 700, 128
    q16, k16, v16, do16 = inputs.qkv_bf16(480, B, H, n_q, n_k, d, with_do=True)
    if kind == "peaked":
        scale = 1.0
        v16 = quarter(v16)
        g = np.random.default_rng(480)
        bias = (2 * g.standard_normal((1, H, n_q, n_k))).astype(np.float32)
    else:
        scale = default_scale(d)
        rise = {"rise3": 3.0, "rise12": 12.0}[kind]
        ramp = np.arange(n_k) * (rise / 64.0) / LOG2E  # natural-log units of the scores
        bias = np.broadcast_to(ramp, (1, H, n_q, n_k)).astype(np.float32)
    b16 = inputs.bf16_round(np.ascontiguousarray(bias))
    q, k, v, do, b = (to_dev(x) for x in (q16, k16, v16, do16, b16))
    o, lse = gpu.fwd_bias(q, k, v, b, causal=causal, scale=scale)
    grads = gpu.bwd_bias(q, k, v, o, lse, do, b, causal=causal, scale=scale)
    torch.cuda.synchronize()
    f = inputs.bf16_to_f64
    o_ref, l_ref = oracle.forward_bias(f(q16), f(k16), f(v16), f(b16), scale, causal)
    what = f"bias {kind} causal {causal}"
    assert_fwd_close(from_dev(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, what)
    ref = oracle.backward_bias(f(q16), f(k16), f(v16), f(do16), f(b16), scale, causal)
    for name, g_, r in zip(("dQ", "dK", "dV"), grads, ref):
        g_ = from_dev(g_)
        assert np.all(np.isfinite(g_)), f"{what}: non-finite {name}"
        e = rel_fro(g_, r)
        assert e <= GRAD_REL_FRO, f"{what}: {name} relative Frobenius error {e:.3e}"

