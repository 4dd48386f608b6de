"""FP8 forward with incoherent processing through the C ABI against the oracle (oracle/fp8.py).

* Every FP8 code and scale the kernels write (Q and K after the rotation, V transposed) must
  equal the oracle's bit for bit: both sides take each rounding decision in fp32 the same way.
* O: the kernels quantize P relative to their running row maximum, the oracle relative to the
  final one, so O is compared against a per-element bound derived from the E4M3 step
  (oracle.fp8.o_tolerance); LSE with the usual relative bar (1e-3).
* The pages' claim: on outlier features the rotation lowers the FP8 error by about 2.6x; the GPU
  output must show at least 2x against exact attention.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import oracle.fp8 as F8
from exact_attention_fa_amd import inputs
from tests.helpers import LSE_REL, default_scale, from_dev, lse_err, to_dev

pytestmark = pytest.mark.gpu


def run(fa, q16, k16, v16, causal, inc, seed, scale):
    import torch
    B, H, Nq, d = q16.shape
    Nk = k16.shape[2]
    o, lse, ws = fa.fwd_fp8(to_dev(q16), to_dev(k16), to_dev(v16), causal=causal,
                            incoherent=inc, seed=seed, scale=scale)
    torch.cuda.synchronize()
    views = {k: t.cpu().numpy() for k, t in fa.fp8_workspace_views(ws, B, H, Nq, Nk, d).items()}
    return from_dev(o), lse.cpu().numpy().astype(np.float64), views


def check(fa, q16, k16, v16, causal, inc, seed, what, heads=None):
    B, H, Nq, d = q16.shape
    Nk = k16.shape[2]
    scale = default_scale(d)
    o, lse, views = run(fa, q16, k16, v16, causal, inc, seed, scale)
    f = inputs.bf16_to_f64
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        pr = F8.prepare_head(f(q16[b, h]), f(k16[b, h]), f(v16[b, h]), inc, seed)
        tag = f"{what} head ({b},{h})"
        assert np.array_equal(views["q8"][b, h], pr["q8"]), f"{tag}: Q codes differ"
        assert np.array_equal(views["k8"][b, h], pr["k8"]), f"{tag}: K codes differ"
        assert np.array_equal(views["v8t"][b, h][:, :Nk], pr["v8"].T), f"{tag}: V codes differ"
        assert np.all(views["v8t"][b, h][:, Nk:] == 0), f"{tag}: V padding not zero"
        assert np.array_equal(views["sq"][b, h], pr["sq"]), f"{tag}: Q scales differ"
        assert np.array_equal(views["sk"][b, h], pr["sk"]), f"{tag}: K scales differ"
        assert views["sv"][b, h] == pr["sv"][0], f"{tag}: V scale differs"
        o_ref, l_ref = F8.attention_from_codes(pr, scale, causal)
        tol = F8.o_tolerance(pr, scale, causal)
        err = np.abs(o[b, h] - o_ref)
        assert np.all(np.isfinite(o[b, h])), f"{tag}: non-finite O"
        assert np.all(err <= tol), f"{tag}: O error {err.max():.3e} beyond the E4M3 bound " \
                                   f"(worst ratio {np.max(err / tol):.2f})"
        el = lse_err(lse[b, h], l_ref)
        assert el <= LSE_REL, f"{tag}: LSE relative error {el:.3e}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("inc", [False, True])
@pytest.mark.parametrize("n", [1, 17, 64, 255, 300])
def test_fp8_ragged(gpu, n, inc, causal, d):
    q16, k16, v16 = inputs.qkv_bf16(70 + n, 2, 2, n, n, d)
    check(gpu, q16, k16, v16, causal, inc, 2**33 + n, f"n{n} d{d} causal{causal} inc{inc}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq,nk,causal", [(5, 77, True), (130, 1000, True), (200, 333, False),
                                          (333, 200, False), (64, 4097, True)])
def test_fp8_rectangular(gpu, nq, nk, causal, d):
    q16, k16, v16 = inputs.qkv_bf16(71, 1, 2, nq, nk, d)
    check(gpu, q16, k16, v16, causal, True, 5, f"{nq}x{nk} d{d} causal{causal}")


def test_fp8_outliers_codes_and_bound(gpu):
    """Outlier inputs (large dynamic range per block) through the same bit-exact and bound
    checks."""
    q16, k16, v16 = (inputs.outlier_bf16(72, t, 1, 2, 300, 128) for t in ("q", "k", "v"))
    for inc in (False, True):
        check(gpu, q16, k16, v16, True, inc, 77, f"outliers inc{inc}")


def test_fp8_tiny_blocks_codes(gpu):
    """Blocks whose largest |x| is below 448 * 2^-128 (scale s under 2^-128, so 1 / s overflows
    fp32 and the quantization divides by s): one 32-row Q block, one 64-row K block and the
    whole V of one head scaled by 2^-124; codes, scales and outputs checked as everywhere."""
    q16, k16, v16 = inputs.qkv_bf16(74, 1, 2, 150, 150, 128)
    f = inputs.bf16_to_f64
    tiny = 2.0 ** -124
    q16[0, 0, 32:64] = inputs.bf16_round(f(q16[0, 0, 32:64]) * tiny)
    k16[0, 1, 64:128] = inputs.bf16_round(f(k16[0, 1, 64:128]) * tiny)
    v16[0, 1] = inputs.bf16_round(f(v16[0, 1]) * tiny)
    for inc in (False, True):
        p0 = F8.prepare_head(f(q16[0, 0]), f(k16[0, 0]), f(v16[0, 0]), inc, 78)
        p1 = F8.prepare_head(f(q16[0, 1]), f(k16[0, 1]), f(v16[0, 1]), inc, 78)
        for sc in (p0["sq"][1], p1["sk"][1], p1["sv"][0]):
            assert sc < 2.0 ** -128, "the case must take the division branch"
        check(gpu, q16, k16, v16, False, inc, 78, f"tiny blocks inc{inc}")


def test_fp8_b4_h16_n2048(gpu):
    q16, k16, v16 = inputs.qkv_bf16(2, 4, 16, 2048, 2048, 128)
    check(gpu, q16, k16, v16, True, True, 1, "B4 H16 N2048 causal",
          heads=[(0, 0), (1, 7), (3, 15)])


@pytest.mark.slow
def test_fp8_full_size_heads(gpu):
    """B2 H16 N8192 d128 causal launched whole; two heads' codes and outputs checked."""
    q16, k16, v16 = inputs.qkv_bf16(3, 2, 16, 8192, 8192, 128)
    check(gpu, q16, k16, v16, True, True, 3, "B2 H16 N8192 causal", heads=[(0, 3), (1, 12)])


def test_fp8_incoherent_lowers_error_on_outliers(gpu):
    """The pages report about 2.6x lower FP8 attention error with the rotation. On synthetic
    outlier features (1 % of entries plus N(0, 10^2)) the RMS error of the GPU output against
    exact fp64 attention must drop by at least 1.8x, and by the same factor as the oracle's
    FP8 algorithm on the same inputs (within 5 %); the factor varies with the draw (about 2.0 to
    2.7 on these shapes)."""
    B, H, N, d = 1, 8, 512, 128
    q16, k16, v16 = (inputs.outlier_bf16(73, t, B, H, N, d) for t in ("q", "k", "v"))
    f = inputs.bf16_to_f64
    scale = default_scale(d)
    ref, _ = oracle.forward(f(q16), f(k16), f(v16), scale, False)
    err, err_or = {}, {}
    for inc in (False, True):
        o, _, _ = run(gpu, q16, k16, v16, False, inc, 11, scale)
        err[inc] = math.sqrt(np.mean((o - ref) ** 2))
        o_or, _, _ = F8.forward_fp8(f(q16), f(k16), f(v16), scale, False, inc, 11)
        err_or[inc] = math.sqrt(np.mean((o_or - ref) ** 2))
    ratio, ratio_or = err[False] / err[True], err_or[False] / err_or[True]
    print(f"FP8 RMS error: plain {err[False]:.3e}, incoherent {err[True]:.3e}, ratio {ratio:.2f} "
          f"(oracle {ratio_or:.2f})")
    assert ratio > 1.8, ratio
    assert abs(ratio / ratio_or - 1) < 0.05, (ratio, ratio_or)


def test_fp8_determinism_and_seed(gpu):
    import torch
    q16, k16, v16 = inputs.qkv_bf16(74, 1, 2, 300, 300, 128)
    q, k, v = to_dev(q16), to_dev(k16), to_dev(v16)
    o1, l1, _ = gpu.fwd_fp8(q, k, v, causal=True, seed=5)
    o2, l2, _ = gpu.fwd_fp8(q, k, v, causal=True, seed=5)
    o3, _, _ = gpu.fwd_fp8(q, k, v, causal=True, seed=6)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and not torch.equal(o1, o3)
