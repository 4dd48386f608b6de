"""FP8 forward with incoherent processing through the C ABI against the oracle (oracle/fp8.py).

* Codes and scales: the oracle forms the rotation as an fp64 matrix product and the quotient
  x / s in fp64 with one E4M3 rounding; the kernels evaluate the same steps in fp32. Every scale
  must agree to within 4 fp32 units in the last place, and every code must be equal, except that
  a code may be the neighbouring E4M3 value where the oracle's quotient lies within the fp32
  evaluation error of a rounding midpoint (a tie that fp32 arithmetic may resolve the other way).
  Such codes are counted and printed.
* O and LSE: the oracle's attention step runs on the codes and scales the kernels wrote. The
  kernels quantize P relative to their running row maximum, the oracle relative to the
  final one, so O is compared against the per-element bound oracle.fp8.o_tolerance (pinned on the
  CPU) and, tighter, its RMS deviation per head against that of the oracle's own output with P
  quantized on a grid shifted by 2^0.25 or 2^0.5; LSE with the usual relative bar (1e-3).
* The pages' claim: on outlier features the rotation lowers the FP8 error by about 2.6x; the GPU
  output must show at least 2x against exact attention, as the oracle does on the same inputs.
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

U32 = 2.0 ** -24  # unit roundoff of fp32


def run(fa, q16, k16, v16, causal, inc, seed, scale):
    import torch
    B, H, Nq, d = q16.shape
    Nk = k16.shape[2]
    o, lse, ws = fa.fwd_fp8(to_dev(q16), to_dev(k16), to_dev(v16), causal=causal,
                            incoherent=inc, seed=seed, scale=scale)
    torch.cuda.synchronize()
    views = {k: t.cpu().numpy() for k, t in fa.fp8_workspace_views(ws, B, H, Nq, Nk, d).items()}
    return from_dev(o), lse.cpu().numpy().astype(np.float64), views


def check_scales(s_gpu, s_or, tag):
    s_gpu = np.asarray(s_gpu, dtype=np.float32).ravel()
    s_or = np.asarray(s_or, dtype=np.float32).ravel()
    ulp = np.spacing(np.abs(s_or)).astype(np.float64)
    diff = np.abs(s_gpu.astype(np.float64) - s_or.astype(np.float64))
    assert np.all(diff <= 4 * ulp), f"{tag}: scales differ by {np.max(diff / ulp):.0f} ulp"


def check_codes(c_gpu, c_or, quot, rows, s_or, s_gpu, rotated, tag) -> int:
    """Codes equal (either zero code for a zero), or neighbours at a near-tie. rows: the unquantized fp64 rows (rotated or
    not); s_or, s_gpu: per-row scales of the oracle and the kernel. The fp32 evaluation error of
    x / s is bounded by that of a d-term fp32 sum of |x_i| / sqrt(d) (the rotation, any order),
    one fp32 multiply, and the kernel's scale; returns the number of neighbour codes."""
    d = rows.shape[1]
    s_or = np.asarray(s_or, dtype=np.float64)[:, None]
    s_gpu = np.asarray(s_gpu, dtype=np.float64)[:, None]
    gamma = d * U32 / (1 - d * U32)
    l1 = np.sum(np.abs(rows), axis=1, keepdims=True) / math.sqrt(d) if rotated else 0.0
    slack = (gamma * l1 + 2 * U32 * np.abs(rows)) / s_or + 4 * U32 * np.abs(quot) \
        + np.abs(quot) * np.abs(s_gpu - s_or) / s_gpu
    # the two zero codes (0x00, 0x80) are the same value
    diff = (c_gpu != c_or) & ~(((c_gpu & 0x7F) == 0) & ((c_or & 0x7F) == 0))
    if not np.any(diff):
        return 0
    step = np.abs(F8.e4m3_code_index(c_gpu[diff]) - F8.e4m3_code_index(c_or[diff]))
    near = F8.e4m3_tie_distance(quot[diff]) <= slack[diff]
    assert np.all(step == 1) and np.all(near), \
        f"{tag}: {int(np.sum(~near | (step != 1)))} codes differ away from a rounding tie"
    return int(np.sum(diff))


def check(fa, q16, k16, v16, causal, inc, seed, what, heads=None):
    B, H, Nq, d = q16.shape
    Nk = k16.shape[2]
    scale = default_scale(d)
    o, lse, views = run(fa, q16, k16, v16, causal, inc, seed, scale)
    f = inputs.bf16_to_f64
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    ties = 0
    for b, h in heads:
        pr = F8.prepare_head(f(q16[b, h]), f(k16[b, h]), f(v16[b, h]), inc, seed)
        tag = f"{what} head ({b},{h})"
        sq, sk, sv = views["sq"][b, h], views["sk"][b, h], views["sv"][b, h]
        check_scales(sq, pr["sq"], tag + " Q")
        check_scales(sk, pr["sk"], tag + " K")
        check_scales([sv], pr["sv"], tag + " V")
        rq = lambda s: np.repeat(np.asarray(s, dtype=np.float64), 32)[:Nq]  # noqa: E731
        rk = lambda s: np.repeat(np.asarray(s, dtype=np.float64), 64)[:Nk]  # noqa: E731
        ties += check_codes(views["q8"][b, h], pr["q8"], pr["qy"], pr["qr"], rq(pr["sq"]),
                            rq(sq), inc, tag + " Q")
        ties += check_codes(views["k8"][b, h], pr["k8"], pr["ky"], pr["kr"], rk(pr["sk"]),
                            rk(sk), inc, tag + " K")
        ties += check_codes(views["v8t"][b, h][:, :Nk].T, pr["v8"], pr["vy"], pr["vr"],
                            np.full(Nk, float(pr["sv"][0])), np.full(Nk, float(sv)), False,
                            tag + " V")
        assert np.all(views["v8t"][b, h][:, Nk:] == 0), f"{tag}: V padding not zero"
        # the attention step on the codes and scales the kernels wrote (checked above against
        # the oracle's quantization; they differ from it at most at rounding ties)
        used = dict(q8=views["q8"][b, h], sq=sq, k8=views["k8"][b, h], sk=sk,
                    v8=views["v8t"][b, h][:, :Nk].T, sv=np.array([sv], dtype=np.float32))
        o_ref, l_ref = F8.attention_from_codes(used, scale, causal)
        tol = F8.o_tolerance(used, scale, causal)
        err = np.abs(o[b, h] - o_ref)
        assert np.all(np.isfinite(o[b, h])), f"{tag}: non-finite O"
        assert np.all(err <= tol), f"{tag}: O error {err.max():.3e} beyond the E4M3 bound " \
                                   f"(worst ratio {np.max(err / tol):.2f})"
        rms = math.sqrt(np.mean(err ** 2))
        sim = []
        for shift in (0.25, 0.5):
            o_s, _ = F8.attention_from_codes(used, scale, causal, p_shift=shift)
            o_s = inputs.bf16_to_f64(inputs.bf16_round(o_s.astype(np.float32)))
            sim.append(math.sqrt(np.mean((o_s - o_ref) ** 2)))
        assert rms <= max(sim) + 1e-6, f"{tag}: O RMS deviation {rms:.3e} above that of a " \
                                       f"shifted P grid ({max(sim):.3e})"
        el = lse_err(lse[b, h], l_ref)
        assert el <= LSE_REL, f"{tag}: LSE relative error {el:.3e}"
    if ties:
        print(f"{what}: {ties} code(s) resolved to the neighbouring value at a rounding tie")


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
            assert sc < 2.0 ** -128, "the case needs a scale whose fp32 reciprocal overflows"
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
    """The pages report about 2.6x lower FP8 attention error with the rotation, on inputs they do
    not describe. On synthetic outlier features (1 % of entries plus N(0, 10^2)), pooled over 32
    heads, the RMS error of the GPU output against exact fp64 attention must drop by at least 2x,
    and by the same factor as the oracle's FP8 algorithm on the same inputs (within 5 %). The
    factor depends on the outlier mix: about 2.0-2.1 for this one, 1.3-2.8 across the mixes
    tried on the CPU (0.3-3 % of entries, magnitudes 10-30)."""
    B, H, N, d = 1, 32, 512, 128
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
          f"(oracle {ratio_or:.2f}; the pages report about 2.6)")
    assert ratio >= 2.0, ratio
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
