"""Host-side pieces: the seeded bf16 generator and the work/traffic counts behind the rates."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

from exact_attention_fa_amd import inputs, metrics

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_round_hand_patterns():
    # (fp32 bits, expected bf16 bits), worked by hand for round-to-nearest-even
    cases = [
        (0x3F800000, 0x3F80),  # 1.0 exact
        (0x3F808000, 0x3F80),  # halfway, even low bit 0 -> stays
        (0x3F818000, 0x3F82),  # halfway, odd low bit 1 -> rounds up to even
        (0x3F808001, 0x3F81),  # just above halfway -> up
        (0x3F807FFF, 0x3F80),  # just below halfway -> down
        (0xBF80C000, 0xBF81),  # negative, above halfway -> magnitude up
        (0x00000000, 0x0000),
        (0x80000000, 0x8000),
        (0x7F7FFFFF, 0x7F80),  # largest finite fp32 rounds to +inf in bf16 (RNE overflow)
    ]
    x = np.array([c[0] for c in cases], dtype=np.uint32).view(np.float32)
    got = inputs.bf16_round(x)
    assert [int(g) for g in got] == [c[1] for c in cases]
    back = inputs.bf16_to_f32(np.array([0x3F80, 0xC040, 0x4049], dtype=np.uint16))
    assert back.tolist() == [1.0, -3.0, 3.140625]


def test_bf16_round_is_nearest():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32)
    r = inputs.bf16_to_f64(inputs.bf16_round(x))
    err = np.abs(r - x.astype(np.float64))
    ulp = np.exp2(np.floor(np.log2(np.abs(x.astype(np.float64)))) - 7)
    assert np.all(err <= ulp / 2 + 1e-30)


def test_generator_seeded_per_slice():
    a = inputs.tensor_bf16(3, "k", 2, 3, 17, 8)
    b = inputs.tensor_bf16(3, "k", 2, 3, 17, 8, threads=1)
    assert np.array_equal(a, b)
    assert np.array_equal(a[1, 2], inputs.slice_bf16(3, "k", 1, 2, 17, 8))
    c = inputs.tensor_bf16(3, "v", 2, 3, 17, 8)
    assert not np.array_equal(a, c)
    x = inputs.bf16_to_f64(inputs.tensor_bf16(1, "q", 1, 4, 4096, 16))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01


def _golden():
    with open(os.path.join(GOLDEN, "pages_numbers.json")) as f:
        return json.load(f)


def test_metrics_against_pages_numbers():
    g = _golden()
    pm = g["p_matrix_fp16_bytes"]
    for n, printed in pm["rows"]:
        assert metrics.score_matrix_bytes(n, pm["elem_bytes"]) == pytest.approx(printed, rel=pm["rel_tol"])
    sh = g["a100_share_of_80gb"]
    assert metrics.score_matrix_bytes(sh["n"], 2) / (sh["gb"] * 1e9) == pytest.approx(sh["share"], abs=sh["abs_tol"])
    r = g["a100_ridge"]
    assert r["peak_tflops"] / r["bw_tbps"] == pytest.approx(r["flop_per_byte"], rel=r["rel_tol"])
    si = g["standard_intensity"]
    n = 4096
    assert metrics.attention_flops(1, 1, n, n, si["d"]) / metrics.standard_attention_hbm_bytes(n) == si["flop_per_byte"]
    t = g["a100_times"]
    compute_ms = metrics.attention_flops(1, 1, t["n"], t["n"], t["d"]) / (t["peak_tflops"] * 1e12) * 1e3
    io_ms = metrics.standard_attention_hbm_bytes(t["n"]) / (t["bw_tbps"] * 1e12) * 1e3
    assert compute_ms == pytest.approx(t["compute_ms"], abs=t["abs_tol_ms"])
    assert io_ms == pytest.approx(t["io_ms"], abs=t["abs_tol_ms"])
    kv = g["kv_cache"]
    per_tok = metrics.kv_cache_bytes_per_token(kv["d_model"], kv["n_layers"], kv["elem_bytes"])
    assert per_tok / 1e6 == pytest.approx(kv["mb_per_token"], rel=kv["rel_tol"])
    assert per_tok * kv["tokens"] / 1e9 == pytest.approx(kv["session_gb"], rel=kv["rel_tol"])
    io = g["io_reduction"]
    assert io["m"] / io["d"] ** 2 == pytest.approx(io["factor"], rel=io["rel_tol"])


def test_metric_conventions():
    # causal halves, backward is 2.5x; the decode bytes are dominated by reading K and V once
    f = metrics.attention_flops(2, 16, 8192, 8192, 128)
    assert metrics.attention_flops(2, 16, 8192, 8192, 128, causal=True) == f / 2
    assert metrics.attention_flops(2, 16, 8192, 8192, 128, causal=True, backward=True) == f / 2 * 2.5
    assert metrics.executed_bwd_flops(2, 16, 8192, 8192, 128, True) == pytest.approx(f / 2 * 3.5)
    assert metrics.decode_bytes(8, 32, 65536, 128) == 2 * 8 * 32 * 65536 * 128 * 2 + 2 * 8 * 32 * 128 * 2 + 8 * 32 * 4
    assert metrics.MI355X_BF16_DENSE_TFLOPS == pytest.approx(256 * 2.4e9 * 4096 / 1e12, rel=1e-4)
